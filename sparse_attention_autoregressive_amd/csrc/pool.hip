// Token compression by mean pooling (Light Forcing summary, execution flow, stage 2):
// block-level means of queries and keys, frame-level means of keys.
//
// One wave pools one block at a time: lane l reads 16-byte chunk l % C of every TL-th
// token of the block (C = 16-byte chunks per token, TL = 64 / C token lanes),
// accumulating in fp32; the TL partial sums of each chunk are
// added across lanes in a fixed order, and the first C lanes write the block mean (the
// sum divided by the block's true token count). Every input byte is read once, with
// fully coalesced loads.
//
// With frame means requested, a 1024-thread workgroup owns one whole frame: its 16
// waves take the frame's blocks in turn, keep the running sum of their block sums, and
// the frame mean is the sum of the waves' sums (added in a fixed order) divided by the
// frame's token count. Without, a 256-thread workgroup owns four blocks (one per wave),
// which keeps short tensors (the chunk's queries) spread over every CU. Each lane keeps
// up to 16 tokens' loads in flight. A combined launch pools a chunk's queries and all
// keys together (16 query blocks per workgroup); every block is summed by one wave with
// the same code either way, so results match the separate launches bitwise. Results
// are deterministic.
#include "lf_device.h"
#include "lf_kernels.h"

namespace lf {

constexpr int kPoolWaves = 4;        // waves per workgroup without frame means
constexpr int kFrameWaves = 16;      // waves per workgroup owning a whole frame

template <typename T>
struct Chunk16;

template <>
struct Chunk16<float> {
  static constexpr int E = 4;  // elements per 16-byte chunk
  __device__ static __forceinline__ void add(const float* p, float* acc) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    acc[0] += v.x; acc[1] += v.y; acc[2] += v.z; acc[3] += v.w;
  }
};

template <>
struct Chunk16<__bf16> {
  static constexpr int E = 8;
  __device__ static __forceinline__ void add(const __bf16* p, float* acc) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(w[i] << 16);
      acc[2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

// Sum over the TL token lanes holding the same chunk (lanes c, c + C, c + 2C, ...):
// a butterfly over the lane bits above C, in a fixed order.
template <int C>
__device__ __forceinline__ float token_lane_sum(float x) {
#pragma unroll
  for (int m = C; m < kWave; m <<= 1) x += __shfl_xor(x, m, kWave);
  return x;
}

// Sums of block j of a frame (the frame's tokens [j*bs, j*bs + len)) into `sum`,
// valid in lanes < C (lane c holds chunk c). Up to kBatch tokens per lane are loaded
// before any is added, so a wave keeps kBatch * 1 KB in flight.
constexpr int kBatch = 16;

template <typename T, int D>
__device__ __forceinline__ void block_sum(const T* __restrict__ frame, int j, int bs, int len, int lane,
                                          float* sum) {
  constexpr int E = Chunk16<T>::E;
  constexpr int C = D / E;
  constexpr int TL = kWave / C;
  const int c = lane % C, s = lane / C;
  const T* base = frame + static_cast<size_t>(j) * bs * D + c * E;
  float a[E], b[E];
#pragma unroll
  for (int e = 0; e < E; ++e) a[e] = b[e] = 0.f;
  for (int t0 = 0; t0 < len; t0 += kBatch * TL) {
    uint4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int t = t0 + s + u * TL;
      v[u] = t < len ? *reinterpret_cast<const uint4*>(base + static_cast<size_t>(t) * D) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) Chunk16<T>::add(reinterpret_cast<const T*>(&v[u]), (u & 1) ? b : a);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) sum[e] = token_lane_sum<C>(a[e] + b[e]);
}

// The work of workgroup `wg` (W waves). FRAMES: one workgroup per (b, h, frame), writing
// block and frame means. Otherwise one workgroup per (b, h, frame, group of W blocks),
// block means only.
template <typename T, int D, bool FRAMES, int W>
__device__ __forceinline__ void pool_part(const T* __restrict__ x, float* __restrict__ blk, float* __restrict__ frm,
                                          int n_frames, int tpf, int bs, int n_bpf, long long x_stride,
                                          int out_stride, int wg, float (*fs)[D]) {
  constexpr int E = Chunk16<T>::E;
  constexpr int C = D / E;
  const int groups = FRAMES ? 1 : (n_bpf + W - 1) / W;
  const int grp = wg % groups;
  const int bf = wg / groups;                         // bh * n_frames + f
  const int bh = bf / n_frames, f = bf - bh * n_frames;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const T* frame = x + (static_cast<size_t>(bh) * x_stride + static_cast<size_t>(f) * tpf) * D;
  const size_t of = static_cast<size_t>(bh) * out_stride + f;   // output frame slot
  float* blk_row = blk + of * n_bpf * D;

  float fsum[E];
#pragma unroll
  for (int e = 0; e < E; ++e) fsum[e] = 0.f;
  const int j0 = FRAMES ? wave : grp * W + wave;
  const int dj = FRAMES ? W : n_bpf;               // without frames: one block per wave
  for (int j = j0; j < n_bpf; j += dj) {
    const int len = min(bs, tpf - j * bs);
    float sum[E];
    block_sum<T, D>(frame, j, bs, len, lane, sum);
    if (lane < C) {
      const float inv = 1.0f / static_cast<float>(len);
      float* out = blk_row + static_cast<size_t>(j) * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; e += 4)
        *reinterpret_cast<float4*>(out + e) =
            make_float4(sum[e] * inv, sum[e + 1] * inv, sum[e + 2] * inv, sum[e + 3] * inv);
#pragma unroll
      for (int e = 0; e < E; ++e) fsum[e] += sum[e];
    }
  }
  if (!FRAMES) return;
  if (lane < C) {
#pragma unroll
    for (int e = 0; e < E; ++e) fs[wave][lane * E + e] = fsum[e];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) t += fs[w][threadIdx.x];
    frm[of * D + threadIdx.x] = t / static_cast<float>(tpf);
  }
}

template <typename T, int D, bool FRAMES>
__global__ void __launch_bounds__((FRAMES ? kFrameWaves : kPoolWaves) * kWave) pool_kernel(
    const T* __restrict__ x, float* __restrict__ blk, float* __restrict__ frm, int n_frames, int tpf, int bs,
    int n_bpf, long long x_stride, int out_stride) {
  constexpr int W = FRAMES ? kFrameWaves : kPoolWaves;
  __shared__ __attribute__((aligned(16))) float fs[W][D];
  pool_part<T, D, FRAMES, W>(x, blk, frm, n_frames, tpf, bs, n_bpf, x_stride, out_stride, blockIdx.x, fs);
}

// Queries (block means) and keys (block and frame means) in one launch: the first n_qwg
// workgroups pool query blocks, 16 per workgroup, the rest one key frame each.
template <typename T, int D>
__global__ void __launch_bounds__(kFrameWaves * kWave) pool_qk_kernel(
    const T* __restrict__ q, const T* __restrict__ k, float* __restrict__ q_blk, float* __restrict__ k_blk,
    float* __restrict__ k_frm, int n_qframes, int n_kframes, int tpf, int bs, int n_bpf, long long q_stride,
    long long k_stride, int k_out_stride, int n_qwg) {
  __shared__ __attribute__((aligned(16))) float fs[kFrameWaves][D];
  const int wg = blockIdx.x;
  if (wg < n_qwg)
    pool_part<T, D, false, kFrameWaves>(q, q_blk, nullptr, n_qframes, tpf, bs, n_bpf, q_stride, n_qframes, wg, fs);
  else
    pool_part<T, D, true, kFrameWaves>(k, k_blk, k_frm, n_kframes, tpf, bs, n_bpf, k_stride, k_out_stride,
                                       wg - n_qwg, fs);
}

template <typename T, int D>
static hipError_t launch_pool_t(const void* x, int BH, int n_frames, int tpf, int bs, int n_bpf,
                                long long x_stride, int out_stride, float* blk, float* frm, hipStream_t st) {
  const unsigned frames = static_cast<unsigned>(BH) * n_frames;
  if (frm != nullptr) {
    hipLaunchKernelGGL((pool_kernel<T, D, true>), dim3(frames), dim3(kFrameWaves * kWave), 0, st,
                       static_cast<const T*>(x), blk, frm, n_frames, tpf, bs, n_bpf, x_stride, out_stride);
  } else {
    const unsigned groups = (n_bpf + kPoolWaves - 1) / kPoolWaves;
    hipLaunchKernelGGL((pool_kernel<T, D, false>), dim3(frames * groups), dim3(kPoolWaves * kWave), 0, st,
                       static_cast<const T*>(x), blk, frm, n_frames, tpf, bs, n_bpf, x_stride, out_stride);
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_pool_qk_t(const void* q, const void* k, int BH, int n_qframes, int n_kframes, int tpf,
                                   int bs, int n_bpf, long long q_stride, long long k_stride, int k_out_stride,
                                   float* q_blk, float* k_blk, float* k_frm, hipStream_t st) {
  const int n_qwg = BH * n_qframes * ((n_bpf + kFrameWaves - 1) / kFrameWaves);
  const unsigned grid = static_cast<unsigned>(n_qwg) + static_cast<unsigned>(BH) * n_kframes;
  hipLaunchKernelGGL((pool_qk_kernel<T, D>), dim3(grid), dim3(kFrameWaves * kWave), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(k), q_blk, k_blk, k_frm, n_qframes, n_kframes,
                     tpf, bs, n_bpf, q_stride, k_stride, k_out_stride, n_qwg);
  return hipGetLastError();
}

hipError_t launch_pool_qk(const void* q, const void* k, bool bf16, int d, int BH, int n_qframes, int n_kframes,
                          int tpf, int bs, int n_bpf, long long q_stride, long long k_stride, int k_out_stride,
                          float* q_blk, float* k_blk, float* k_frm, hipStream_t st) {
  if (bf16) {
    return d == 128 ? launch_pool_qk_t<__bf16, 128>(q, k, BH, n_qframes, n_kframes, tpf, bs, n_bpf, q_stride,
                                                    k_stride, k_out_stride, q_blk, k_blk, k_frm, st)
                    : launch_pool_qk_t<__bf16, 64>(q, k, BH, n_qframes, n_kframes, tpf, bs, n_bpf, q_stride,
                                                   k_stride, k_out_stride, q_blk, k_blk, k_frm, st);
  }
  return d == 128 ? launch_pool_qk_t<float, 128>(q, k, BH, n_qframes, n_kframes, tpf, bs, n_bpf, q_stride,
                                                 k_stride, k_out_stride, q_blk, k_blk, k_frm, st)
                  : launch_pool_qk_t<float, 64>(q, k, BH, n_qframes, n_kframes, tpf, bs, n_bpf, q_stride, k_stride,
                                                k_out_stride, q_blk, k_blk, k_frm, st);
}

hipError_t launch_pool(const void* x, bool bf16, int d, int BH, int n_frames, int tpf, int bs,
                       int n_bpf, long long x_stride, int out_stride, float* blk, float* frm, hipStream_t st) {
  if (bf16) {
    return d == 128 ? launch_pool_t<__bf16, 128>(x, BH, n_frames, tpf, bs, n_bpf, x_stride, out_stride, blk, frm, st)
                    : launch_pool_t<__bf16, 64>(x, BH, n_frames, tpf, bs, n_bpf, x_stride, out_stride, blk, frm, st);
  }
  return d == 128 ? launch_pool_t<float, 128>(x, BH, n_frames, tpf, bs, n_bpf, x_stride, out_stride, blk, frm, st)
                  : launch_pool_t<float, 64>(x, BH, n_frames, tpf, bs, n_bpf, x_stride, out_stride, blk, frm, st);
}

}  // namespace lf
