// Token compression by mean pooling (Light Forcing summary, execution flow, stage 2):
// block-level means of queries and keys, frame-level means of keys.
//
// Block means: one wave pools one block: lane l reads 16-byte chunk l % C of every
// TL-th token of the block (C = 16-byte chunks per token, TL = 64 / C token lanes),
// accumulating in fp32, with up to 16 tokens' loads in flight per lane; the TL partial
// sums of each chunk are added across lanes in a fixed order, and the first C lanes
// write the block mean (the sum divided by the block's true token count). Every input
// byte is read once, with fully coalesced loads. The waves of a launch walk one flat
// list of blocks (all query blocks, then all key blocks), four waves per workgroup, so
// even a chunk's few frames spread over every CU: a frame's 400 KB is read by about
// seven CUs instead of one.
//
// Frame means: a second, small launch forms each frame's mean from its block means,
// weighted by the blocks' token counts and added in block order, divided by the frame's
// token count (a full 64-token block contributes its exact sum). Both launches are the
// same whether queries and keys are pooled together or apart, so the results match
// bitwise. Results are deterministic.
#include "lf_device.h"
#include "lf_kernels.h"

namespace lf {

constexpr int kPoolWaves = 4;        // waves (blocks) per workgroup of the block-mean launch
constexpr int kFrameThreads = 256;   // threads per workgroup of the frame-mean launch

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
//
// Summation order (shared with the prologue, whose four waves each take one quarter):
// load u of every batch goes to the lane's accumulator set q = u / kQuarter, added in
// batch and u order; the four sets are combined as ((A0 + A1) + (A2 + A3)); then the
// token lanes' sums are added by the fixed butterfly.
constexpr int kBatch = 16;
constexpr int kQuarters = 4;
constexpr int kQuarter = kBatch / kQuarters;
constexpr int kProLoads = 2;         // prologue loads in flight per lane (kQuarter a multiple)
static_assert(kQuarter % kProLoads == 0, "whole steps per quarter");

template <int E, int C>
__device__ __forceinline__ void combine_quarters(const float (&A)[kQuarters][E], float* sum) {
#pragma unroll
  for (int e = 0; e < E; ++e) sum[e] = token_lane_sum<C>((A[0][e] + A[1][e]) + (A[2][e] + A[3][e]));
}

template <typename T, int D>
__device__ __forceinline__ void block_sum(const T* __restrict__ frame, int j, int bs, int len, int lane,
                                          float* sum) {
  constexpr int E = Chunk16<T>::E;
  constexpr int C = D / E;
  constexpr int TL = kWave / C;
  const int c = lane % C, s = lane / C;
  const T* base = frame + static_cast<size_t>(j) * bs * D + c * E;
  float A[kQuarters][E];
#pragma unroll
  for (int q = 0; q < kQuarters; ++q)
#pragma unroll
    for (int e = 0; e < E; ++e) A[q][e] = 0.f;
  for (int t0 = 0; t0 < len; t0 += kBatch * TL) {
    uint4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int t = t0 + s + u * TL;
      v[u] = t < len ? *reinterpret_cast<const uint4*>(base + static_cast<size_t>(t) * D) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) Chunk16<T>::add(reinterpret_cast<const T*>(&v[u]), A[u / kQuarter]);
  }
  combine_quarters<E, C>(A, sum);
}

// One tensor's share of a block-mean launch: n_blocks = BH * n_frames * n_bpf blocks,
// the (b, h) slices x_stride tokens apart in x and out_stride frames apart in blk.
template <typename T>
struct PoolJob {
  const T* x;
  float* blk;
  long long x_stride;
  int n_frames, out_stride, n_blocks;
};

template <typename T, int D>
__device__ __forceinline__ void pool_block(const PoolJob<T>& p, int b, int tpf, int bs, int n_bpf, int lane) {
  constexpr int E = Chunk16<T>::E;
  constexpr int C = D / E;
  const int bf = b / n_bpf, j = b - bf * n_bpf;     // bf = bh * n_frames + f
  const int bh = bf / p.n_frames, f = bf - bh * p.n_frames;
  const T* frame = p.x + (static_cast<size_t>(bh) * p.x_stride + static_cast<size_t>(f) * tpf) * D;
  const int len = min(bs, tpf - j * bs);
  float sum[E];
  block_sum<T, D>(frame, j, bs, len, lane, sum);
  if (lane < C) {
    const float inv = 1.0f / static_cast<float>(len);
    float* out = p.blk + ((static_cast<size_t>(bh) * p.out_stride + f) * n_bpf + j) * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; e += 4)
      *reinterpret_cast<float4*>(out + e) =
          make_float4(sum[e] * inv, sum[e + 1] * inv, sum[e + 2] * inv, sum[e + 3] * inv);
  }
}

// The frame mean of one channel of one frame: the frame's block means, each weighted by
// its token count, added in block order, divided by the frame's token count. `slot` is
// the frame's index in the pooled tensors (b, h slice offset included).
template <int D>
__device__ __forceinline__ void frame_mean_channel(const float* __restrict__ blk, float* __restrict__ frm,
                                                   size_t slot, int c, int tpf, int bs, int n_bpf) {
  const float* row = blk + slot * n_bpf * D + c;
  float s = 0.f;
#pragma unroll 8
  for (int j = 0; j < n_bpf; ++j) s += row[static_cast<size_t>(j) * D] * static_cast<float>(min(bs, tpf - j * bs));
  frm[slot * D + c] = s / static_cast<float>(tpf);
}

// Frame means of frames [f0, f0 + n_frames) of every (b, h) slice of a pooled-key cache
// (slices out_stride frames apart) whose block means an earlier launch wrote: one thread
// per (slice frame, channel), n_items = BH * n_frames * D.
struct LagJob {
  const float* blk;
  float* frm;
  int f0, n_frames, out_stride, n_items;
};

template <int D>
__device__ __forceinline__ void lag_item(const LagJob& L, int t, int tpf, int bs, int n_bpf) {
  if (t >= L.n_items) return;
  const int bf = t / D, c = t % D;
  const int bh = bf / L.n_frames, f = L.f0 + (bf - bh * L.n_frames);
  frame_mean_channel<D>(L.blk, L.frm, static_cast<size_t>(bh) * L.out_stride + f, c, tpf, bs, n_bpf);
}

// Wave w of the first block_wgs workgroups pools block w of the list "a's blocks, then
// b's blocks"; the workgroups after them form the frame means of the lag job.
template <typename T, int D>
__global__ void __launch_bounds__(kPoolWaves * kWave) block_mean_kernel(PoolJob<T> a, PoolJob<T> b, LagJob lag,
                                                                        int block_wgs, int tpf, int bs, int n_bpf) {
  if (static_cast<int>(blockIdx.x) >= block_wgs) {
    lag_item<D>(lag, (blockIdx.x - block_wgs) * (kPoolWaves * kWave) + threadIdx.x, tpf, bs, n_bpf);
    return;
  }
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kPoolWaves + threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  if (w < a.n_blocks)
    pool_block<T, D>(a, w, tpf, bs, n_bpf, lane);
  else if (w - a.n_blocks < b.n_blocks)
    pool_block<T, D>(b, w - a.n_blocks, tpf, bs, n_bpf, lane);
}

// Thread (frame, channel): frame_mean_channel for every frame of a launch.
// n_slices_frames = BH * n_frames.
template <int D>
__global__ void __launch_bounds__(kFrameThreads) frame_mean_kernel(const float* __restrict__ blk,
                                                                   float* __restrict__ frm, int n_slice_frames,
                                                                   int n_frames, int out_stride, int tpf, int bs,
                                                                   int n_bpf) {
  const int t = blockIdx.x * kFrameThreads + threadIdx.x;
  const int bf = t / D, c = t % D;
  if (bf >= n_slice_frames) return;
  const int bh = bf / n_frames, f = bf - bh * n_frames;
  frame_mean_channel<D>(blk, frm, static_cast<size_t>(bh) * out_stride + f, c, tpf, bs, n_bpf);
}

template <int D>
static unsigned lag_wgs(const LagJob& lag) {
  return static_cast<unsigned>((lag.n_items + kPoolWaves * kWave - 1) / (kPoolWaves * kWave));
}

template <typename T, int D>
static hipError_t launch_t(PoolJob<T> a, PoolJob<T> b, float* frm, LagJob lag, int BH, int tpf, int bs, int n_bpf,
                           hipStream_t st) {
  const unsigned waves = static_cast<unsigned>(a.n_blocks) + static_cast<unsigned>(b.n_blocks);
  const unsigned bwgs = (waves + kPoolWaves - 1) / kPoolWaves;
  hipLaunchKernelGGL((block_mean_kernel<T, D>), dim3(bwgs + lag_wgs<D>(lag)), dim3(kPoolWaves * kWave), 0, st, a, b, lag,
                     static_cast<int>(bwgs), tpf, bs, n_bpf);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (frm == nullptr) return hipSuccess;
  // frame means of b (the keys)
  const int n_sf = BH * b.n_frames;
  const unsigned grid = static_cast<unsigned>((static_cast<long long>(n_sf) * D + kFrameThreads - 1) / kFrameThreads);
  hipLaunchKernelGGL((frame_mean_kernel<D>), dim3(grid), dim3(kFrameThreads), 0, st, b.blk, frm, n_sf, b.n_frames,
                     b.out_stride, tpf, bs, n_bpf);
  return hipGetLastError();
}

template <typename T>
static PoolJob<T> job(const void* x, float* blk, int BH, int n_frames, int n_bpf, long long x_stride,
                      int out_stride) {
  return PoolJob<T>{static_cast<const T*>(x), blk, x_stride, n_frames, out_stride, BH * n_frames * n_bpf};
}

static LagJob no_lag() { return LagJob{nullptr, nullptr, 0, 1, 1, 0}; }

template <typename T>
static hipError_t launch_d(int d, PoolJob<T> a, PoolJob<T> b, float* frm, LagJob lag, int BH, int tpf, int bs,
                           int n_bpf, hipStream_t st) {
  return d == 128 ? launch_t<T, 128>(a, b, frm, lag, BH, tpf, bs, n_bpf, st)
                  : launch_t<T, 64>(a, b, frm, lag, BH, tpf, bs, n_bpf, st);
}

hipError_t launch_pool_qk(const void* q, const void* k, bool bf16, int d, int BH, int n_qframes, int n_kframes,
                          int tpf, int bs, int n_bpf, long long q_stride, long long k_stride, int k_out_stride,
                          float* q_blk, float* k_blk, float* k_frm, hipStream_t st) {
  if (bf16)
    return launch_d<__bf16>(d, job<__bf16>(q, q_blk, BH, n_qframes, n_bpf, q_stride, n_qframes),
                            job<__bf16>(k, k_blk, BH, n_kframes, n_bpf, k_stride, k_out_stride), k_frm, no_lag(), BH,
                            tpf, bs, n_bpf, st);
  return launch_d<float>(d, job<float>(q, q_blk, BH, n_qframes, n_bpf, q_stride, n_qframes),
                         job<float>(k, k_blk, BH, n_kframes, n_bpf, k_stride, k_out_stride), k_frm, no_lag(), BH, tpf,
                         bs, n_bpf, st);
}

hipError_t launch_pool(const void* x, bool bf16, int d, int BH, int n_frames, int tpf, int bs,
                       int n_bpf, long long x_stride, int out_stride, float* blk, float* frm, hipStream_t st) {
  // a single tensor rides in the second slot (the one whose frame means are formed)
  if (bf16)
    return launch_d<__bf16>(d, PoolJob<__bf16>{nullptr, nullptr, 0, 1, 1, 0},
                            job<__bf16>(x, blk, BH, n_frames, n_bpf, x_stride, out_stride), frm, no_lag(), BH, tpf, bs,
                            n_bpf, st);
  return launch_d<float>(d, PoolJob<float>{nullptr, nullptr, 0, 1, 1, 0},
                         job<float>(x, blk, BH, n_frames, n_bpf, x_stride, out_stride), frm, no_lag(), BH, tpf, bs,
                         n_bpf, st);
}

hipError_t launch_pool_step(const PoolStepArgs& a, bool bf16, int d, hipStream_t st) {
  const LagJob lag{a.k_blk, a.k_frm, a.f_lag, a.n_lag > 0 ? a.n_lag : 1, a.cache_stride, a.BH * a.n_lag * d};
  float* kb_new = a.k_blk + static_cast<size_t>(a.f_new) * a.n_bpf * d;
  if (bf16)
    return launch_d<__bf16>(d, job<__bf16>(a.q, a.q_blk, a.BH, a.n_qframes, a.n_bpf, a.q_stride, a.n_qframes),
                            job<__bf16>(a.k, kb_new, a.BH, a.n_new, a.n_bpf, a.k_stride, a.cache_stride), nullptr, lag,
                            a.BH, a.tpf, a.bs, a.n_bpf, st);
  return launch_d<float>(d, job<float>(a.q, a.q_blk, a.BH, a.n_qframes, a.n_bpf, a.q_stride, a.n_qframes),
                         job<float>(a.k, kb_new, a.BH, a.n_new, a.n_bpf, a.k_stride, a.cache_stride), nullptr, lag, a.BH,
                         a.tpf, a.bs, a.n_bpf, st);
}

// ---------------------------------------------------------------------------------
// Query/key prologue fused with pooling: RMSNorm over each token's d channels (gamma
// shared by all heads), then a rotary embedding whose adjacent channel pairs turn with
// the token's frame, row or column (first d/2 - 2*floor(d/6) pairs, next floor(d/6),
// last floor(d/6); pair i of an axis with n pairs at position*theta^(-i/n)). The
// rounded result is stored and, in the same pass, summed into block means exactly as
// the block-mean kernel would sum the stored tensor (same lanes, batches and order), so
// a following lf_pool of the output would give bitwise the same means. One wave per
// block; the 16 lanes of a token (bf16, d = 128) reduce its sum of squares with DPP
// lane moves. Angles are reduced in revolutions and evaluated with the hardware sine and
// cosine.

template <typename T>
struct Out16;

template <>
struct Out16<float> {
  __device__ static __forceinline__ float round(float x) { return x; }
  __device__ static __forceinline__ void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

template <>
struct Out16<__bf16> {
  __device__ static __forceinline__ float round(float x) { return static_cast<float>(static_cast<__bf16>(x)); }
  __device__ static __forceinline__ void store(__bf16* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (__float_as_uint(v[2 * i]) >> 16) | (__float_as_uint(v[2 * i + 1]) & 0xFFFF0000u);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// Sum over the C consecutive lanes holding one token's chunks, the same value in each:
// pairs within quads and half-rows and rows with DPP moves (no LDS round trip), wider
// groups with xor shuffles. Every step adds partners in the same order in both lanes of
// a pair, so all lanes of the token end with bitwise the same sum.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int C>
__device__ __forceinline__ float token_sum(float x) {
  if (C > 1) x = dpp_add<0xB1>(x);     // quad_perm [1, 0, 3, 2]
  if (C > 2) x = dpp_add<0x4E>(x);     // quad_perm [2, 3, 0, 1]
  if (C > 4) x = dpp_add<0x141>(x);    // row_half_mirror
  if (C > 8) x = dpp_add<0x140>(x);    // row_mirror
#pragma unroll
  for (int m = 16; m < C; m <<= 1) x += __shfl_xor(x, m, kWave);
  return x;
}

template <typename T>
struct ProJob {
  const T* x;
  T* y;
  const float* gamma;
  float* blk;
  long long x_stride, y_stride;   // tokens between (b, h) slices of x and of y
  int n_frames, frame0, out_stride, n_blocks, lat_w;
  float eps;
  float rev[kMaxPairs];           // turn per unit of position of each rotary pair (revolutions)
};

// One block of one job per workgroup: wave q takes loads u in [q kQuarter, (q + 1) kQuarter)
// of every batch; part_s holds the quarter sums of waves 1..3.
template <typename T, int D>
__device__ __forceinline__ void prologue_block(const ProJob<T>& p, int w, int tpf, int bs, int n_bpf,
                                               float (*part_s)[kWave][Chunk16<T>::E]) {
  constexpr int E = Chunk16<T>::E;
  constexpr int C = D / E;
  constexpr int TL = kWave / C;
  const int q = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave, c = lane % C, s = lane / C;
  const int bf = w / n_bpf, j = w - bf * n_bpf;
  const int bh = bf / p.n_frames, f = bf - bh * p.n_frames;
  const size_t in_frame = (static_cast<size_t>(f) * tpf + static_cast<size_t>(j) * bs) * D + c * E;
  const T* xin = p.x + static_cast<size_t>(bh) * p.x_stride * D + in_frame;
  T* yout = p.y + static_cast<size_t>(bh) * p.y_stride * D + in_frame;
  const int len = min(bs, tpf - j * bs);

  float gm[E];
#pragma unroll
  for (int e = 0; e < E; ++e) gm[e] = p.gamma[c * E + e];
  // the lane's E/2 rotary pairs: axis and turn (revolutions) per unit of position
  constexpr int NHW = D / 6, NT = D / 2 - 2 * NHW;
  int axis[E / 2];
  float rev[E / 2];
#pragma unroll
  for (int m = 0; m < E / 2; ++m) {
    const int k = c * (E / 2) + m;
    axis[m] = k < NT ? 0 : (k < NT + NHW ? 1 : 2);
    rev[m] = p.rev[k];
  }
  const int pos_t = p.frame0 + f;

  float A[E];
#pragma unroll
  for (int e = 0; e < E; ++e) A[e] = 0.f;
  for (int t0 = 0; t0 < len; t0 += kBatch * TL) {
    // the lane's first token of this quarter: row and column by one division, then the
    // column advances by TL per token (wrapping into the next row; a row narrower than TL
    // wraps several times)
    const int tok = j * bs + t0 + s + q * kQuarter * TL;
    int row = tok / p.lat_w;
    int col = tok - row * p.lat_w;
    // the quarter's loads kProLoads at a time, in a loop the compiler keeps rolled: the
    // kernel then fits 64 VGPRs and eight waves per SIMD; the tokens are transformed and
    // added in the same order as with the whole quarter in flight
#pragma unroll 1
    for (int h = 0; h < kQuarter; h += kProLoads) {
      uint4 v[kProLoads];
#pragma unroll
      for (int i = 0; i < kProLoads; ++i) {
        const int t = t0 + s + (q * kQuarter + h + i) * TL;
        v[i] = t < len ? *reinterpret_cast<const uint4*>(xin + static_cast<size_t>(t) * D) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
    for (int i = 0; i < kProLoads; ++i) {
      const int u = h + i;
      const int t = t0 + s + (q * kQuarter + u) * TL;
      if (u > 0) {
        col += TL;
        while (col >= p.lat_w) {
          col -= p.lat_w;
          ++row;
        }
      }
      float x[E];
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = 0.f;
      Chunk16<T>::add(reinterpret_cast<const T*>(&v[i]), x);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) ss = fmaf(x[e], x[e], ss);
      ss = token_sum<C>(ss);
      const float inv = rsqrtf(ss * (1.0f / D) + p.eps);
      // each pair rotated as soon as its angle is known, in place (few live registers)
#pragma unroll
      for (int m = 0; m < E / 2; ++m) {
        float r = static_cast<float>(axis[m] == 0 ? pos_t : (axis[m] == 1 ? row : col)) * rev[m];
        r -= rintf(r);
        const float rc = __builtin_amdgcn_cosf(r), rs = __builtin_amdgcn_sinf(r);
        const float y0 = x[2 * m] * inv * gm[2 * m], y1 = x[2 * m + 1] * inv * gm[2 * m + 1];
        x[2 * m] = Out16<T>::round(y0 * rc - y1 * rs);
        x[2 * m + 1] = Out16<T>::round(y0 * rs + y1 * rc);
      }
      const bool valid = t < len;
      if (valid) Out16<T>::store(yout + static_cast<size_t>(t) * D, x);
#pragma unroll
      for (int e = 0; e < E; ++e) A[e] += valid ? x[e] : 0.f;
    }
    }
  }
  // the block mean from the four quarter sums, in the order lf_pool uses
  if (q > 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) part_s[q - 1][lane][e] = A[e];
  }
  __syncthreads();
  if (q != 0) return;
  float Aq[kQuarters][E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    Aq[0][e] = A[e];
    Aq[1][e] = part_s[0][lane][e];
    Aq[2][e] = part_s[1][lane][e];
    Aq[3][e] = part_s[2][lane][e];
  }
  float sum[E];
  combine_quarters<E, C>(Aq, sum);
  if (lane < C) {
    const float invl = 1.0f / static_cast<float>(len);
    float* out = p.blk + ((static_cast<size_t>(bh) * p.out_stride + f) * n_bpf + j) * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; e += 4)
      *reinterpret_cast<float4*>(out + e) =
          make_float4(sum[e] * invl, sum[e + 1] * invl, sum[e + 2] * invl, sum[e + 3] * invl);
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(kQuarters * kWave) prologue_kernel(ProJob<T> jq, ProJob<T> jk, LagJob lag, int nq_wgs,
                                                                     int nk_wgs, int tpf, int bs, int n_bpf) {
  __shared__ float part_s[kQuarters - 1][kWave][Chunk16<T>::E];
  const int w = blockIdx.x;
  if (w < nq_wgs)
    prologue_block<T, D>(jq, w, tpf, bs, n_bpf, part_s);
  else if (w < nq_wgs + nk_wgs)
    prologue_block<T, D>(jk, w - nq_wgs, tpf, bs, n_bpf, part_s);
  else
    lag_item<D>(lag, (w - nq_wgs - nk_wgs) * (kQuarters * kWave) + threadIdx.x, tpf, bs, n_bpf);
}

template <typename T, int D>
static ProJob<T> pro_job(const ProlArgs& a, const void* x, void* y, const float* gamma, float* blk, long long x_stride,
                         long long y_stride, int out_stride) {
  ProJob<T> p{static_cast<const T*>(x), static_cast<T*>(y), gamma, blk, x_stride, y_stride, a.n_frames, a.frame0,
              out_stride, a.BH * a.n_frames * a.n_bpf, a.lat_w, a.eps, {}};
  for (int k = 0; k < D / 2; ++k) p.rev[k] = a.rev[k];
  return p;
}

template <typename T, int D>
static hipError_t launch_prologue_t(const ProlArgs& a, hipStream_t st) {
  const ProJob<T> p = pro_job<T, D>(a, a.x, a.y, a.gamma, a.blk, a.x_stride, a.y_stride, a.out_stride);
  hipLaunchKernelGGL((prologue_kernel<T, D>), dim3(static_cast<unsigned>(p.n_blocks)), dim3(kQuarters * kWave), 0, st, p,
                     p, no_lag(), p.n_blocks, 0, a.tpf, a.bs, a.n_bpf);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (a.frm == nullptr) return hipSuccess;
  const int n_sf = a.BH * a.n_frames;
  const unsigned fgrid = static_cast<unsigned>((static_cast<long long>(n_sf) * D + kFrameThreads - 1) / kFrameThreads);
  hipLaunchKernelGGL((frame_mean_kernel<D>), dim3(fgrid), dim3(kFrameThreads), 0, st, a.blk, a.frm, n_sf, a.n_frames,
                     a.out_stride, a.tpf, a.bs, a.n_bpf);
  return hipGetLastError();
}

hipError_t launch_prologue(const ProlArgs& a, bool bf16, int d, hipStream_t st) {
  if (bf16) return d == 128 ? launch_prologue_t<__bf16, 128>(a, st) : launch_prologue_t<__bf16, 64>(a, st);
  return d == 128 ? launch_prologue_t<float, 128>(a, st) : launch_prologue_t<float, 64>(a, st);
}

// Queries and the chunk's new keys in one launch (a.x/a.y/a.gamma/a.blk: the queries;
// the step arguments: the keys, written into a KV cache view, their block means into a
// pooled-key cache at frame f_new), plus the lagged frame means.
template <typename T, int D>
static hipError_t launch_prologue_step_t(const ProlArgs& a, const ProlStepArgs& s, hipStream_t st) {
  const ProJob<T> jq = pro_job<T, D>(a, a.x, a.y, a.gamma, a.blk, a.x_stride, a.x_stride, a.n_frames);
  const ProJob<T> jk = pro_job<T, D>(a, s.k, s.k_out, s.gamma_k, s.k_blk + static_cast<size_t>(s.f_new) * a.n_bpf * D,
                                     a.x_stride, s.k_out_stride, s.cache_stride);
  const LagJob lag{s.k_blk, s.k_frm, s.f_lag, s.n_lag > 0 ? s.n_lag : 1, s.cache_stride, a.BH * s.n_lag * D};
  const unsigned grid = static_cast<unsigned>(jq.n_blocks + jk.n_blocks) + lag_wgs<D>(lag);
  hipLaunchKernelGGL((prologue_kernel<T, D>), dim3(grid), dim3(kQuarters * kWave), 0, st, jq, jk, lag, jq.n_blocks,
                     jk.n_blocks, a.tpf, a.bs, a.n_bpf);
  return hipGetLastError();
}

hipError_t launch_prologue_step(const ProlArgs& a, const ProlStepArgs& s, bool bf16, int d, hipStream_t st) {
  if (bf16)
    return d == 128 ? launch_prologue_step_t<__bf16, 128>(a, s, st) : launch_prologue_step_t<__bf16, 64>(a, s, st);
  return d == 128 ? launch_prologue_step_t<float, 128>(a, s, st) : launch_prologue_step_t<float, 64>(a, s, st);
}

}  // namespace lf
