// Token compression by mean pooling (Light Forcing summary, execution flow, stage 2):
// block-level means of queries and keys, frame-level means of keys.
//
// pool_blocks: one 256-thread workgroup per (b, h, block). The block's tokens are
// streamed once from HBM with 16-byte loads: thread t reads chunk t % C of every
// P-th token (C = 16-byte chunks per token, P = 256 / C token lanes), accumulating in
// fp32; the P partial sums meet in LDS and are added in a fixed order, so results are
// deterministic. Many small workgroups (B*H*n_frames*n_bpf) keep every CU streaming.
//
// frame_means: one workgroup per (b, h, frame), d threads; weights the frame's fp32
// block means by their token counts (the true frame mean up to fp32 rounding).
#include "lf_device.h"
#include "lf_kernels.h"

namespace lf {

template <typename T>
__device__ __forceinline__ void load16_to_f32(const T* p, float* out);

template <>
__device__ __forceinline__ void load16_to_f32<float>(const float* p, float* out) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}

template <>
__device__ __forceinline__ void load16_to_f32<__bf16>(const __bf16* p, float* out) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(256) pool_blocks_kernel(const T* __restrict__ x,
                                                          float* __restrict__ blk,
                                                          int n_frames, int tpf, int bs,
                                                          int n_bpf, long long x_stride) {
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int C = D / E;           // chunks per token
  constexpr int P = 256 / C;         // tokens in flight per pass
  __shared__ float red[P][D + 4];

  const int nb = n_frames * n_bpf;
  const int bh = blockIdx.x / nb;
  const int gb = blockIdx.x - bh * nb;
  const int f = gb / n_bpf, j = gb - f * n_bpf;
  const int len = min(bs, tpf - j * bs);
  const T* base = x + (static_cast<size_t>(bh) * x_stride + f * tpf + j * bs) * D;

  const int c = threadIdx.x % C, s = threadIdx.x / C;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;

  int t = s;
  for (; t + 3 * P < len; t += 4 * P) {  // four independent loads in flight
    float v0[E], v1[E], v2[E], v3[E];
    load16_to_f32<T>(base + static_cast<size_t>(t) * D + c * E, v0);
    load16_to_f32<T>(base + static_cast<size_t>(t + P) * D + c * E, v1);
    load16_to_f32<T>(base + static_cast<size_t>(t + 2 * P) * D + c * E, v2);
    load16_to_f32<T>(base + static_cast<size_t>(t + 3 * P) * D + c * E, v3);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += ((v0[e] + v1[e]) + (v2[e] + v3[e]));
  }
  for (; t < len; t += P) {
    float v0[E];
    load16_to_f32<T>(base + static_cast<size_t>(t) * D + c * E, v0);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += v0[e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[s][c * E + e] = acc[e];
  __syncthreads();

  const float inv = 1.0f / static_cast<float>(len);
  for (int i = threadIdx.x; i < D; i += 256) {
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < P; ++r) sum += red[r][i];
    blk[(static_cast<size_t>(bh) * nb + gb) * D + i] = sum * inv;
  }
}

template <int D>
__global__ void __launch_bounds__(D) frame_means_kernel(const float* __restrict__ blk,
                                                        float* __restrict__ frm, int n_frames,
                                                        int tpf, int bs, int n_bpf) {
  const int bh = blockIdx.x / n_frames;
  const int f = blockIdx.x - bh * n_frames;
  const float* b = blk + (static_cast<size_t>(bh) * n_frames + f) * n_bpf * D + threadIdx.x;
  float sum = 0.f;
#pragma unroll 8
  for (int j = 0; j < n_bpf; ++j) sum = fmaf(b[j * D], static_cast<float>(min(bs, tpf - j * bs)), sum);
  frm[(static_cast<size_t>(bh) * n_frames + f) * D + threadIdx.x] = sum / static_cast<float>(tpf);
}

template <typename T, int D>
static hipError_t launch_pool_t(const void* x, int BH, int n_frames, int tpf, int bs, int n_bpf,
                                long long x_stride, float* blk, float* frm, hipStream_t st) {
  const unsigned nblk = static_cast<unsigned>(BH) * n_frames * n_bpf;
  hipLaunchKernelGGL((pool_blocks_kernel<T, D>), dim3(nblk), dim3(256), 0, st,
                     static_cast<const T*>(x), blk, n_frames, tpf, bs, n_bpf, x_stride);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || frm == nullptr) return e;
  hipLaunchKernelGGL((frame_means_kernel<D>), dim3(static_cast<unsigned>(BH) * n_frames), dim3(D),
                     0, st, blk, frm, n_frames, tpf, bs, n_bpf);
  return hipGetLastError();
}

hipError_t launch_pool(const void* x, bool bf16, int d, int BH, int n_frames, int tpf, int bs,
                       int n_bpf, long long x_stride, float* blk, float* frm, hipStream_t st) {
  if (bf16) {
    return d == 128 ? launch_pool_t<__bf16, 128>(x, BH, n_frames, tpf, bs, n_bpf, x_stride, blk, frm, st)
                    : launch_pool_t<__bf16, 64>(x, BH, n_frames, tpf, bs, n_bpf, x_stride, blk, frm, st);
  }
  return d == 128 ? launch_pool_t<float, 128>(x, BH, n_frames, tpf, bs, n_bpf, x_stride, blk, frm, st)
                  : launch_pool_t<float, 64>(x, BH, n_frames, tpf, bs, n_bpf, x_stride, blk, frm, st);
}

}  // namespace lf
