// Measurement aids: the dense bf16 matrix-core ceiling (register-only MFMA chains, no
// memory traffic inside the loop, plus the shader clock over the loop measured against
// the 100 MHz reference) and the achievable HBM read rate (a plain streaming read).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "lf_kernels.h"

namespace lf {

typedef __bf16 bf16x8v __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16v __attribute__((__vector_size__(16 * sizeof(float))));

__global__ void __launch_bounds__(256) mfma_probe_kernel(float* __restrict__ sink, long long* __restrict__ clocks,
                                                         int iters) {
  bf16x8v a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(1e-3f * static_cast<float>((threadIdx.x + i) & 63));
    b[i] = static_cast<__bf16>(2e-3f * static_cast<float>(i));
  }
  f32x16v c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const long long t0 = __builtin_readcyclecounter();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  const long long t1 = __builtin_readcyclecounter();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clocks[0] = t1 - t0;
    clocks[1] = r1 - r0;
  }
}

hipError_t launch_mfma_probe(int n_wg, int iters, float* sink, long long* clocks, hipStream_t st) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(static_cast<unsigned>(n_wg)), dim3(256), 0, st, sink, clocks, iters);
  return hipGetLastError();
}

// Streaming read: every thread reads 16-byte chunks i, i + stride, ... of the buffer with
// eight loads in flight and folds them into one float (so the loads are kept).
constexpr int kReadThreads = 256;
__global__ void __launch_bounds__(kReadThreads) hbm_read_kernel(const uint4* __restrict__ x, long long n16,
                                                                float* __restrict__ sink) {
  const long long tid = static_cast<long long>(blockIdx.x) * kReadThreads + threadIdx.x;
  const long long stride = static_cast<long long>(gridDim.x) * kReadThreads;
  uint32_t acc = 0;
  long long i = tid;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = x[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = x[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[tid] = __uint_as_float(acc);
}

hipError_t launch_hbm_read(const void* x, long long bytes, int n_wg, float* sink, hipStream_t st) {
  hipLaunchKernelGGL(hbm_read_kernel, dim3(static_cast<unsigned>(n_wg)), dim3(kReadThreads), 0, st,
                     static_cast<const uint4*>(x), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace lf
