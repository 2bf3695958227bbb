// Device helpers shared by the HSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lf {

constexpr int kWave = 64;

// Frame-aligned block geometry: block j of a frame covers the frame's tokens
// [j*bs, min((j+1)*bs, tpf)); global block id g = frame*n_bpf + j.
struct BlockGeom {
  int tpf, bs, n_bpf;
  __device__ __forceinline__ int start(int g) const {
    int f = g / n_bpf, j = g - f * n_bpf;
    return f * tpf + j * bs;
  }
  __device__ __forceinline__ int len(int g) const {
    int j = g % n_bpf;
    return min(bs, tpf - j * bs);
  }
};

// Sort key for top-k: larger key = higher score, and among equal scores the lower id.
// Float scores map monotonically onto uint32 (negative zero folded onto zero), the id
// is stored complemented in the low word. Key 0 is below every real key and marks an
// empty slot.
__device__ __forceinline__ uint32_t ordered_bits(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t rank_key(float s, uint32_t id) {
  return (static_cast<uint64_t>(ordered_bits(s)) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - id);
}
__device__ __forceinline__ uint32_t key_id(uint64_t k) {
  return 0xFFFFFFFFu - static_cast<uint32_t>(k);
}

__device__ __forceinline__ uint64_t lanes_below_mask() {
  const int l = threadIdx.x % kWave;
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace lf
