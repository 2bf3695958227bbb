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

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int mask) {
  uint32_t lo = static_cast<uint32_t>(x), hi = static_cast<uint32_t>(x >> 32);
  lo = __shfl_xor(lo, mask, kWave);
  hi = __shfl_xor(hi, mask, kWave);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Bitonic sort, descending, of SEG*P keys held by each SEG-lane segment of the wave:
// element e = p*SEG + (lane % SEG) lives in slot p of that lane. Partners closer than
// SEG are exchanged across lanes (xor shuffles stay inside the segment); farther
// partners are slots of the same lane. Every lane of the wave must call this.
template <int SEG, int P>
__device__ __forceinline__ void bitonic_desc(uint64_t (&key)[P]) {
  const int lane_e = threadIdx.x % SEG;
  constexpr int N = SEG * P;
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= SEG) {
        const int js = j / SEG;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const int q = p ^ js;
          if (q > p) {
            const int e = p * SEG + lane_e;  // lower element of the pair
            const bool desc = (e & k) == 0;
            uint64_t a = key[p], b = key[q];
            uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
            key[p] = desc ? hi : lo;
            key[q] = desc ? lo : hi;
          }
        }
      } else {
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const int e = p * SEG + lane_e;
          const uint64_t other = shfl_xor_u64(key[p], j);
          const bool is_lo = (e & j) == 0;
          const bool desc = (e & k) == 0;
          const bool keep_max = (is_lo == desc);
          const uint64_t mx = key[p] > other ? key[p] : other;
          const uint64_t mn = key[p] > other ? other : key[p];
          key[p] = keep_max ? mx : mn;
        }
      }
    }
  }
}

__device__ __forceinline__ uint64_t lanes_below_mask() {
  const int l = threadIdx.x % kWave;
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace lf
