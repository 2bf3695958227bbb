// Two-level mask selection (Light Forcing summary, execution flow, stage 3).
//
// select_frames: one wave per row (b, h, query block r). Lane l of slot p owns frame
// f = 64p + l; if f is in the memory set M it scores p_r(f) = <q~_r, k^_f> (q~_r is
// broadcast from LDS, k^_f streamed with 16-byte loads) and packs (score, id) into a
// 64-bit key. A wave bitonic sort (descending; equal scores -> lower id first) puts
// the top-min(k_f, |M|) frames in the first elements; they and the always-kept frames
// are flagged in LDS and emitted in ascending order with a ballot prefix count.
//
// select_blocks: frame-major. One 256-thread workgroup per (b, h, frame tau, tile of
// 64 query blocks) first finds which rows of its tile listed tau (and at which slot t
// of T_r), then stages the frame's n_bpf pooled keys k~^(tau) in LDS once and scores
// o_r(tau, j) = <q~_r, k~_j^(tau)> for those rows only, one row per SEG-lane segment
// (lane j = block j). A segment bitonic sort selects J_r(tau); the chosen ids
// tau*n_bpf + j go to slots t*k_b .. t*k_b + k_b - 1 of the row's list in ascending j.
// Frames listed by no row of the tile cost one scan and exit.
#include "lf_device.h"
#include "lf_kernels.h"

namespace lf {

template <int D>
__device__ __forceinline__ float dot_lds_global(const float* q_lds, const float* __restrict__ k) {
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 8
  for (int c = 0; c < D; c += 4) {
    const float4 kv = *reinterpret_cast<const float4*>(k + c);
    const float4 qv = *reinterpret_cast<const float4*>(q_lds + c);
    a0 = fmaf(qv.x, kv.x, a0);
    a1 = fmaf(qv.y, kv.y, a1);
    a2 = fmaf(qv.z, kv.z, a2);
    a3 = fmaf(qv.w, kv.w, a3);
  }
  return (a0 + a1) + (a2 + a3);
}

template <int D, int P>
__global__ void __launch_bounds__(256) select_frames_kernel(const float* __restrict__ q_blk,
                                                            const float* __restrict__ k_frm,
                                                            int n_rows, int n_qb, int n_kframes,
                                                            FrameSets sets, int k_eff, int W_f,
                                                            int* __restrict__ frames_out) {
  __shared__ __attribute__((aligned(16))) float q_s[4][D];
  __shared__ unsigned char flag_s[4][64 * P];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int row = blockIdx.x * 4 + wave;
  if (row >= n_rows) return;  // whole wave leaves; no workgroup barrier follows
  const int bh = row / n_qb;

  for (int c = lane; c < D; c += kWave) q_s[wave][c] = q_blk[static_cast<size_t>(row) * D + c];
#pragma unroll
  for (int p = 0; p < P; ++p) flag_s[wave][p * 64 + lane] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const float* kf = k_frm + static_cast<size_t>(bh) * n_kframes * D;
  uint64_t key[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int f = p * 64 + lane;
    key[p] = 0;
    if (f < n_kframes && ((sets.mem[p] >> lane) & 1ull)) {
      key[p] = rank_key(dot_lds_global<D>(q_s[wave], kf + static_cast<size_t>(f) * D), f);
    }
  }
  bitonic_desc<64, P>(key);

  // flag always-kept frames and the k_eff best memory frames
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int f = p * 64 + lane;
    if ((sets.forced[p] >> lane) & 1ull) flag_s[wave][f] = 1;
    if (p * 64 + lane < k_eff && key[p] != 0) flag_s[wave][key_id(key[p])] = 1;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  int* out = frames_out + static_cast<size_t>(row) * W_f;
  int count = 0;
  const uint64_t below = lanes_below_mask();
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int f = p * 64 + lane;
    const bool on = f < n_kframes && flag_s[wave][f] != 0;
    const uint64_t m = __ballot(on);
    const int pos = count + __popcll(m & below);
    if (on && pos < W_f) out[pos] = f;
    count += __popcll(m);
  }
}

template <int D, int SEG>
__global__ void __launch_bounds__(256) select_blocks_kernel(
    const float* __restrict__ q_blk, const float* __restrict__ k_blk,
    const int* __restrict__ frames, int n_qb, int n_kframes, int n_bpf, int W_f, int k_b,
    int kb_eff, int n_tiles, int* __restrict__ blocks_out) {
  constexpr int SEGS = 64 / SEG;  // rows per wave pass
  __shared__ __attribute__((aligned(16))) float k_s[SEG][D + 4];
  __shared__ int item_s[64 * 4];   // (row in tile) | (slot t << 8)
  __shared__ int count_s;
  __shared__ unsigned char flag_s[4][64];

  const int tile = blockIdx.x % n_tiles;
  const int rest = blockIdx.x / n_tiles;
  const int tau = rest % n_kframes;
  const int bh = rest / n_kframes;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int W_b = W_f * kb_eff;

  // 1. rows of this tile whose T_r contains tau (wave 0; one lane per row)
  if (wave == 0) {
    const int r = tile * 64 + lane;
    int slot = -1;
    if (r < n_qb) {
      const int* fr = frames + (static_cast<size_t>(bh) * n_qb + r) * W_f;
      for (int t = 0; t < W_f; ++t) {
        if (fr[t] == tau) { slot = t; break; }
      }
    }
    const bool on = slot >= 0;
    const uint64_t m = __ballot(on);
    if (on) item_s[__popcll(m & lanes_below_mask())] = lane | (slot << 8);
    if (lane == 0) count_s = __popcll(m);
  }
  __syncthreads();
  const int count = count_s;
  if (count == 0) return;

  const size_t row0 = static_cast<size_t>(bh) * n_qb + tile * 64;
  if (kb_eff >= n_bpf) {  // every block of the frame is kept: no scores needed
    for (int i = threadIdx.x; i < count * n_bpf; i += 256) {
      const int it = item_s[i / n_bpf], j = i % n_bpf;
      const int r = it & 0xFF, t = it >> 8;
      blocks_out[(row0 + r) * W_b + t * kb_eff + j] = tau * n_bpf + j;
    }
    return;
  }

  // 2. stage k~^(tau): n_bpf rows of D floats
  const float* kb = k_blk + (static_cast<size_t>(bh) * n_kframes + tau) * n_bpf * D;
  for (int i = threadIdx.x; i < n_bpf * (D / 4); i += 256) {
    const int j = i / (D / 4), c = (i % (D / 4)) * 4;
    *reinterpret_cast<float4*>(&k_s[j][c]) = *reinterpret_cast<const float4*>(kb + j * D + c);
  }
  __syncthreads();

  // 3. score, select and emit, one row per segment
  const int seg = lane / SEG, j = lane % SEG;
  const uint64_t below = lanes_below_mask();
  const uint64_t seg_mask = (SEG == 64) ? ~0ull : (0xFFFFFFFFull << (seg * SEG));
  for (int base = wave * SEGS; base < count; base += 4 * SEGS) {
    const int i = base + seg;
    const bool active = i < count;
    const int it = active ? item_s[i] : 0;
    const int r = it & 0xFF, t = it >> 8;
    uint64_t key[1] = {0};
    if (active && j < n_bpf) {
      const float* q = q_blk + (row0 + r) * D;
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 8
      for (int c = 0; c < D; c += 4) {
        const float4 qv = *reinterpret_cast<const float4*>(q + c);
        const float4 kv = *reinterpret_cast<const float4*>(&k_s[j][c]);
        a0 = fmaf(qv.x, kv.x, a0);
        a1 = fmaf(qv.y, kv.y, a1);
        a2 = fmaf(qv.z, kv.z, a2);
        a3 = fmaf(qv.w, kv.w, a3);
      }
      key[0] = rank_key((a0 + a1) + (a2 + a3), j);
    }
    bitonic_desc<SEG, 1>(key);
    // element j of the sorted segment holds the (j+1)-th best block
    flag_s[wave][lane] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (active && j < kb_eff) flag_s[wave][seg * SEG + key_id(key[0])] = 1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const bool on = active && j < n_bpf && flag_s[wave][lane] != 0;
    const uint64_t m = __ballot(on) & seg_mask;
    if (on) {
      const int pos = __popcll(m & below);
      blocks_out[(row0 + r) * W_b + t * kb_eff + pos] = tau * n_bpf + j;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int D>
static hipError_t launch_select_frames_d(const float* q_blk, const float* k_frm, int n_rows,
                                         int n_qb, int n_kframes, const FrameSets& sets,
                                         int k_eff, int W_f, int* out, hipStream_t st) {
  const dim3 grid((n_rows + 3) / 4), block(256);
  if (n_kframes <= 64)
    hipLaunchKernelGGL((select_frames_kernel<D, 1>), grid, block, 0, st, q_blk, k_frm, n_rows,
                       n_qb, n_kframes, sets, k_eff, W_f, out);
  else if (n_kframes <= 128)
    hipLaunchKernelGGL((select_frames_kernel<D, 2>), grid, block, 0, st, q_blk, k_frm, n_rows,
                       n_qb, n_kframes, sets, k_eff, W_f, out);
  else
    hipLaunchKernelGGL((select_frames_kernel<D, 4>), grid, block, 0, st, q_blk, k_frm, n_rows,
                       n_qb, n_kframes, sets, k_eff, W_f, out);
  return hipGetLastError();
}

hipError_t launch_select_frames(const float* q_blk, const float* k_frm, int d, int n_rows,
                                int n_qb, int n_kframes, const FrameSets& sets, int k_eff,
                                int W_f, int* out, hipStream_t st) {
  return d == 128 ? launch_select_frames_d<128>(q_blk, k_frm, n_rows, n_qb, n_kframes, sets,
                                                k_eff, W_f, out, st)
                  : launch_select_frames_d<64>(q_blk, k_frm, n_rows, n_qb, n_kframes, sets,
                                               k_eff, W_f, out, st);
}

template <int D>
static hipError_t launch_select_blocks_d(const float* q_blk, const float* k_blk, const int* frames,
                                         int BH, int n_qb, int n_kframes, int n_bpf, int W_f,
                                         int k_b, int kb_eff, int* out, hipStream_t st) {
  const int n_tiles = (n_qb + 63) / 64;
  const dim3 grid(static_cast<unsigned>(BH) * n_kframes * n_tiles), block(256);
  if (n_bpf <= 32)
    hipLaunchKernelGGL((select_blocks_kernel<D, 32>), grid, block, 0, st, q_blk, k_blk, frames,
                       n_qb, n_kframes, n_bpf, W_f, k_b, kb_eff, n_tiles, out);
  else
    hipLaunchKernelGGL((select_blocks_kernel<D, 64>), grid, block, 0, st, q_blk, k_blk, frames,
                       n_qb, n_kframes, n_bpf, W_f, k_b, kb_eff, n_tiles, out);
  return hipGetLastError();
}

hipError_t launch_select_blocks(const float* q_blk, const float* k_blk, const int* frames, int d,
                                int BH, int n_qb, int n_kframes, int n_bpf, int W_f, int k_b,
                                int kb_eff, int* out, hipStream_t st) {
  return d == 128 ? launch_select_blocks_d<128>(q_blk, k_blk, frames, BH, n_qb, n_kframes, n_bpf,
                                                W_f, k_b, kb_eff, out, st)
                  : launch_select_blocks_d<64>(q_blk, k_blk, frames, BH, n_qb, n_kframes, n_bpf,
                                               W_f, k_b, kb_eff, out, st);
}

}  // namespace lf
