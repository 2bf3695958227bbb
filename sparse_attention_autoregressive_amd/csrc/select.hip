// Two-level mask selection (Light Forcing summary, execution flow, stage 3).
//
// select_frames: one 512-thread workgroup per (b, h, tile of 16 query blocks). The tile's
// q~ rows and, when |M| <= 64, the memory set's frame means k^_f are staged in LDS with
// coalesced loads; each wave then takes two rows. Lane l of slot p owns candidate
// e = 64p + l (the e-th frame of M in ascending id order) and scores
// p_r(f) = <q~_r, k^_f>, packed with the frame id into a 64-bit key. A wave bitonic
// sort (descending; equal scores -> lower id first) puts the top-min(k_f, |M|) frames in
// the first elements; they and the always-kept frames are flagged in LDS and emitted in
// ascending order with a ballot prefix count.
//
// select_blocks: frame-major. One 512-thread workgroup per (b, h, frame tau, tile of 16
// query blocks) stages the tile's q~ rows and the frame's n_bpf pooled keys k~^(tau) in
// LDS while wave 0 finds which rows listed tau (and at which slot t of T_r). Each wave
// then scores o_r(tau, j) = <q~_r, k~_j^(tau)> for up to two rows (one per SEG-lane
// segment, lane j = block j), a segment bitonic sort selects J_r(tau), and the chosen
// ids tau*n_bpf + j go to slots t*k_b .. t*k_b + k_b - 1 of the row's list in ascending
// j. Rows that did not list tau cost nothing beyond the scan.
#include "lf_device.h"
#include "lf_kernels.h"

namespace lf {

constexpr int kSelRows = 16;     // query blocks per workgroup
constexpr int kSelThreads = 512;

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__device__ __forceinline__ float dot4(const float* q, const float* k) {
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 8
  for (int c = 0; c < D; c += 4) {
    const float4 qv = *reinterpret_cast<const float4*>(q + c);
    const float4 kv = *reinterpret_cast<const float4*>(k + c);
    a0 = fmaf(qv.x, kv.x, a0);
    a1 = fmaf(qv.y, kv.y, a1);
    a2 = fmaf(qv.z, kv.z, a2);
    a3 = fmaf(qv.w, kv.w, a3);
  }
  return (a0 + a1) + (a2 + a3);
}

// Stages `rows` rows of D floats from global (row stride D) into LDS (row stride D + 4),
// using threads [t0, t0 + nt) of the workgroup.
template <int D>
__device__ __forceinline__ void stage_rows(float* dst, const float* __restrict__ src, int rows,
                                           int t0, int nt) {
  for (int i = static_cast<int>(threadIdx.x) - t0; i < rows * (D / 4); i += nt) {
    const int rr = i / (D / 4), cc = (i % (D / 4)) * 4;
    *reinterpret_cast<float4*>(dst + rr * (D + 4) + cc) =
        *reinterpret_cast<const float4*>(src + static_cast<size_t>(rr) * D + cc);
  }
}

template <int D, int P>
__global__ void __launch_bounds__(kSelThreads) select_frames_kernel(
    const float* __restrict__ q_blk, const float* __restrict__ k_frm, int n_qb, int n_kframes,
    FrameSets sets, int n_mem, int k_eff, int W_f, int n_tiles, int* __restrict__ frames_out) {
  constexpr int WAVES = kSelThreads / kWave;
  constexpr int STAGE = 64;                       // memory frames staged in LDS at most
  __shared__ __attribute__((aligned(16))) float q_s[kSelRows][D + 4];
  __shared__ __attribute__((aligned(16))) float k_s[STAGE][D + 4];
  __shared__ int mem_s[64 * P];
  __shared__ unsigned char flag_s[WAVES][64 * P];

  const int tile = blockIdx.x % n_tiles, bh = blockIdx.x / n_tiles;
  const int r0 = tile * kSelRows;
  const int rows = min(kSelRows, n_qb - r0);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const size_t row_base = static_cast<size_t>(bh) * n_qb + r0;
  const float* kf = k_frm + static_cast<size_t>(bh) * n_kframes * D;
  const bool staged = n_mem <= STAGE;

  // ascending list of memory frames (wave 0), q~ rows (all)
  if (wave == 0) {
    int count = 0;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const bool on = (sets.mem[p] >> lane) & 1ull;
      const uint64_t m = __ballot(on);
      if (on) mem_s[count + __popcll(m & lanes_below_mask())] = p * 64 + lane;
      count += __popcll(m);
    }
  }
  stage_rows<D>(&q_s[0][0], q_blk + row_base * D, rows, 0, kSelThreads);
  __syncthreads();
  if (staged) {
    for (int i = threadIdx.x; i < n_mem * (D / 4); i += blockDim.x) {
      const int rr = i / (D / 4), cc = (i % (D / 4)) * 4;
      *reinterpret_cast<float4*>(&k_s[rr][cc]) =
          *reinterpret_cast<const float4*>(kf + static_cast<size_t>(mem_s[rr]) * D + cc);
    }
    __syncthreads();
  }

  const uint64_t below = lanes_below_mask();
  for (int rr = wave; rr < rows; rr += WAVES) {
    uint64_t key[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int e = p * 64 + lane;
      key[p] = 0;
      if (e < n_mem) {
        const int f = mem_s[e];
        const float s = staged ? dot4<D>(q_s[rr], k_s[e]) : dot4<D>(q_s[rr], kf + static_cast<size_t>(f) * D);
        key[p] = rank_key(s, f);
      }
      flag_s[wave][p * 64 + lane] = 0;
    }
    bitonic_desc<64, P>(key);
    wave_lds_sync();
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int f = p * 64 + lane;
      if ((sets.forced[p] >> lane) & 1ull) flag_s[wave][f] = 1;
      if (p * 64 + lane < k_eff && key[p] != 0) flag_s[wave][key_id(key[p])] = 1;
    }
    wave_lds_sync();
    int* out = frames_out + (row_base + rr) * W_f;
    int count = 0;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int f = p * 64 + lane;
      const bool on = f < n_kframes && flag_s[wave][f] != 0;
      const uint64_t m = __ballot(on);
      const int pos = count + __popcll(m & below);
      if (on && pos < W_f) out[pos] = f;
      count += __popcll(m);
    }
    wave_lds_sync();
  }
}

template <int D, int SEG>
__global__ void __launch_bounds__(kSelThreads) select_blocks_kernel(
    const float* __restrict__ q_blk, const float* __restrict__ k_blk,
    const int* __restrict__ frames, int n_qb, int n_kframes, int n_bpf, int W_f, int kb_eff,
    int n_tiles, int* __restrict__ blocks_out) {
  constexpr int WAVES = kSelThreads / kWave;
  constexpr int SEGS = 64 / SEG;  // rows per wave pass
  __shared__ __attribute__((aligned(16))) float k_s[SEG][D + 4];
  __shared__ __attribute__((aligned(16))) float q_s[kSelRows][D + 4];
  __shared__ int item_s[kSelRows];   // (row in tile) | (slot t << 8)
  __shared__ int count_s;
  __shared__ unsigned char flag_s[WAVES][64];

  const int tile = blockIdx.x % n_tiles;
  const int rest = blockIdx.x / n_tiles;
  const int tau = rest % n_kframes;
  const int bh = rest / n_kframes;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int W_b = W_f * kb_eff;
  const int r0 = tile * kSelRows;
  const int rows = min(kSelRows, n_qb - r0);
  const size_t row_base = static_cast<size_t>(bh) * n_qb + r0;
  const bool all_blocks = kb_eff >= n_bpf;

  // 1. rows of this tile whose T_r contains tau (wave 0, one lane per row), while the
  //    other waves stage q~ rows and k~^(tau)
  if (wave == 0) {
    int slot = -1;
    if (lane < rows) {
      const int* fr = frames + (row_base + lane) * W_f;
      for (int t = 0; t < W_f; ++t) {
        if (fr[t] == tau) { slot = t; break; }
      }
    }
    const bool on = slot >= 0;
    const uint64_t m = __ballot(on);
    if (on) item_s[__popcll(m & lanes_below_mask())] = lane | (slot << 8);
    if (lane == 0) count_s = __popcll(m);
  } else if (!all_blocks) {
    stage_rows<D>(&k_s[0][0], k_blk + (static_cast<size_t>(bh) * n_kframes + tau) * n_bpf * D, n_bpf,
                  kWave, kSelThreads - kWave);
    stage_rows<D>(&q_s[0][0], q_blk + row_base * D, rows, kWave, kSelThreads - kWave);
  }
  __syncthreads();
  const int count = count_s;
  if (count == 0) return;

  if (all_blocks) {  // every block of the frame is kept: no scores needed
    for (int i = threadIdx.x; i < count * n_bpf; i += blockDim.x) {
      const int it = item_s[i / n_bpf], jj = i % n_bpf;
      blocks_out[(row_base + (it & 0xFF)) * W_b + (it >> 8) * kb_eff + jj] = tau * n_bpf + jj;
    }
    return;
  }

  // 2. score, select and emit, one row per segment
  const int seg = lane / SEG, j = lane % SEG;
  const uint64_t below = lanes_below_mask();
  const uint64_t seg_mask = (SEG == 64) ? ~0ull : (0xFFFFFFFFull << (seg * SEG));
  for (int base = wave * SEGS; base < count; base += WAVES * SEGS) {
    const int i = base + seg;
    const bool active = i < count;
    const int it = active ? item_s[i] : 0;
    const int r = it & 0xFF, t = it >> 8;
    uint64_t key[1] = {0};
    if (active && j < n_bpf) key[0] = rank_key(dot4<D>(q_s[r], k_s[j]), j);
    bitonic_desc<SEG, 1>(key);
    // element j of the sorted segment holds the (j+1)-th best block
    flag_s[wave][lane] = 0;
    wave_lds_sync();
    if (active && j < kb_eff) flag_s[wave][seg * SEG + key_id(key[0])] = 1;
    wave_lds_sync();
    const bool on = active && j < n_bpf && flag_s[wave][lane] != 0;
    const uint64_t m = __ballot(on) & seg_mask;
    if (on) blocks_out[(row_base + r) * W_b + t * kb_eff + __popcll(m & below)] = tau * n_bpf + j;
    wave_lds_sync();
  }
}

template <int D>
static hipError_t launch_select_frames_d(const float* q_blk, const float* k_frm, int BH, int n_qb,
                                         int n_kframes, const FrameSets& sets, int n_mem,
                                         int k_eff, int W_f, int* out, hipStream_t st) {
  const int n_tiles = (n_qb + kSelRows - 1) / kSelRows;
  const dim3 grid(static_cast<unsigned>(BH) * n_tiles), block(kSelThreads);
  if (n_kframes <= 64)
    hipLaunchKernelGGL((select_frames_kernel<D, 1>), grid, block, 0, st, q_blk, k_frm, n_qb,
                       n_kframes, sets, n_mem, k_eff, W_f, n_tiles, out);
  else if (n_kframes <= 128)
    hipLaunchKernelGGL((select_frames_kernel<D, 2>), grid, block, 0, st, q_blk, k_frm, n_qb,
                       n_kframes, sets, n_mem, k_eff, W_f, n_tiles, out);
  else
    hipLaunchKernelGGL((select_frames_kernel<D, 4>), grid, block, 0, st, q_blk, k_frm, n_qb,
                       n_kframes, sets, n_mem, k_eff, W_f, n_tiles, out);
  return hipGetLastError();
}

hipError_t launch_select_frames(const float* q_blk, const float* k_frm, int d, int BH, int n_qb,
                                int n_kframes, const FrameSets& sets, int n_mem, int k_eff,
                                int W_f, int* out, hipStream_t st) {
  return d == 128 ? launch_select_frames_d<128>(q_blk, k_frm, BH, n_qb, n_kframes, sets, n_mem,
                                                k_eff, W_f, out, st)
                  : launch_select_frames_d<64>(q_blk, k_frm, BH, n_qb, n_kframes, sets, n_mem,
                                               k_eff, W_f, out, st);
}

template <int D>
static hipError_t launch_select_blocks_d(const float* q_blk, const float* k_blk, const int* frames,
                                         int BH, int n_qb, int n_kframes, int n_bpf, int W_f,
                                         int kb_eff, int* out, hipStream_t st) {
  const int n_tiles = (n_qb + kSelRows - 1) / kSelRows;
  const dim3 grid(static_cast<unsigned>(BH) * n_kframes * n_tiles), block(kSelThreads);
  if (n_bpf <= 32)
    hipLaunchKernelGGL((select_blocks_kernel<D, 32>), grid, block, 0, st, q_blk, k_blk, frames,
                       n_qb, n_kframes, n_bpf, W_f, kb_eff, n_tiles, out);
  else
    hipLaunchKernelGGL((select_blocks_kernel<D, 64>), grid, block, 0, st, q_blk, k_blk, frames,
                       n_qb, n_kframes, n_bpf, W_f, kb_eff, n_tiles, out);
  return hipGetLastError();
}

hipError_t launch_select_blocks(const float* q_blk, const float* k_blk, const int* frames, int d,
                                int BH, int n_qb, int n_kframes, int n_bpf, int W_f, int kb_eff,
                                int* out, hipStream_t st) {
  return d == 128 ? launch_select_blocks_d<128>(q_blk, k_blk, frames, BH, n_qb, n_kframes, n_bpf,
                                                W_f, kb_eff, out, st)
                  : launch_select_blocks_d<64>(q_blk, k_blk, frames, BH, n_qb, n_kframes, n_bpf,
                                               W_f, kb_eff, out, st);
}

}  // namespace lf
