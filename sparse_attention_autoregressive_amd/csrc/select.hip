// Two-level mask selection (Light Forcing summary, execution flow, stage 3; technical
// summary section 2.2), one 256-thread workgroup per row (b, h, query block r).
//
// Scores. Every inner product of the row's pooled query q~_r with a pooled key (a frame
// mean k^_f or a block mean k~_j^(tau)) is computed by a group of 8 lanes: lane c of the
// group holds q~ elements 4c + 32i .. +3 (i < d/32) in registers and reads the same
// elements of the key row, so each 16-byte load of the group covers one whole 128-byte
// line of the row. The 8 partial sums are added with DPP lane moves in a fixed order
// (deterministic), and the group's first lane stores the score, packed with its id into
// a 64-bit rank key (larger = better; equal scores -> lower id first), in LDS.
//
// Frame stage: keys of the memory set M; thread e counts the keys above its own (its
// rank) and keeps frame e if the rank is below min(k_f, |M|) (every frame of M, with no
// scores computed, when k_f >= |M|). The frame ids of M and of the always-kept frames are
// read with q~ at the start, one per thread, so no list read waits in this chain. The kept
// frames and the always-kept ones are flagged by frame id and compacted in ascending
// order into T_r.
//
// Block stage: keys of the n_bpf blocks of each frame of T_r (up to kSlots frames per
// pass); the waves rank the blocks of the pass's frames the same way -- two frames per
// wave at once, one per half-wave, when n_bpf <= 32 -- and write the chosen ids
// tau*n_bpf + j, ascending in j, to slots t*k_b .. t*k_b + k_b - 1 of the row's list.
// When k_b covers the frame, every block is listed without scoring.
//
// Rows are dealt head-major to the XCDs, so one head's pooled keys stay in one L2.
#include "lf_device.h"
#include "lf_kernels.h"

namespace lf {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kGroup = 8;                          // lanes per inner product
constexpr int kGroups = kSelThreads / kGroup;      // inner products in flight per pass
constexpr int kSlots = 16;                         // frames of T_r scored per pass
static_assert(kListFrames == kSelThreads, "one listed frame id per thread");

// x + (x of the lane the DPP control selects), within rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float add_dpp(float x) {
  const int y = __builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false);
  return x + __int_as_float(y);
}

// Sum over the 8 lanes of a group (aligned to 8): pairs (xor 1), quads (xor 2), then the
// two quads (mirror within each half row of 8). Every lane of the group gets the same value.
__device__ __forceinline__ float group_sum(float x) {
  x = add_dpp<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  x = add_dpp<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x = add_dpp<0x141>(x);   // row_half_mirror
  return x;
}

// q~ slice of lane c of a group: elements 4c + 32i .. 4c + 32i + 3.
template <int D>
struct QSlice {
  float4 v[D / 32];
};

template <int D>
__device__ __forceinline__ float group_dot(const QSlice<D>& q, const float* __restrict__ row, int c) {
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    const float4 k = *reinterpret_cast<const float4*>(row + 4 * c + 32 * i);
    a0 = fmaf(q.v[i].x, k.x, a0);
    a1 = fmaf(q.v[i].y, k.y, a1);
    a0 = fmaf(q.v[i].z, k.z, a0);
    a1 = fmaf(q.v[i].w, k.w, a1);
  }
  return group_sum(a0 + a1);
}

// Number of keys among keys[0..n) above `mine` (keys are distinct).
// Eight keys are read per step, so their LDS reads are in flight together.
__device__ __forceinline__ int rank_of(uint64_t mine, const uint64_t* keys, int n) {
  int r = 0, i = 0;
  for (; i + 8 <= n; i += 8) {
    uint64_t k[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) k[u] = keys[i + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) r += k[u] > mine ? 1 : 0;
  }
  for (; i < n; ++i) r += keys[i] > mine ? 1 : 0;
  return r;
}

// Frame tau of slot t of T_r: from LDS when the frame stage ran, else from the caller's
// list, clamped into [0, n_kframes).
template <bool FRAMES, typename TS>
__device__ __forceinline__ int frame_at(const TS* t_s, const SelectArgs& a, int row, int W_f, int t) {
  return FRAMES ? t_s[t] : min(max(a.frames_in[static_cast<size_t>(row) * W_f + t], 0), a.n_kframes - 1);
}

// Block stage of one row: T_r's frames (t_s, or the caller's list), up to kSlots per
// pass, each frame's n_bpf block scores ranked and the chosen ids written ascending.
template <int D, bool FRAMES, typename TS>
__device__ __forceinline__ void block_stage(const SelectArgs& a, const QSlice<D>& q, int row, int bh, int W_f,
                                            const TS* t_s, uint64_t (*bkey_s)[64]) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int grp = threadIdx.x / kGroup, c = threadIdx.x % kGroup;
  const uint64_t below = lanes_below_mask();
  const int n_bpf = a.n_bpf, kb = a.kb_eff;
  int* out = a.blocks_out + static_cast<size_t>(row) * W_f * kb;
  if (kb >= n_bpf) {                               // every block of every frame is kept
    for (int i = threadIdx.x; i < W_f * n_bpf; i += kSelThreads) {
      const int t = i / n_bpf, j = i - t * n_bpf;
      out[t * kb + j] = frame_at<FRAMES>(t_s, a, row, W_f, t) * n_bpf + j;
    }
    return;
  }
  const float* kbase = a.k_blk + static_cast<size_t>(bh) * a.kf_stride * n_bpf * D;
  for (int t0 = 0; t0 < W_f; t0 += kSlots) {
    const int nt = min(kSlots, W_f - t0);
    for (int e = grp; e < nt * n_bpf; e += kGroups) {
      const int t = e / n_bpf, j = e - t * n_bpf;
      const float s = group_dot<D>(q, kbase + (static_cast<size_t>(frame_at<FRAMES>(t_s, a, row, W_f, t0 + t)) * n_bpf + j) * D, c);
      if (c == 0) bkey_s[t][j] = rank_key(s, static_cast<uint32_t>(j));
    }
    __syncthreads();
    if (n_bpf <= 32) {
      // two frames per wave at once: lanes 0-31 rank slot tb, lanes 32-63 slot tb + 1
      const int half = lane >> 5, jl = lane & 31;
      const uint64_t below_half = jl == 0 ? 0ull : (~0ull >> (64 - jl)) << (32 * half);
      for (int tb = 2 * wave; tb < nt; tb += 2 * kSelWaves) {
        const int t = tb + half;
        const bool on = t < nt && jl < n_bpf && rank_of(bkey_s[t][jl], bkey_s[t], n_bpf) < kb;
        const uint64_t m = __ballot(on);
        if (on) out[(t0 + t) * kb + __popcll(m & below_half)] = frame_at<FRAMES>(t_s, a, row, W_f, t0 + t) * n_bpf + jl;
      }
    } else {
      for (int t = wave; t < nt; t += kSelWaves) {
        const bool mine = lane < n_bpf;
        const bool on = mine && rank_of(bkey_s[t][lane], bkey_s[t], n_bpf) < kb;
        const uint64_t m = __ballot(on);
        if (on) out[(t0 + t) * kb + __popcll(m & below)] = frame_at<FRAMES>(t_s, a, row, W_f, t0 + t) * n_bpf + lane;
      }
    }
    __syncthreads();
  }
}

// FRAMES: compute T_r (and write it if frames_out is set); otherwise read it from
// frames_in, clamping ids into [0, n_kframes) so a malformed list cannot send a read out
// of bounds. BLOCKS: compute and write the block list.
template <int D, bool FRAMES, bool BLOCKS>
__global__ void __launch_bounds__(kSelThreads) select_kernel(SelectArgs a) {
  __shared__ uint64_t fkey_s[kListFrames];         // frame-stage keys, by position in M
  __shared__ unsigned char flag_s[kListFrames];
  __shared__ int t_s[kListFrames];                 // T_r
  __shared__ uint64_t bkey_s[kSlots][64];          // block-stage keys of one pass

  // head-major rows, consecutive rows on one XCD (workgroups are dealt round-robin)
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per = nwg / 8, rem = nwg % 8;
  const int row = xcd * per + min(xcd, rem) + slot;        // b*H*n_qb + h*n_qb + r
  const int bh = row / a.n_qb;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int grp = threadIdx.x / kGroup, c = threadIdx.x % kGroup;
  const uint64_t below = lanes_below_mask();

  QSlice<D> q;
  {
    const float* qr = a.q_blk + static_cast<size_t>(row) * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) q.v[i] = *reinterpret_cast<const float4*>(qr + 4 * c + 32 * i);
  }

  // ids of M and of the always-kept frames, one per thread, read with q~ at the start
  const int mem_id = FRAMES && threadIdx.x < a.n_mem ? a.lists.mem[threadIdx.x] : -1;
  const int forced_id = FRAMES && threadIdx.x < a.n_forced ? a.lists.forced[threadIdx.x] : -1;

  int W_f = a.W_f;
  if (FRAMES) {
    // when the budget covers M every memory frame is kept, and no score is needed
    const bool keep_all = a.k_eff >= a.n_mem;
    const float* kf = a.k_frm + static_cast<size_t>(bh) * a.kf_stride * D;
    for (int e = grp; !keep_all && e < a.n_mem; e += kGroups) {
      const int f = a.lists.mem[e];
      const float s = group_dot<D>(q, kf + static_cast<size_t>(f) * D, c);
      if (c == 0) fkey_s[e] = rank_key(s, static_cast<uint32_t>(f));
    }
    for (int i = threadIdx.x; i < a.n_kframes; i += kSelThreads) flag_s[i] = 0;
    __syncthreads();
    if (mem_id >= 0 && (keep_all || rank_of(fkey_s[threadIdx.x], fkey_s, a.n_mem) < a.k_eff))
      flag_s[mem_id] = 1;
    if (forced_id >= 0) flag_s[forced_id] = 1;
    __syncthreads();
    if (wave == 0) {
      int count = 0;
      for (int f0 = 0; f0 < a.n_kframes; f0 += kWave) {
        const int f = f0 + lane;
        const bool on = f < a.n_kframes && flag_s[f] != 0;
        const uint64_t m = __ballot(on);
        const int pos = count + __popcll(m & below);
        if (on) {
          t_s[pos] = f;
          if (a.frames_out) a.frames_out[static_cast<size_t>(row) * W_f + pos] = f;
        }
        count += __popcll(m);
      }
    }
    if (!BLOCKS) return;
    __syncthreads();
  }

  block_stage<D, FRAMES>(a, q, row, bh, W_f, t_s, bkey_s);
}

// Frame stage for calls with more than kListFrames key frames (long histories): M and the
// always-kept frames arrive as bit masks and wave 0 expands them in LDS (ascending ids);
// the ids, keys, flags and T_r live in dynamic LDS sized for the call. Frame scores are
// the same 8-lane inner products as above; the top k_eff keys are taken in k_eff rounds,
// each the block-wide maximum of the keys below the previous round's (keys are distinct,
// and a key carries its frame id), so a round costs one pass over |M| / 256 keys per
// thread rather than a rank count over all |M| keys. Results equal the listed kernel's.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    const uint64_t y = __shfl_xor(x, m, kWave);
    x = y > x ? y : x;
  }
  return x;
}

template <int D, bool BLOCKS>
__global__ void __launch_bounds__(kSelThreads) select_long_kernel(SelectArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_s[];
  __shared__ uint64_t bkey_s[kSlots][64];
  __shared__ uint64_t max_s[2][kSelWaves];
  const int n_mem = a.n_mem, n_kf = a.n_kframes, W_f = a.W_f;
  // dynamic LDS: keys [n_mem] | T_r [W_f] | ids of M [n_mem] | flags [n_kframes]
  uint64_t* keys_s = reinterpret_cast<uint64_t*>(dyn_s);
  int16_t* t_s = reinterpret_cast<int16_t*>(keys_s + n_mem);
  int16_t* mem_s = t_s + W_f;
  unsigned char* flag_s = reinterpret_cast<unsigned char*>(mem_s + n_mem);

  const int nwg = gridDim.x;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per = nwg / 8, rem = nwg % 8;
  const int row = xcd * per + min(xcd, rem) + slot;
  const int bh = row / a.n_qb;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int grp = threadIdx.x / kGroup, c = threadIdx.x % kGroup;
  const uint64_t below = lanes_below_mask();

  QSlice<D> q;
  {
    const float* qr = a.q_blk + static_cast<size_t>(row) * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) q.v[i] = *reinterpret_cast<const float4*>(qr + 4 * c + 32 * i);
  }
  if (wave == 0) {
    int mcount = 0;
    for (int f0 = 0; f0 < n_kf; f0 += kWave) {
      const uint64_t mw = a.masks.mem[f0 / kWave], fw = a.masks.forced[f0 / kWave];
      const int f = f0 + lane;
      if (f < n_kf) flag_s[f] = static_cast<unsigned char>((fw >> lane) & 1ull);
      if ((mw >> lane) & 1ull) mem_s[mcount + __popcll(mw & below)] = static_cast<int16_t>(f);
      mcount += __popcll(mw);
    }
  }
  __syncthreads();
  const bool keep_all = a.k_eff >= n_mem;
  if (keep_all) {
    for (int e = threadIdx.x; e < n_mem; e += kSelThreads) flag_s[mem_s[e]] = 1;
  } else {
    const float* kf = a.k_frm + static_cast<size_t>(bh) * a.kf_stride * D;
    for (int e = grp; e < n_mem; e += kGroups) {
      const int f = mem_s[e];
      const float s = group_dot<D>(q, kf + static_cast<size_t>(f) * D, c);
      if (c == 0) keys_s[e] = rank_key(s, static_cast<uint32_t>(f));
    }
    __syncthreads();
    uint64_t bound = ~0ull;
    for (int r = 0; r < a.k_eff; ++r) {
      uint64_t best = 0;
      for (int e = threadIdx.x; e < n_mem; e += kSelThreads) {
        const uint64_t k = keys_s[e];
        if (k < bound && k > best) best = k;
      }
      best = wave_max_u64(best);
      if (lane == 0) max_s[r & 1][wave] = best;
      __syncthreads();
      bound = max_s[r & 1][0];
#pragma unroll
      for (int w = 1; w < kSelWaves; ++w) bound = max_s[r & 1][w] > bound ? max_s[r & 1][w] : bound;
      if (threadIdx.x == 0) flag_s[key_id(bound)] = 1;
    }
  }
  __syncthreads();
  if (wave == 0) {
    int count = 0;
    for (int f0 = 0; f0 < n_kf; f0 += kWave) {
      const int f = f0 + lane;
      const bool on = f < n_kf && flag_s[f] != 0;
      const uint64_t m = __ballot(on);
      const int pos = count + __popcll(m & below);
      if (on) {
        t_s[pos] = static_cast<int16_t>(f);
        if (a.frames_out) a.frames_out[static_cast<size_t>(row) * W_f + pos] = f;
      }
      count += __popcll(m);
    }
  }
  if (!BLOCKS) return;
  __syncthreads();
  block_stage<D, true>(a, q, row, bh, W_f, t_s, bkey_s);
}

// Dynamic LDS of select_long_kernel.
static size_t long_select_lds(const SelectArgs& a) {
  return static_cast<size_t>(a.n_mem) * 8 + static_cast<size_t>(a.W_f) * 2 + static_cast<size_t>(a.n_mem) * 2 +
         static_cast<size_t>(a.n_kframes);
}

template <int D, bool BLOCKS>
static hipError_t launch_select_long_d(const SelectArgs& a, int n_rows, hipStream_t st) {
  hipLaunchKernelGGL((select_long_kernel<D, BLOCKS>), dim3(static_cast<unsigned>(n_rows)), dim3(kSelThreads),
                     static_cast<unsigned>(long_select_lds(a)), st, a);
  return hipGetLastError();
}

template <int D, bool FRAMES, bool BLOCKS>
static hipError_t launch_select_d(const SelectArgs& a, int n_rows, hipStream_t st) {
  hipLaunchKernelGGL((select_kernel<D, FRAMES, BLOCKS>), dim3(static_cast<unsigned>(n_rows)),
                     dim3(kSelThreads), 0, st, a);
  return hipGetLastError();
}

template <bool FRAMES, bool BLOCKS>
static hipError_t launch_select_t(const SelectArgs& a, int d, int n_rows, hipStream_t st) {
  return d == 128 ? launch_select_d<128, FRAMES, BLOCKS>(a, n_rows, st)
                  : launch_select_d<64, FRAMES, BLOCKS>(a, n_rows, st);
}

hipError_t launch_select(const SelectArgs& a, int d, int n_rows, bool frames, bool blocks, hipStream_t st) {
  if (frames && a.n_kframes > kListFrames) {
    if (blocks)
      return d == 128 ? launch_select_long_d<128, true>(a, n_rows, st) : launch_select_long_d<64, true>(a, n_rows, st);
    return d == 128 ? launch_select_long_d<128, false>(a, n_rows, st) : launch_select_long_d<64, false>(a, n_rows, st);
  }
  if (frames && blocks) return launch_select_t<true, true>(a, d, n_rows, st);
  if (frames) return launch_select_t<true, false>(a, d, n_rows, st);
  return launch_select_t<false, true>(a, d, n_rows, st);
}

// ---------------------------------------------------------------------------------
// Single-level selection (the one-granularity variant HSA is contrasted with): every key
// block of the prefix is scored by the same 8-lane group dot product, the rank keys go to
// LDS, a bitonic sort over the next power of two (empty slots hold key 0, below every
// real key) orders them, the first K ids are flagged, and wave 0 compacts the flags into
// the row's ascending list.
constexpr int kMax1D = 4096;                       // key blocks per row (LDS keys: 32 KB)

template <int D>
__global__ void __launch_bounds__(kSelThreads) select_1d_kernel(Select1DArgs a) {
  __shared__ uint64_t key_s[kMax1D];
  __shared__ unsigned char flag_s[kMax1D];
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per = nwg / 8, rem = nwg % 8;
  const int row = xcd * per + min(xcd, rem) + slot;
  const int bh = row / a.n_qb;
  const int grp = threadIdx.x / kGroup, c = threadIdx.x % kGroup;
  const int n = a.n_kb;
  int np2 = 1;
  while (np2 < n) np2 <<= 1;

  QSlice<D> q;
  {
    const float* qr = a.q_blk + static_cast<size_t>(row) * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) q.v[i] = *reinterpret_cast<const float4*>(qr + 4 * c + 32 * i);
  }
  const float* kbase = a.k_blk + static_cast<size_t>(bh) * a.kb_stride * D;
  for (int e = grp; e < n; e += kGroups) {
    const float sc = group_dot<D>(q, kbase + static_cast<size_t>(e) * D, c);
    if (c == 0) key_s[e] = rank_key(sc, static_cast<uint32_t>(e));
  }
  for (int e = n + threadIdx.x; e < np2; e += kSelThreads) key_s[e] = 0;
  for (int e = threadIdx.x; e < n; e += kSelThreads) flag_s[e] = 0;
  __syncthreads();
  // bitonic sort, descending
  for (int k = 2; k <= np2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < np2 / 2; i += kSelThreads) {
        const int lo = 2 * i - (i & (j - 1)), hi = lo + j;
        const uint64_t x = key_s[lo], y = key_s[hi];
        const bool desc = (lo & k) == 0;
        if (desc ? x < y : x > y) {
          key_s[lo] = y;
          key_s[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < a.K; i += kSelThreads) flag_s[key_id(key_s[i])] = 1;
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const uint64_t below = lanes_below_mask();
    int* out = a.blocks_out + static_cast<size_t>(row) * a.K;
    int count = 0;
    for (int e0 = 0; e0 < n; e0 += kWave) {
      const int e = e0 + lane;
      const bool on = e < n && flag_s[e] != 0;
      const uint64_t m = __ballot(on);
      if (on) out[count + __popcll(m & below)] = e;
      count += __popcll(m);
    }
  }
}

hipError_t launch_select_1d(const Select1DArgs& a, int d, int n_rows, hipStream_t st) {
  if (d == 128)
    hipLaunchKernelGGL((select_1d_kernel<128>), dim3(static_cast<unsigned>(n_rows)), dim3(kSelThreads), 0, st, a);
  else
    hipLaunchKernelGGL((select_1d_kernel<64>), dim3(static_cast<unsigned>(n_rows)), dim3(kSelThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace lf
