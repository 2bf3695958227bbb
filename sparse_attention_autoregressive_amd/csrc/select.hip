// Two-level mask selection (Light Forcing summary, execution flow, stage 3; technical
// summary section 2.2), one 256-thread workgroup per row (b, h, query block r) for up to
// kListFrames key frames; longer histories take select_long_kernel (further below).
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

// Inner product of the group's q~ slices with the matching slices k of a key row.
template <int D>
__device__ __forceinline__ float slice_dot(const QSlice<D>& q, const float4 (&k)[D / 32]) {
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    a0 = fmaf(q.v[i].x, k[i].x, a0);
    a1 = fmaf(q.v[i].y, k[i].y, a1);
    a0 = fmaf(q.v[i].z, k[i].z, a0);
    a1 = fmaf(q.v[i].w, k[i].w, a1);
  }
  return group_sum(a0 + a1);
}

template <int D>
__device__ __forceinline__ float group_dot(const QSlice<D>& q, const float* __restrict__ row, int c) {
  float4 k[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) k[i] = *reinterpret_cast<const float4*>(row + 4 * c + 32 * i);
  return slice_dot<D>(q, k);
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

// Block stage of nr <= R rows of one head on T threads: each row's T_r (t_s + rr * W_f,
// or the caller's list), SLOTS / R frames of every row per pass, each frame's n_bpf
// block scores ranked and the chosen ids written ascending. Group g scores the blocks of
// row g % R with that row's q~ slices, U block means in flight, so the R rows share each
// pass and its barriers.
template <int D, int R, bool FRAMES, int U = 1, int T = kSelThreads, int SLOTS = kSlots, typename TS>
__device__ __forceinline__ void block_stage(const SelectArgs& a, const QSlice<D> (&q)[R], int row0, int nr, int bh,
                                            int W_f, const TS* t_s, uint64_t (*bkey_s)[64]) {
  constexpr int WAVES = T / kWave, GROUPS = T / kGroup;
  constexpr int S = SLOTS / R;                     // frames of each row per pass
  constexpr int GR = GROUPS / R;                   // groups per row
  static_assert(SLOTS % R == 0 && GROUPS % R == 0, "rows divide the pass");
  if (R == 1) nr = 1;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int grp = threadIdx.x / kGroup, c = threadIdx.x % kGroup;
  const uint64_t below = lanes_below_mask();
  const int n_bpf = a.n_bpf, kb = a.kb_eff;
  auto frame = [&](int rr, int t) { return frame_at<FRAMES>(t_s + rr * W_f, a, row0 + rr, W_f, t); };
  auto out = [&](int rr) { return a.blocks_out + static_cast<size_t>(row0 + rr) * W_f * kb; };
  if (kb >= n_bpf) {                               // every block of every frame is kept
    for (int i = threadIdx.x; i < nr * W_f * n_bpf; i += T) {
      const int u = i / n_bpf, j = i - u * n_bpf;
      const int rr = R == 1 ? 0 : u / W_f, t = u - rr * W_f;
      out(rr)[t * kb + j] = frame(rr, t) * n_bpf + j;
    }
    return;
  }
  const int gr = grp % R, gi = grp / R;
  QSlice<D> qg = q[0];
#pragma unroll
  for (int rr = 1; rr < R; ++rr)
    if (gr == rr) qg = q[rr];
  const float* kbase = a.k_blk + static_cast<size_t>(bh) * a.kf_stride * n_bpf * D;
  for (int t0 = 0; t0 < W_f; t0 += S) {
    const int nt = min(S, W_f - t0);
    if (gr < nr) {
      const int ne = nt * n_bpf;
      for (int e0 = gi; e0 < ne; e0 += U * GR) {
        float4 k[U][D / 32];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int e = min(e0 + u * GR, ne - 1), t = e / n_bpf, j = e - t * n_bpf;
          const float* kr = kbase + (static_cast<size_t>(frame(gr, t0 + t)) * n_bpf + j) * D;
#pragma unroll
          for (int i = 0; i < D / 32; ++i) k[u][i] = *reinterpret_cast<const float4*>(kr + 4 * c + 32 * i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int e = e0 + u * GR;
          if (e >= ne) break;
          const int t = e / n_bpf, j = e - t * n_bpf;
          const float s = slice_dot<D>(qg, k[u]);
          if (c == 0) bkey_s[gr * S + t][j] = rank_key(s, static_cast<uint32_t>(j));
        }
      }
    }
    __syncthreads();
    const int ns = nr * nt;                        // slot u: row u / nt, frame t0 + u % nt
    if (n_bpf <= 32) {
      // two frames per wave at once: lanes 0-31 rank slot ub, lanes 32-63 slot ub + 1
      const int half = lane >> 5, jl = lane & 31;
      const uint64_t below_half = jl == 0 ? 0ull : (~0ull >> (64 - jl)) << (32 * half);
      for (int ub = 2 * wave; ub < ns; ub += 2 * WAVES) {
        const int u = ub + half;
        const int rr = R == 1 ? 0 : u / nt, t = u - rr * nt;
        const bool on = u < ns && jl < n_bpf && rank_of(bkey_s[rr * S + t][jl], bkey_s[rr * S + t], n_bpf) < kb;
        const uint64_t m = __ballot(on);
        if (on) out(rr)[(t0 + t) * kb + __popcll(m & below_half)] = frame(rr, t0 + t) * n_bpf + jl;
      }
    } else {
      for (int u = wave; u < ns; u += WAVES) {
        const int rr = R == 1 ? 0 : u / nt, t = u - rr * nt;
        const bool on = lane < n_bpf && rank_of(bkey_s[rr * S + t][lane], bkey_s[rr * S + t], n_bpf) < kb;
        const uint64_t m = __ballot(on);
        if (on) out(rr)[(t0 + t) * kb + __popcll(m & below)] = frame(rr, t0 + t) * n_bpf + lane;
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

  const QSlice<D> q1[1] = {q};
  block_stage<D, 1, FRAMES>(a, q1, row, 1, bh, W_f, t_s, bkey_s);
}

// Maximum (MAX) or minimum of x over the wave, in every lane: within rows of 16 lanes by
// DPP moves (pairs, quads, half rows, rows), then across row pairs and wave halves.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), CTRL, 0xF, 0xF, false));
}
template <bool MAX>
__device__ __forceinline__ uint32_t pick(uint32_t x, uint32_t y) {
  return MAX ? max(x, y) : min(x, y);
}
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x) {
  x = pick<MAX>(x, dpp_u32<0xB1>(x));    // quad_perm [1, 0, 3, 2]
  x = pick<MAX>(x, dpp_u32<0x4E>(x));    // quad_perm [2, 3, 0, 1]
  x = pick<MAX>(x, dpp_u32<0x141>(x));   // row_half_mirror
  x = pick<MAX>(x, dpp_u32<0x140>(x));   // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = pick<MAX>(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return pick<MAX>(b[0], b[1]);
}

// Position of the largest score over the wave's (score, position) pairs, ties to the
// lower position (positions are distinct); every lane gets it. Ties across lanes are
// rare, so a single holder is read directly.
__device__ __forceinline__ uint32_t wave_top_pos(uint32_t score, uint32_t pos) {
  const uint32_t top = wave_reduce<true>(score);
  const uint64_t holders = __ballot(score == top);
  return __popcll(holders) == 1
             ? static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(pos), __builtin_ctzll(holders)))
             : wave_reduce<false>(score == top ? pos : 0xFFFFFFFFu);
}

// Sum of x over the lanes below this one, for 0 <= x < 128: bit b of the sum's terms is
// counted with a ballot, so no value crosses lanes through LDS.
__device__ __forceinline__ int wave_excl_sum(int x) {
  const uint64_t below = lanes_below_mask();
  int s = 0;
#pragma unroll
  for (int b = 0; b < 7; ++b) s += __popcll(__ballot((x >> b) & 1) & below) << b;
  return s;
}

// LDS layout of select_long_kernel, in bytes from the start of dynamic LDS.
struct LongLds {
  int n_words, sc_stride;                // mask words per row; score entries per row (4 k)
  size_t bits, t, mem, total;            // offsets of the row bits, T_r, the ids of M; size
};
__host__ __device__ inline LongLds long_lds(int R, int n_mem, int n_kframes, int W_f, bool keep_all) {
  LongLds L;
  L.n_words = (n_kframes + 63) / 64;
  L.sc_stride = (n_mem + 3) & ~3;
  L.bits = keep_all ? 0 : static_cast<size_t>(R) * L.sc_stride * 4;
  L.t = L.bits + static_cast<size_t>(R) * L.n_words * 8;
  L.mem = L.t + static_cast<size_t>(R) * W_f * 2;
  L.total = L.mem + static_cast<size_t>(n_mem) * 2;
  return L;
}

// Selection for calls with more than kListFrames key frames (long histories).
// - M and the always-kept frames arrive as bit masks. Wave 0 stores M's 64-frame words
//   and, per word, the count of members before it (a prefix over the words'
//   populations); every thread then places its frames' ids in ascending order.
// - A 512-thread workgroup takes kLongRows consecutive rows of one head. Every row scores
//   the same frames of M, so each frame mean an 8-lane group loads is dotted with both
//   rows' q~ slices (the same group inner product, term for term, as the listed
//   kernel's), which halves the frame means' L2 traffic; each group keeps kLongUnroll
//   frame means in flight. Scores are stored as 32-bit order-preserving bits per row.
// - Wave w takes row w's top k_eff (lane l reads positions 4 l + 256 i + 0..3 of M,
//   16 bytes at a time). The largest score wins, at its lowest position when several are
//   equal, which ranks M as the listed kernel's (score, lower frame id first) keys do,
//   since positions ascend with frame ids. The candidates are first cut to the scores at
//   or above the k_eff-th largest of the lanes' maxima (they include the top k_eff); up to
//   64 of them, one per lane, leave each round two wave reductions. Otherwise (k_eff > 64,
//   or many equal scores) each round scans all of the row's scores. Each winner sets its
//   frame's bit over the always-kept frames' bits.
// - Each row's bits are compacted into T_r by the same prefix count, and both rows' block
//   stages share passes (block_stage with two rows).
constexpr int kLongUnroll = 4;                     // frame means in flight per group
constexpr int kLongRows = 2;                       // rows per workgroup
constexpr int kLongSlots = 16;                     // block-stage frames per pass
constexpr int kLongBlockUnroll = 2;                // block means in flight per group
constexpr int kLongThreads = 512;                  // threads per workgroup

template <int D, bool BLOCKS>
__global__ void __launch_bounds__(kLongThreads) select_long_kernel(SelectArgs a) {
  constexpr int R = kLongRows, T = kLongThreads, GROUPS = T / kGroup;
  static_assert(R >= 1 && R <= T / kWave, "one row per wave in the top-k rounds");
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_s[];
  __shared__ uint64_t bkey_s[kLongSlots][64];
  __shared__ uint64_t mw_s[kMaxFrames / 64];       // M's mask words
  __shared__ int16_t pre_s[kMaxFrames / 64];       // members of M in the words before
  __shared__ uint2 cand_s[kLongRows][kWave];       // top-k candidates (score, position) per row
  const int n_mem = a.n_mem, W_f = a.W_f;
  const bool keep_all = a.k_eff >= n_mem;
  const LongLds L = long_lds(R, n_mem, a.n_kframes, W_f, keep_all);
  uint32_t* sc_s = reinterpret_cast<uint32_t*>(dyn_s);
  uint64_t* bits_s = reinterpret_cast<uint64_t*>(dyn_s + L.bits);
  int16_t* t_s = reinterpret_cast<int16_t*>(dyn_s + L.t);
  int16_t* mem_s = reinterpret_cast<int16_t*>(dyn_s + L.mem);

  // R rows of one head per workgroup, head-major over the XCDs
  const int groups = (a.n_qb + R - 1) / R;
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per = nwg / 8, rem = nwg % 8;
  const int gid = xcd * per + min(xcd, rem) + slot;
  const int bh = gid / groups, j0 = (gid - bh * groups) * R;
  const int row0 = bh * a.n_qb + j0, nr = min(R, a.n_qb - j0);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int grp = threadIdx.x / kGroup, c = threadIdx.x % kGroup;

  QSlice<D> q[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const float* qr = a.q_blk + static_cast<size_t>(row0 + min(rr, nr - 1)) * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) q[rr].v[i] = *reinterpret_cast<const float4*>(qr + 4 * c + 32 * i);
  }
  for (int i = threadIdx.x; i < R * W_f; i += T) t_s[i] = 0;   // every T_r entry a valid id
  if (!keep_all && threadIdx.x < R * (L.sc_stride - n_mem))      // score places past |M|: none
    sc_s[(threadIdx.x / (L.sc_stride - n_mem)) * L.sc_stride + n_mem + threadIdx.x % (L.sc_stride - n_mem)] = 0u;
  static_assert(kMaxFrames / 64 == kWave, "one mask word per lane of wave 0");
  if (wave == 0) {
    const uint64_t mw = lane < L.n_words ? a.masks.mem[lane] : 0ull;
    const uint64_t fw = lane < L.n_words ? a.masks.forced[lane] : 0ull;
    mw_s[lane] = mw;
    pre_s[lane] = static_cast<int16_t>(wave_excl_sum(__popcll(mw)));
    if (lane < L.n_words) {
#pragma unroll
      for (int rr = 0; rr < R; ++rr) bits_s[rr * L.n_words + lane] = keep_all ? (fw | mw) : fw;
    }
  }
  __syncthreads();
  // M's ids in ascending order: frame f goes to the members below it
  for (int f = threadIdx.x; f < a.n_kframes; f += T) {
    const uint64_t w = mw_s[f / 64];
    const int b = f % 64;
    if ((w >> b) & 1ull) mem_s[pre_s[f / 64] + __popcll(w & ((1ull << b) - 1))] = static_cast<int16_t>(f);
  }
  __syncthreads();
  if (!keep_all) {
    // kLongUnroll frame means per group in flight: each group walks ~|M| / 64 frames
    const float* kf = a.k_frm + static_cast<size_t>(bh) * a.kf_stride * D;
    for (int e0 = grp; e0 < n_mem; e0 += kLongUnroll * GROUPS) {
      float4 k[kLongUnroll][D / 32];
#pragma unroll
      for (int u = 0; u < kLongUnroll; ++u) {
        const float* kr = kf + static_cast<size_t>(mem_s[min(e0 + u * GROUPS, n_mem - 1)]) * D;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) k[u][i] = *reinterpret_cast<const float4*>(kr + 4 * c + 32 * i);
      }
#pragma unroll
      for (int u = 0; u < kLongUnroll; ++u) {
        const int e = e0 + u * GROUPS;
        if (e >= n_mem) break;
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          if (rr < nr) {
            const float s = slice_dot<D>(q[rr], k[u]);
            if (c == 0) sc_s[rr * L.sc_stride + e] = max(ordered_bits(s), 1u);   // 0 marks a taken entry
          }
        }
      }
    }
    __syncthreads();
    if (wave < nr) {
      // wave w: row w's scores in LDS; lane l reads positions 4 l + 256 i + (0..3) of M
      // (consecutive lanes, consecutive 16-byte chunks: no bank conflicts), four chunks
      // per batch
      uint32_t* scr = sc_s + wave * L.sc_stride;
      uint64_t* bits = bits_s + wave * L.n_words;
      auto scan = [&](auto&& f) {                // f(score, position), ascending positions
        for (int b0 = 4 * lane; b0 < n_mem; b0 += 4 * 4 * kWave) {
          uint4 v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int p = b0 + u * 4 * kWave;
            v[u] = p < n_mem ? *reinterpret_cast<const uint4*>(scr + p) : make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int p = b0 + u * 4 * kWave;
            if (p < n_mem) {                     // places past |M| in the chunk hold 0
              f(v[u].x, p);
              f(v[u].y, p + 1);
              f(v[u].z, p + 2);
              f(v[u].w, p + 3);
            }
          }
        }
      };
      auto keep = [&](uint32_t pos) {
        if (lane == 0) {
          const int f = mem_s[min(static_cast<int>(pos), n_mem - 1)];
          bits[f / 64] |= 1ull << (f % 64);
        }
      };
      // Candidates: every score at or above t, the k_eff-th largest of the lanes' maxima.
      // The lanes holding those maxima hold k_eff scores >= t, so the row's top k_eff are
      // all candidates; with at most 64 of them, one per lane, a round is two reductions.
      bool done = false;
      if (a.k_eff <= kWave) {
        uint32_t v = 0;
        scan([&](uint32_t x, int) { v = max(v, x); });
        uint32_t t = 0;
        for (int r = 0; r < a.k_eff; ++r) {
          t = wave_reduce<true>(v);
          if (lane == __builtin_ctzll(__ballot(v == t))) v = 0;
        }
        t = max(t, 1u);                          // 0 is no score
        int cnt = 0;
        scan([&](uint32_t x, int) { cnt += x >= t ? 1 : 0; });
        int off = wave_excl_sum(cnt);            // cnt <= 4 |M| / 256 <= 64
        const int total = __builtin_amdgcn_readlane(off + cnt, kWave - 1);
        if (total <= kWave) {
          uint2* cand = cand_s[wave];
          scan([&](uint32_t x, int p) {
            if (x >= t) cand[off++] = make_uint2(x, static_cast<uint32_t>(p));
          });
          uint32_t cs = lane < total ? cand[lane].x : 0u;
          const uint32_t cp = lane < total ? cand[lane].y : 0u;
          for (int r = 0; r < a.k_eff; ++r) {
            const uint32_t win = wave_top_pos(cs, cp);
            if (cp == win) cs = 0u;
            keep(win);
          }
          done = true;
        }
      }
      if (!done) {
        // every score: a round takes the largest remaining and clears it (lane 0 writes
        // the 0; the wave's later reads of the row see it, LDS operations of a wave
        // being done in order)
        for (int r = 0; r < a.k_eff; ++r) {
          uint32_t best = 0, bpos = 0;
          scan([&](uint32_t x, int p) {
            const bool gt = x > best;            // ascending positions: ties keep the lower
            best = gt ? x : best;
            bpos = gt ? static_cast<uint32_t>(p) : bpos;
          });
          const uint32_t win = wave_top_pos(best, bpos);
          if (lane == 0) scr[min(static_cast<int>(win), n_mem - 1)] = 0u;
          keep(win);
        }
      }
    }
    __syncthreads();
  }
  if (wave < nr) {
    const uint64_t w = lane < L.n_words ? bits_s[wave * L.n_words + lane] : 0ull;
    int pos = wave_excl_sum(__popcll(w));
    int16_t* t = t_s + wave * W_f;
    int* fo = a.frames_out ? a.frames_out + static_cast<size_t>(row0 + wave) * W_f : nullptr;
    for (uint64_t m = w; m && pos < W_f; m &= m - 1, ++pos) {
      const int f = 64 * lane + __builtin_ctzll(m);
      t[pos] = static_cast<int16_t>(f);
      if (fo) fo[pos] = f;
    }
  }
  if (!BLOCKS) return;
  __syncthreads();
  block_stage<D, R, true, kLongBlockUnroll, T, kLongSlots>(a, q, row0, nr, bh, W_f, t_s, bkey_s);
}

constexpr size_t kLongLdsMax = 160 * 1024 - sizeof(uint64_t) * kLongSlots * 64;

template <int D, bool BLOCKS>
static hipError_t launch_select_long_d(const SelectArgs& a, int n_rows, hipStream_t st) {
  const int n_bh = n_rows / a.n_qb, groups = (a.n_qb + kLongRows - 1) / kLongRows;
  const size_t lds = long_lds(kLongRows, a.n_mem, a.n_kframes, a.W_f, a.k_eff >= a.n_mem).total;
  if (lds > kLongLdsMax) return hipErrorInvalidValue;
  if (lds > 64 * 1024) {
    // dynamic LDS past 64 KB is declared for the kernel (up to the 160 KB a workgroup can
    // address); a runtime that does not need the declaration may refuse it, so its status
    // is cleared and the launch's own status decides
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&select_long_kernel<D, BLOCKS>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLongLdsMax));
    (void)hipGetLastError();
  }
  hipLaunchKernelGGL((select_long_kernel<D, BLOCKS>), dim3(static_cast<unsigned>(n_bh * groups)),
                     dim3(kLongThreads), static_cast<unsigned>(lds), st, a);
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
