// Block-sparse attention over the HSA mask (Light Forcing summary, execution flow,
// stage 3; gist.science technical summary, section 2.2): every query token of query
// block r attends only to the tokens of the key blocks listed for r, with a softmax
// over those tokens.
//
// attn_bf16_kernel -- the hot path, bf16 in / bf16 out, fp32 accumulation and softmax.
//   One 128-thread workgroup (2 waves) per row (b, h, r); wave w owns query rows
//   [32w, 32w+32) of the block. Listed key blocks are walked as 32-token tiles (a 64-token
//   block is two tiles, a short block one masked tile). Each tile's K and V rows are
//   copied global -> LDS with direct 16-byte loads (no VGPR staging), double-buffered so
//   the next tile streams in while the current one is used, and stored with a 16-byte
//   chunk XOR swizzle so the MFMA operand reads are bank-conflict free.
//   Both products run on bf16 matrix cores (v_mfma_f32_32x32x16_bf16) in transposed
//   form so one lane always owns one query row:
//     S^T = K Q^T   (A = K tile from LDS, B = Q fragment kept in registers)
//     O^T += V^T P^T (A = V^T fragment gathered from LDS, B = P^T straight from the
//                     S^T accumulator after exp2, no lane shuffles)
//   The softmax runs in base 2 with scale*log2(e) folded into the logits. Weights are
//   taken against a per-query reference: the normalised output sum(p v) / sum(p) does not
//   depend on it, and bf16/fp32 weights keep their relative precision anywhere in their
//   exponent range, so the reference only has to keep the weights finite. A first pass
//   fixes it at the query's maximum over the row's first tile and spends no work on a
//   running maximum. If a later score rose far above it (a row sum beyond 2^64 or not
//   finite), the workgroup redoes the row with the running maximum (the classic online
//   softmax: the O accumulator and row sum are rescaled when a tile's maximum exceeds the
//   one in use by more than a slack). Row sums come from the matrix cores.
//   Workgroups are numbered head-major and spread so that consecutive rows (same head,
//   same K/V working set) land on the same XCD and share its L2.
//
// attn_f32_kernel -- fp32 variant (small problems, e.g. d=64 checks), one thread per
//   query token, exact fp32 dot products and exp2 on the vector units.
#include "lf_device.h"
#include "lf_kernels.h"

namespace lf {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------------- fp32
template <int D>
__global__ void __launch_bounds__(128) attn_f32_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) float k_s[32][D];
  __shared__ __attribute__((aligned(16))) float v_s[32][D];
  const int row = blockIdx.x;
  const int bh = row / a.n_qb, r = row - bh * a.n_qb;
  const BlockGeom geo{a.tpf, a.bs, a.n_bpf};
  const int q_start = geo.start(r), q_len = geo.len(r);
  const int t = threadIdx.x;

  const float* Q = static_cast<const float*>(a.q) +
                   (static_cast<size_t>(bh) * a.q_stride + q_start + min(t, q_len - 1)) * D;
  float q[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) { q[c] = Q[c]; o[c] = 0.f; }
  float m = -1e30f, lsum = 0.f;

  const float* K = static_cast<const float*>(a.k) + static_cast<size_t>(bh) * a.kv_stride * D;
  const float* V = static_cast<const float*>(a.v) + static_cast<size_t>(bh) * a.kv_stride * D;
  const int* bl = a.blocks + static_cast<size_t>(row) * a.W_b;

  for (int n = 0; n < a.W_b; ++n) {
    const int g = bl[n];
    if (g < 0 || g >= a.n_kb) continue;
    const int ks = geo.start(g), kl = geo.len(g);
    for (int p = 0; p < kl; p += 32) {
      const int nv = min(32, kl - p);
      __syncthreads();
      for (int i = t; i < nv * (D / 4); i += 128) {
        const int rr = i / (D / 4), c = (i % (D / 4)) * 4;
        const size_t off = static_cast<size_t>(ks + p + rr) * D + c;
        *reinterpret_cast<float4*>(&k_s[rr][c]) = *reinterpret_cast<const float4*>(K + off);
        *reinterpret_cast<float4*>(&v_s[rr][c]) = *reinterpret_cast<const float4*>(V + off);
      }
      __syncthreads();
      float s[32];
      float mt = m;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        s[i] = -INFINITY;
        if (i < nv) {
          float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
          for (int c = 0; c < D; c += 4) {
            a0 = fmaf(q[c], k_s[i][c], a0);
            a1 = fmaf(q[c + 1], k_s[i][c + 1], a1);
            a2 = fmaf(q[c + 2], k_s[i][c + 2], a2);
            a3 = fmaf(q[c + 3], k_s[i][c + 3], a3);
          }
          s[i] = ((a0 + a1) + (a2 + a3)) * a.scale_log2;
          mt = fmaxf(mt, s[i]);
        }
      }
      const float corr = exp2f(m - mt);
      m = mt;
      lsum *= corr;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] *= corr;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i < nv) {
          const float pi = exp2f(s[i] - m);
          lsum += pi;
#pragma unroll
          for (int c = 0; c < D; ++c) o[c] = fmaf(pi, v_s[i][c], o[c]);
        }
      }
    }
  }
  if (t < q_len) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    float* O = static_cast<float*>(a.o) + (static_cast<size_t>(bh) * a.q_stride + q_start + t) * D;
#pragma unroll
    for (int c = 0; c < D; c += 4)
      *reinterpret_cast<float4*>(O + c) = make_float4(o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv);
  }
}

// ---------------------------------------------------------------------------------- bf16
typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) void lds_void;
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): inside each group of 16 lanes, lane
// c receives element (c % 4) of the 8-byte words addressed by lanes c/4, 4 + c/4,
// 8 + c/4 and 12 + c/4, i.e. lane 4r + q supplies row r, columns 4q..4q+3 of a 4 x 16
// tile of 16-bit values and lane c gets column c.
__device__ __forceinline__ uint2 ds_read_tr16(const lds_u8* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
  return __builtin_bit_cast(uint2, v);
}

// Running-max slack (log2 units): the O accumulator and row sum are rescaled only when
// a tile's maximum exceeds the max in use by more than this, so p = 2^(x - m) <= 2^8.
constexpr float kRescaleSlack = 8.0f;
// Fixed-reference pass: a row sum at or beyond this (weights up to ~2^64 above the
// reference) sends the row to the running-maximum pass. Below it, with at most 2^18
// weights per row, O stays finite for any |v| < 2^46.
constexpr float kFixedRefLimit = 0x1p64f;
// Listed blocks staged in LDS at a time (longer lists are walked in segments).
constexpr int kListSeg = 256;

// LDS layouts of the 32-token tiles (16-byte chunks XOR-swizzled per row).
// K is read as MFMA A operands: 16 consecutive lanes take 16 consecutive rows at one
// logical chunk, so the swizzle spreads those rows over all 16 (d = 128) chunk slots;
// with d = 64 two rows share a 256-byte bank window, hence the (row >> 1) term.
// V is read with transposing reads: a 32-lane half takes 4 consecutive rows at 4
// consecutive chunks, so the swizzle moves each of the 4 rows to its own 4-chunk block.
template <int D>
__device__ __forceinline__ int k_swz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int D>
__device__ __forceinline__ int v_swz(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }

// Per-lane state of one attention row, shared by the tile steps.
template <int D>
struct AttnLane {
  static constexpr int KS = D / 16;           // MFMA k-steps over d (S^T)
  static constexpr int DT = D / 32;           // 32-wide d tiles (O^T)
  static constexpr int ROWB = D * 2;          // bytes per token row
  static constexpr int TILE = 32 * ROWB;      // bytes per 32-token K (or V) tile
  static constexpr int LOADS = TILE / (128 * 16);
  bf16x8 qf[KS];                              // Q^T fragments (query j, d 16s + 8g ..)
  f32x16 acc[DT];                             // O^T accumulators (query j)
  f32x4 lsum;                                 // row sum of query j (all four entries)
  bf16x8 sum_sel;                             // 0/1 selector operand of the row-sum MFMA
  float m;                                    // max in use (scaled log2 units)
  int k_off[KS];                              // K A-operand byte offsets in a tile
  int v_off[DT];                              // V^T transposing-read byte offsets (keys 0..3)
  int cp_koff[LOADS], cp_voff[LOADS];         // global -> LDS copy: tile byte offset of slot l
};

// K and V of one (b, h) are read through buffer resources: the tile's first byte goes in
// a scalar offset and each lane adds a fixed 32-bit offset, so the copies need no vector
// address arithmetic. Reads past the resource's size return zeros.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// Copies the 32-token K and V tiles starting at token tok0 from global memory straight
// into LDS. Each wave fills 1 KB pieces 2i + w of each tile; the lane writes its 16-byte
// slot and fetches the chunk that the tile's swizzle maps there. Rows past the tile's
// valid tokens are copied as they are (tokens of the next block, or zeros past the end of
// the buffer): their scores are masked, so they meet zero weights.
template <int D>
__device__ __forceinline__ void issue_tile(lds_u8* k_lds, lds_u8* v_lds, rsrc_t kr, rsrc_t vr, int tok0,
                                           const AttnLane<D>& s, int w) {
  const int base = __builtin_amdgcn_readfirstlane(tok0 * AttnLane<D>::ROWB);
#pragma unroll
  for (int i = 0; i < AttnLane<D>::LOADS; ++i) {
    const int piece = (i * 2 + w) * 1024;     // wave-uniform LDS offset
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(k_lds + piece), 16, s.cp_koff[i], base, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(v_lds + piece), 16, s.cp_voff[i], base, 0, 0);
  }
}

// One 32-token tile of one wave: S^T = K Q^T, softmax weights, O^T += V^T P^T. With
// `track`, the tile's maximum updates the reference (and rescales O and the row sum when
// it grows past the slack); without, the weights use the reference as it stands.
template <int D>
__device__ __forceinline__ void tile_compute(const lds_u8* Kt, const lds_u8* Vt, int nv, int g, float c,
                                             AttnLane<D>& s, bool track) {
  constexpr int KS = AttnLane<D>::KS, DT = AttnLane<D>::DT, ROWB = AttnLane<D>::ROWB;
  typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
  f32x16 sacc;
#pragma unroll
  for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
  // wave priority is raised while this wave issues matrix-core work, so a SIMD's other
  // wave, busy with its softmax, yields issue slots to it and the matrix core stays fed
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    const bf16x8 kf = *reinterpret_cast<lds_bf16x8*>(Kt + s.k_off[st]);
    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, s.qf[st], sacc, 0, 0, 0);
  }
  __builtin_amdgcn_s_setprio(0);
  // V^T fragments, in flight while the softmax runs; rows 16ks + 8h of the lane's column
  bf16x8 vf[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint2 lo = ds_read_tr16(Vt + s.v_off[dt] + 16 * ks * ROWB);
      const uint2 hi = ds_read_tr16(Vt + s.v_off[dt] + (16 * ks + 8) * ROWB);
      const u32x4 wv = {lo.x, lo.y, hi.x, hi.y};
      vf[dt][ks] = __builtin_bit_cast(bf16x8, wv);
    }
  // sacc[v] = S^T[key 8(v/4) + 4g + v%4][query j]. Short tiles (rare) mask their tail
  // keys; the empty asm keeps the compiler from turning the branch into selects that
  // would run on every tile.
  if (nv < 32) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (8 * (v / 4) + 4 * g + (v % 4) >= nv) sacc[v] = -INFINITY;
  }
  if (track) {
    // scale > 0, so the max of the raw scores gives the max of the scaled ones; lanes j
    // and j + 32 hold the two key halves of query j
    float mt = sacc[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mt = fmaxf(mt, sacc[v]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
    mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
    const bool grow = mt > s.m + kRescaleSlack;
    if (__any(grow)) {
      const float mn = grow ? mt : s.m;
      const float corr = fast_exp2(s.m - mn);
      s.m = mn;
#pragma unroll
      for (int v = 0; v < 4; ++v) s.lsum[v] *= corr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) s.acc[dt][v] *= corr;
    }
  }
  // P^T as bf16 pairs; B slot t of pb[ks] is key 16ks + 8(t/4) + 4g + t%4
  uint32_t pw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    bf16x2 pr;
    pr[0] = static_cast<__bf16>(fast_exp2(fmaf(sacc[2 * i], c, -s.m)));
    pr[1] = static_cast<__bf16>(fast_exp2(fmaf(sacc[2 * i + 1], c, -s.m)));
    pw[i] = __builtin_bit_cast(uint32_t, pr);
  }
  const u32x4 plo = {pw[0], pw[1], pw[2], pw[3]}, phi = {pw[4], pw[5], pw[6], pw[7]};
  const bf16x8 pb[2] = {__builtin_bit_cast(bf16x8, plo), __builtin_bit_cast(bf16x8, phi)};
  __builtin_amdgcn_s_setprio(1);
  // O^T += V^T P^T; the two transposing reads give this lane's d the same keys
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      s.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt][ks], pb[ks], s.acc[dt], 0, 0, 0);
  // Row sums on the matrix cores, from the same rounded weights the PV product uses (so
  // the normalised weights sum to one). Read as a 16x16x32 product, the B operand pb holds
  // in lane l column l%16 with the 8 keys of lane group l/16; groups 0 and 2 belong to
  // query l%16, groups 1 and 3 to query 16 + l%16. The selector has ones in rows
  // {0-3, 8-11} for groups {0, 2} and in rows {4-7, 12-15} for groups {1, 3}, so the rows
  // lane l receives (4(l/16) .. +3 of column l%16) all hold the sum of query l%32.
  s.lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s.sum_sel, pb[0], s.lsum, 0, 0, 0);
  s.lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s.sum_sel, pb[1], s.lsum, 0, 0, 0);
  __builtin_amdgcn_s_setprio(0);
}

template <int D>
__global__ void __launch_bounds__(128, 2) attn_bf16_kernel(AttnArgs a) {
  using L = AttnLane<D>;
  constexpr int KS = L::KS, DT = L::DT, ROWB = L::ROWB, TILE = L::TILE, LOADS = L::LOADS;
  // Double-buffered K and V tiles as four separate LDS objects, so the compiler can tell
  // that reading one buffer does not alias the in-flight copy into the other.
  __shared__ __attribute__((aligned(1024))) unsigned char k_buf0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v_buf0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char k_buf1[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v_buf1[TILE];
  __shared__ int2 tile_s[2 * kListSeg];       // (first token, valid tokens) per 32-token tile
  lds_u8* const kb0 = (lds_u8*)k_buf0;
  lds_u8* const vb0 = (lds_u8*)v_buf0;
  lds_u8* const kb1 = (lds_u8*)k_buf1;
  lds_u8* const vb1 = (lds_u8*)v_buf1;

  // head-major work order, consecutive work items on one XCD (workgroups are dealt
  // round-robin over the 8 XCDs)
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per = nwg / 8, rem = nwg % 8;
  const int work = xcd * per + min(xcd, rem) + slot;
  const int bh = work / a.n_qb, r = work - bh * a.n_qb;

  const int tid = threadIdx.x, l = tid % 64, j = l % 32, g = l / 32;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const BlockGeom geo{a.tpf, a.bs, a.n_bpf};
  const int q_start = geo.start(r), q_len = geo.len(r);
  const int nq = min(max(q_len - 32 * w, 0), 32);

  const __bf16* Qg = static_cast<const __bf16*>(a.q) + static_cast<size_t>(bh) * a.q_stride * D;
  const uint32_t kv_bytes = static_cast<uint32_t>(a.lk) * ROWB;
  const rsrc_t kr = make_rsrc(static_cast<const __bf16*>(a.k) + static_cast<size_t>(bh) * a.kv_stride * D, kv_bytes);
  const rsrc_t vr = make_rsrc(static_cast<const __bf16*>(a.v) + static_cast<size_t>(bh) * a.kv_stride * D, kv_bytes);

  L s;
  {
    const int qrow = q_start + min(32 * w + j, q_len - 1);
    const __bf16* qp = Qg + static_cast<size_t>(qrow) * D + 8 * g;
#pragma unroll
    for (int st = 0; st < KS; ++st) s.qf[st] = *reinterpret_cast<const bf16x8*>(qp + 16 * st);
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) s.acc[dt][v] = 0.f;
  s.m = -1e30f;
#pragma unroll
  for (int v = 0; v < 4; ++v) s.lsum[v] = 0.f;
  {
    const bool rows_a = ((l % 16) & 4) == 0;            // selector rows 0-3 and 8-11
    const bool grp_a = ((l / 16) & 1) == 0;             // key groups 0 and 2
    const __bf16 one = static_cast<__bf16>(rows_a == grp_a ? 1.0f : 0.0f);
#pragma unroll
    for (int t = 0; t < 8; ++t) s.sum_sel[t] = one;
  }
  const float c = a.scale_log2;
#pragma unroll
  for (int st = 0; st < KS; ++st) s.k_off[st] = j * ROWB + (((2 * st + g) ^ k_swz<D>(j)) * 16);
  // V^T A-operand via transposing reads: this lane supplies row 16ks + 8h + 4g + (l%16)/4,
  // columns 32dt + 16((l/16)%2) + 4(l%4) .. +3. The swizzle depends only on the row's low
  // bits, which 16ks + 8h leaves alone, so one offset per dt serves all four reads.
  const int grp = l / 16, i16 = l % 16;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int key = 4 * g + i16 / 4;
    const int d = 32 * dt + 16 * (grp % 2) + 4 * (i16 % 4);
    s.v_off[dt] = key * ROWB + (((d / 8) ^ v_swz<D>(key)) * 16) + (d % 8) * 2;
  }
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int off = (i * 2 + w) * 1024 + l * 16;
    const int row = off / ROWB, pc = (off % ROWB) / 16;   // physical chunk
    s.cp_koff[i] = row * ROWB + (pc ^ k_swz<D>(row)) * 16;
    s.cp_voff[i] = row * ROWB + (pc ^ v_swz<D>(row)) * 16;
  }

  auto tile = [&](int t) {                    // wave-uniform (first token, valid tokens)
    const int2 v = tile_s[t];
    return make_int2(__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y));
  };

  const int* bl = a.blocks + static_cast<size_t>(work) * a.W_b;
  __shared__ int redo_s[2];
  // pass 0: reference fixed by the first tile; pass 1 (only if a query's row sum left the
  // safe range): the row again with the running maximum. Unrolled, so each pass's tile
  // loop is compiled with its own (constant) choice.
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      const bool bad = j < nq && !(s.lsum[0] < kFixedRefLimit);
      if (l == 0) redo_s[w] = __any(bad) ? 1 : 0;
      __syncthreads();
      const bool redo = (redo_s[0] | redo_s[1]) != 0;
      __syncthreads();
      if (!redo) break;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) s.acc[dt][v] = 0.f;
      s.m = -1e30f;
#pragma unroll
      for (int v = 0; v < 4; ++v) s.lsum[v] = 0.f;
    }
    for (int seg0 = 0; seg0 < a.W_b; seg0 += kListSeg) {
      const int nseg = min(kListSeg, a.W_b - seg0);
      const int nt = 2 * nseg;
      __syncthreads();                          // previous segment fully consumed
      for (int i = tid; i < nseg; i += 128) {
        const int gg = bl[seg0 + i];
        int2 t0 = make_int2(0, 0), t1 = make_int2(0, 0);
        if (gg >= 0 && gg < a.n_kb) {
          const int st = geo.start(gg), len = geo.len(gg);
          t0 = make_int2(st, min(32, len));
          if (len > 32) t1 = make_int2(st + 32, len - 32);
        }
        tile_s[2 * i] = t0;
        tile_s[2 * i + 1] = t1;
      }
      __syncthreads();

      // next non-empty tile from index i on (nt if none) and its table entry; entries are
      // read before the barriers that precede their use
      auto next = [&](int i, int2& e) {
        e = make_int2(0, 0);
        for (; i < nt; ++i) {
          e = tile(i);
          if (e.y != 0) break;
        }
        return i;
      };
      int2 cur;
      int t = next(0, cur);
      if (t >= nt) continue;
      issue_tile<D>(kb0, vb0, kr, vr, cur.x, s, w);
      // the segment's first tile (buffer 0) always updates the reference; the loop after it
      // handles two tiles per iteration (buffers 1, 0) so each LDS buffer index is a
      // compile-time constant, and tracks the maximum only in the redo pass
      {
        int2 nx;
        const int t2 = next(t + 1, nx);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t2 < nt) issue_tile<D>(kb1, vb1, kr, vr, nx.x, s, w);
        if (nq > 0) tile_compute<D>(kb0, vb0, cur.y, g, c, s, true);
        t = t2;
        cur = nx;
      }
      while (t < nt) {
        int2 nx;
        int t2 = next(t + 1, nx);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t2 < nt) issue_tile<D>(kb0, vb0, kr, vr, nx.x, s, w);
        if (nq > 0) tile_compute<D>(kb1, vb1, cur.y, g, c, s, pass == 1);
        t = t2;
        cur = nx;
        if (t >= nt) break;

        t2 = next(t + 1, nx);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t2 < nt) issue_tile<D>(kb1, vb1, kr, vr, nx.x, s, w);
        if (nq > 0) tile_compute<D>(kb0, vb0, cur.y, g, c, s, pass == 1);
        t = t2;
        cur = nx;
      }
    }
  }

  const float lt = s.lsum[0];                 // both key halves already summed
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (j < nq) {
    __bf16* op = static_cast<__bf16*>(a.o) + (static_cast<size_t>(bh) * a.q_stride + q_start + 32 * w + j) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = static_cast<__bf16>(s.acc[dt][4 * v4 + e] * inv);
        *reinterpret_cast<bf16x4*>(op + 32 * dt + 8 * v4 + 4 * g) = ov;
      }
    }
  }
}

hipError_t launch_attn_f32(const AttnArgs& a, int d, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.BH) * a.n_qb), block(128);
  if (d == 128)
    hipLaunchKernelGGL((attn_f32_kernel<128>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_f32_kernel<64>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnArgs& a, int d, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.BH) * a.n_qb), block(128);
  if (d == 128)
    hipLaunchKernelGGL((attn_bf16_kernel<128>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<64>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace lf
