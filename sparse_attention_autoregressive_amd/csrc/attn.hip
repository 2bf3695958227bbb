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
//   The online softmax runs in base 2 with scale*log2(e) folded into the logits; the
//   running max is shared by the two lanes of a query (one xor-32 shuffle per tile) and
//   the row sum stays per lane until the end.
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
                   (static_cast<size_t>(bh) * a.lq + q_start + min(t, q_len - 1)) * D;
  float q[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) { q[c] = Q[c]; o[c] = 0.f; }
  float m = -1e30f, lsum = 0.f;

  const float* K = static_cast<const float*>(a.k) + static_cast<size_t>(bh) * a.lk * D;
  const float* V = static_cast<const float*>(a.v) + static_cast<size_t>(bh) * a.lk * D;
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
    float* O = static_cast<float*>(a.o) + (static_cast<size_t>(bh) * a.lq + q_start + t) * D;
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

template <int D>
__global__ void __launch_bounds__(128, 2) attn_bf16_kernel(AttnArgs a) {
  constexpr int KS = D / 16;                  // MFMA k-steps over d (S^T)
  constexpr int DT = D / 32;                  // 32-wide d tiles (O^T)
  constexpr int CH = D / 8;                   // 16-byte chunks per token row
  constexpr int ROWB = D * 2;                 // bytes per token row
  constexpr int TILE = 32 * ROWB;             // bytes per 32-token K (or V) tile
  constexpr int LOADS = TILE / (128 * 16);    // 16-byte loads per thread per operand
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2][2][TILE];

  // head-major work order, consecutive work items on one XCD (workgroups are dealt
  // round-robin over the 8 XCDs)
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per = nwg / 8, rem = nwg % 8;
  const int work = xcd * per + min(xcd, rem) + slot;
  const int bh = work / a.n_qb, r = work - bh * a.n_qb;

  const int tid = threadIdx.x, w = tid / 64, l = tid % 64, j = l % 32, g = l / 32;
  const BlockGeom geo{a.tpf, a.bs, a.n_bpf};
  const int q_start = geo.start(r), q_len = geo.len(r);
  const int nq = min(max(q_len - 32 * w, 0), 32);

  const __bf16* Qg = static_cast<const __bf16*>(a.q) + static_cast<size_t>(bh) * a.lq * D;
  const __bf16* Kg = static_cast<const __bf16*>(a.k) + static_cast<size_t>(bh) * a.lk * D;
  const __bf16* Vg = static_cast<const __bf16*>(a.v) + static_cast<size_t>(bh) * a.lk * D;

  // Q^T fragments: lane (query j, half g) holds d = 16s + 8g .. +7 of its row
  bf16x8 qf[KS];
  {
    const int qrow = q_start + min(32 * w + j, q_len - 1);
    const __bf16* qp = Qg + static_cast<size_t>(qrow) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  }

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[dt][v] = 0.f;
  float m = -1e30f, lsum = 0.f;   // max in use (scaled log2 units) and partial row sum
  const float c = a.scale_log2;

  // per-lane byte offsets inside a tile, independent of the tile
  int k_off[KS];                              // K A-operand: row j, chunk 2s+g (swizzled)
#pragma unroll
  for (int s = 0; s < KS; ++s) k_off[s] = j * ROWB + (((2 * s + g) ^ (j & (CH - 1))) * 16);
  // V^T A-operand via transposing reads: this lane supplies row 16ks + 8h + 4g + (l%16)/4,
  // columns 32dt + 16((l/16)%2) + 4(l%4) .. +3
  const int grp = l / 16, i16 = l % 16;
  int v_off[DT][2][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = 16 * ks + 8 * h + 4 * g + i16 / 4;
        const int d = 32 * dt + 16 * (grp % 2) + 4 * (i16 % 4);
        v_off[dt][ks][h] = key * ROWB + (((d / 8) ^ (key & (CH - 1))) * 16) + (d % 8) * 2;
      }

  const int* bl = a.blocks + static_cast<size_t>(work) * a.W_b;
  auto ok = [&](int e) {
    const int gg = bl[e];
    return gg >= 0 && gg < a.n_kb;
  };

  auto issue = [&](int buf, int tok0, int nv) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int base = (i * 2 + w) * 1024;    // wave-uniform LDS offset
      const int off = base + l * 16;
      const int row = off / ROWB;
      const int cc = ((off % ROWB) / 16) ^ (row & (CH - 1));
      const size_t src = static_cast<size_t>(tok0 + min(row, nv - 1)) * D + cc * 8;
      __builtin_amdgcn_global_load_lds(Kg + src, (__attribute__((address_space(3))) void*)(&smem[buf][0][base]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(Vg + src, (__attribute__((address_space(3))) void*)(&smem[buf][1][base]), 16, 0, 0);
    }
  };

  int n = 0, p = 0;
  while (n < a.W_b && !ok(n)) ++n;
  if (n < a.W_b) {
    const int g0 = bl[n];
    issue(0, geo.start(g0), min(32, geo.len(g0)));
  }
  int buf = 0;
  while (n < a.W_b) {
    const int gc = bl[n];
    const int kl = geo.len(gc);
    const int nv = min(32, kl - 32 * p);
    int n2 = n, p2 = p + 1;
    if (32 * p2 >= kl) {
      p2 = 0;
      ++n2;
      while (n2 < a.W_b && !ok(n2)) ++n2;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (n2 < a.W_b) {
      const int gn = bl[n2];
      issue(buf ^ 1, geo.start(gn) + 32 * p2, min(32, geo.len(gn) - 32 * p2));
    }

    if (nq > 0) {
      const lds_u8* Kt = (const lds_u8*)(&smem[buf][0][0]);
      const lds_u8* Vt = (const lds_u8*)(&smem[buf][1][0]);
      f32x16 sacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>((const unsigned char*)(Kt + k_off[s]));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc, 0, 0, 0);
      }
      // sacc[v] = S^T[key 8(v/4) + 4g + v%4][query j]; scale > 0, so the max of the raw
      // scores gives the max of the scaled ones
      if (nv < 32) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (8 * (v / 4) + 4 * g + (v % 4) >= nv) sacc[v] = -INFINITY;
      }
      float mt = sacc[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mt = fmaxf(mt, sacc[v]);
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * c;
      const bool grow = mt > m + kRescaleSlack;
      if (__any(grow)) {
        const float mn = grow ? mt : m;
        const float corr = fast_exp2(m - mn);
        m = mn;
        lsum *= corr;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[dt][v] *= corr;
      }
      // P^T as bf16 pairs; the row sum takes the same rounded weights the matrix cores
      // multiply, so the normalised weights sum to one (exact for a single dominant key)
      uint32_t pw[8];
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        bf16x2 pr;
        pr[0] = static_cast<__bf16>(fast_exp2(fmaf(sacc[2 * i], c, -m)));
        pr[1] = static_cast<__bf16>(fast_exp2(fmaf(sacc[2 * i + 1], c, -m)));
        pw[i] = __builtin_bit_cast(uint32_t, pr);
        ps0 += __uint_as_float(pw[i] << 16);
        ps1 += __uint_as_float(pw[i] & 0xFFFF0000u);
      }
      lsum += ps0 + ps1;
      bf16x8 pb[2];
      {
        const u32x4 lo = {pw[0], pw[1], pw[2], pw[3]}, hi = {pw[4], pw[5], pw[6], pw[7]};
        pb[0] = __builtin_bit_cast(bf16x8, lo);
        pb[1] = __builtin_bit_cast(bf16x8, hi);
      }
      // O^T += V^T P^T; B slot t of pb[ks] is key 16ks + 8(t/4) + 4g + t%4, and the two
      // transposing reads give this lane's d the same keys
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint2 lo = ds_read_tr16(Vt + v_off[dt][ks][0]);
          const uint2 hi = ds_read_tr16(Vt + v_off[dt][ks][1]);
          const uint32_t wv[4] = {lo.x, lo.y, hi.x, hi.y};
          const bf16x8 va = __builtin_bit_cast(bf16x8, wv);
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks], acc[dt], 0, 0, 0);
        }
      }
    }
    buf ^= 1;
    n = n2;
    p = p2;
  }

  const float lt = lsum + __shfl_xor(lsum, 32, 64);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (j < nq) {
    __bf16* op = static_cast<__bf16*>(a.o) + (static_cast<size_t>(bh) * a.lq + q_start + 32 * w + j) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = static_cast<__bf16>(acc[dt][4 * v4 + e] * inv);
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
