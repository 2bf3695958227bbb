// Kernel launchers behind the C ABI (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lf {

// Memory set and always-kept frames as bit masks over frame ids < 256.
struct FrameSets {
  uint64_t mem[4];
  uint64_t forced[4];
};

// x_stride: tokens between consecutive (b, h) slices of x.
hipError_t launch_pool(const void* x, bool bf16, int d, int BH, int n_frames, int tpf, int bs,
                       int n_bpf, long long x_stride, float* blk, float* frm, hipStream_t st);

hipError_t launch_select_frames(const float* q_blk, const float* k_frm, int d, int BH, int n_qb,
                                int n_kframes, const FrameSets& sets, int n_mem, int k_eff,
                                int W_f, int* out, hipStream_t st);

hipError_t launch_select_blocks(const float* q_blk, const float* k_blk, const int* frames, int d,
                                int BH, int n_qb, int n_kframes, int n_bpf, int W_f, int kb_eff,
                                int* out, hipStream_t st);

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const int* blocks;
  int BH, n_qb, n_kb, W_b;
  int tpf, bs, n_bpf;
  int lq, lk;           // query / key tokens per (b, h)
  long long q_stride;   // tokens between (b, h) slices of q and o
  long long kv_stride;  // tokens between (b, h) slices of k and v
  float scale_log2;     // softmax scale * log2(e)
};

hipError_t launch_attn_f32(const AttnArgs& a, int d, hipStream_t st);
hipError_t launch_attn_bf16(const AttnArgs& a, int d, hipStream_t st);

}  // namespace lf
