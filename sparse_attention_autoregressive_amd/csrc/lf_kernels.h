// Kernel launchers behind the C ABI (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lf {

constexpr int kListFrames = 256;   // key frames whose id lists travel in the kernel arguments
constexpr int kMaxFrames = 4096;   // key frames a frame-selecting call may address

// Frame ids of the memory set M and of the always-kept frames, passed by value (calls
// with at most kListFrames key frames).
struct FrameLists {
  int16_t mem[kListFrames];
  int16_t forced[kListFrames];
};

// The same two sets as bit masks (frame f is bit f % 64 of word f / 64), for any call.
struct FrameMasks {
  uint64_t mem[kMaxFrames / 64];
  uint64_t forced[kMaxFrames / 64];
};

// x_stride: tokens between consecutive (b, h) slices of x; out_stride: frames between
// consecutive (b, h) slices of the outputs.
hipError_t launch_pool(const void* x, bool bf16, int d, int BH, int n_frames, int tpf, int bs,
                       int n_bpf, long long x_stride, int out_stride, float* blk, float* frm, hipStream_t st);

// Queries (block means) and keys (block and frame means) in one launch; q_stride and
// k_stride: tokens between consecutive (b, h) slices of q and k; k_out_stride: frames
// between (b, h) slices of the pooled keys (q_blk is packed).
hipError_t launch_pool_qk(const void* q, const void* k, bool bf16, int d, int BH, int n_qframes, int n_kframes,
                          int tpf, int bs, int n_bpf, long long q_stride, long long k_stride, int k_out_stride,
                          float* q_blk, float* k_blk, float* k_frm, hipStream_t st);

// One launch of the selection kernel over n_rows = B*H*n_qb rows. Frame stage: reads
// q_blk, k_frm, lists, n_mem, n_forced, k_eff and writes frames_out (if set). Block
// stage: reads q_blk, k_blk and the frame lists (from the frame stage, else frames_in)
// and writes blocks_out.
// Query/key prologue (RMSNorm + rotary embedding) fused with block (and frame) pooling.
constexpr int kMaxPairs = 64;   // rotary pairs of the largest head dimension (d = 128)
struct ProlArgs {
  const void* x;
  void* y;
  const float* gamma;   // [d]
  float* blk;           // block means of y, (b, h) slices out_stride frames apart
  float* frm;           // frame means, or nullptr
  long long x_stride;   // tokens between (b, h) slices of x
  long long y_stride;   // tokens between (b, h) slices of y
  int BH, n_frames, frame0, out_stride, tpf, bs, n_bpf, lat_w;
  float eps;
  float rev[kMaxPairs];   // per rotary pair: theta^(-i/n) / (2 pi), revolutions per unit of position
};
hipError_t launch_prologue(const ProlArgs& a, bool bf16, int d, hipStream_t st);

// The keys' half of a steady-state prologue step (ProlArgs describes the queries; both
// share frames, positions and geometry) and the lagged frame means of a pooled-key cache.
struct ProlStepArgs {
  const void* k;          // the chunk's new keys, (b, h) slices ProlArgs::x_stride tokens apart
  void* k_out;            // where they go (a KV cache view), slices k_out_stride tokens apart
  const float* gamma_k;   // [d]
  float* k_blk;           // pooled-key cache, frame 0 (slices cache_stride frames apart)
  float* k_frm;
  long long k_out_stride;
  int cache_stride, f_new, f_lag, n_lag;
};
hipError_t launch_prologue_step(const ProlArgs& a, const ProlStepArgs& s, bool bf16, int d, hipStream_t st);

// Pooling of one steady-state step: query block means, the new key frames' block means
// into a pooled-key cache at frame f_new, and the frame means of cache frames
// [f_lag, f_lag + n_lag) from block means an earlier launch wrote, in one launch.
struct PoolStepArgs {
  const void* q;
  const void* k;
  float* q_blk;
  float* k_blk;           // cache, frame 0
  float* k_frm;
  long long q_stride, k_stride;
  int BH, n_qframes, n_new, f_new, f_lag, n_lag, cache_stride, tpf, bs, n_bpf;
};
hipError_t launch_pool_step(const PoolStepArgs& a, bool bf16, int d, hipStream_t st);

struct SelectArgs {
  const float* q_blk;
  const float* k_frm;
  const float* k_blk;
  const int* frames_in;
  int* frames_out;
  int* blocks_out;
  int n_qb, n_kframes, n_bpf;
  int kf_stride;        // frames between (b, h) slices of k_frm and k_blk
  int n_mem, n_forced, k_eff, W_f, kb_eff;
  FrameLists lists;     // filled when n_kframes <= kListFrames
  FrameMasks masks;     // always filled by a frame-selecting call
};

hipError_t launch_select(const SelectArgs& a, int d, int n_rows, bool frames, bool blocks, hipStream_t st);

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

// Single-level block top-k over all n_kb key blocks of a row's prefix.
constexpr int kMax1DBlocks = 4096;
struct Select1DArgs {
  const float* q_blk;   // [rows, D]
  const float* k_blk;   // (b, h) slices kb_stride blocks apart
  int* blocks_out;      // [rows, K]
  int n_qb, n_kb, kb_stride, K;
};
hipError_t launch_select_1d(const Select1DArgs& a, int d, int n_rows, hipStream_t st);

// Dense bf16 MFMA loop of n_wg 4-wave workgroups (measurement aid).
hipError_t launch_mfma_probe(int n_wg, int iters, float* sink, long long* clocks, hipStream_t st);
// Streaming read of `bytes` (a multiple of 16) by n_wg 256-thread workgroups (measurement aid).
hipError_t launch_hbm_read(const void* x, long long bytes, int n_wg, float* sink, hipStream_t st);

}  // namespace lf
