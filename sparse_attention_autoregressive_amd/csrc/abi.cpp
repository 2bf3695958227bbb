// C ABI of the HSA library: argument validation on the host, the Chunk-Aware Growth
// schedule (host math), and kernel launches on the caller's stream.
// Every check happens before anything is enqueued; a failing call stores a message in
// a thread-local buffer and returns a status. No exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/lf.h"
#include "../../include/lf_probe.h"
#include "lf_kernels.h"

namespace {

thread_local char t_err[512] = "";

lf_status fail(lf_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(t_err, sizeof(t_err), fmt, ap);
  va_end(ap);
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int n_bpf_of(const lf_geom& g) { return (g.tokens_per_frame + g.block_size - 1) / g.block_size; }

// Geometry checks shared by the device calls (d must be 64 or 128).
lf_status check_geom(const lf_geom& g, const char* fn) {
  if (g.B < 1 || g.H < 1) return fail(LF_ERR_INVALID_ARG, "%s: B and H must be >= 1", fn);
  if (g.tokens_per_frame < 1 || g.tokens_per_frame > 65536)
    return fail(LF_ERR_INVALID_ARG, "%s: tokens_per_frame must be in [1, 65536]", fn);
  if (g.block_size < 1 || g.block_size > g.tokens_per_frame)
    return fail(LF_ERR_INVALID_ARG, "%s: block_size must be in [1, tokens_per_frame]", fn);
  if (g.d < 1) return fail(LF_ERR_INVALID_ARG, "%s: d must be >= 1", fn);
  if (g.head_stride < 0 || g.kv_head_stride < 0)
    return fail(LF_ERR_INVALID_ARG, "%s: head_stride and kv_head_stride must be >= 0", fn);
  if (g.frame_stride < 0) return fail(LF_ERR_INVALID_ARG, "%s: frame_stride must be >= 0", fn);
  if (g.d != 64 && g.d != 128) return fail(LF_ERR_UNSUPPORTED, "%s: d=%d unsupported (64 or 128)", fn, g.d);
  return LF_OK;
}

bool fits_int(long long v) { return v >= 0 && v <= 0x7fffffffLL; }

// Frames between (b, h) slices of the pooled key tensors: g.frame_stride, or the call's
// key-frame count when it is 0. Fails when a nonzero stride is below that count.
lf_status pooled_stride(const lf_geom& g, int32_t n_kframes, int* out, const char* fn) {
  if (g.frame_stride != 0 && g.frame_stride < n_kframes)
    return fail(LF_ERR_INVALID_ARG, "%s: frame_stride %d < key-frame count %d", fn, g.frame_stride, n_kframes);
  *out = g.frame_stride ? g.frame_stride : n_kframes;
  return LF_OK;
}

// Clears an error left by earlier, unrelated HIP work so it is not reported as ours.
void pending_error() { (void)hipGetLastError(); }

lf_status hip_status(hipError_t e, const char* fn) {
  if (e == hipSuccess) return LF_OK;
  return fail(LF_ERR_HIP, "%s: HIP error %d (%s)", fn, static_cast<int>(e), hipGetErrorString(e));
}

// Checks of the frame stage shared by lf_select_frames and lf_select; fills the id lists.
lf_status check_frame_stage(const float* q_blk, const float* k_frm, lf_geom g, int32_t n_qb,
                            int32_t n_kframes, const int32_t* mem, int32_t n_mem,
                            const int32_t* forced, int32_t n_forced, int32_t k_f,
                            lf::SelectArgs& a, const char* fn) {
  if (lf_status st = check_geom(g, fn)) return st;
  if (n_qb < 1 || n_kframes < 1) return fail(LF_ERR_INVALID_ARG, "%s: n_qb and n_kframes must be >= 1", fn);
  if (n_kframes > lf::kMaxFrames)
    return fail(LF_ERR_UNSUPPORTED, "%s: n_kframes=%d > %d", fn, n_kframes, lf::kMaxFrames);
  if (n_mem < 0 || n_forced < 0 || k_f < 0) return fail(LF_ERR_INVALID_ARG, "%s: negative count", fn);
  if ((n_mem > 0 && !mem) || (n_forced > 0 && !forced))
    return fail(LF_ERR_INVALID_ARG, "%s: NULL frame-id array", fn);
  if (!q_blk || !k_frm) return fail(LF_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(q_blk) || !aligned16(k_frm)) return fail(LF_ERR_INVALID_ARG, "%s: misaligned buffer", fn);
  bool seen[lf::kMaxFrames] = {};
  bool in_mem[lf::kMaxFrames] = {};
  std::memset(&a.masks, 0, sizeof(a.masks));
  const bool listed = n_kframes <= lf::kListFrames;
  for (int i = 0; i < n_mem; ++i) {
    const int f = mem[i];
    if (f < 0 || f >= n_kframes) return fail(LF_ERR_INVALID_ARG, "%s: mem[%d]=%d out of range", fn, i, f);
    if (seen[f]) return fail(LF_ERR_INVALID_ARG, "%s: duplicate memory frame %d", fn, f);
    seen[f] = in_mem[f] = true;
    if (listed) a.lists.mem[i] = static_cast<int16_t>(f);
    a.masks.mem[f / 64] |= 1ull << (f % 64);
  }
  for (int i = 0; i < n_forced; ++i) {
    const int f = forced[i];
    if (f < 0 || f >= n_kframes) return fail(LF_ERR_INVALID_ARG, "%s: forced[%d]=%d out of range", fn, i, f);
    if (in_mem[f]) return fail(LF_ERR_INVALID_ARG, "%s: frame %d is both forced and in the memory set", fn, f);
    if (seen[f]) return fail(LF_ERR_INVALID_ARG, "%s: duplicate forced frame %d", fn, f);
    seen[f] = true;
    if (listed) a.lists.forced[i] = static_cast<int16_t>(f);
    a.masks.forced[f / 64] |= 1ull << (f % 64);
  }
  if (lf_status st = pooled_stride(g, n_kframes, &a.kf_stride, fn)) return st;
  if (!fits_int(static_cast<long long>(g.B) * g.H * a.kf_stride * g.d))
    return fail(LF_ERR_INVALID_ARG, "%s: problem too large", fn);
  a.k_eff = k_f < n_mem ? k_f : n_mem;
  a.W_f = n_forced + a.k_eff;
  if (a.W_f < 1) return fail(LF_ERR_INVALID_ARG, "%s: empty frame set (W_f = 0)", fn);
  if (!fits_int(static_cast<long long>(g.B) * g.H * n_qb))
    return fail(LF_ERR_INVALID_ARG, "%s: problem too large", fn);
  a.q_blk = q_blk;
  a.k_frm = k_frm;
  a.n_qb = n_qb;
  a.n_kframes = n_kframes;
  a.n_mem = n_mem;
  a.n_forced = n_forced;
  return LF_OK;
}

// Checks of the block stage shared by lf_select_blocks and lf_select.
lf_status check_block_stage(const float* k_blk, lf_geom g, int32_t n_qb, int32_t n_kframes, int32_t W_f,
                            int32_t k_b, int32_t* blocks_out, lf::SelectArgs& a, const char* fn) {
  if (n_qb < 1 || n_kframes < 1 || W_f < 1 || k_b < 1)
    return fail(LF_ERR_INVALID_ARG, "%s: n_qb, n_kframes, W_f and k_b must be >= 1", fn);
  if (n_kframes > 65535) return fail(LF_ERR_UNSUPPORTED, "%s: n_kframes=%d > 65535", fn, n_kframes);
  const int n_bpf = n_bpf_of(g);
  if (n_bpf > 64) return fail(LF_ERR_UNSUPPORTED, "%s: %d blocks per frame > 64", fn, n_bpf);
  if (!k_blk || !blocks_out) return fail(LF_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(k_blk) || (reinterpret_cast<uintptr_t>(blocks_out) & 3u))
    return fail(LF_ERR_INVALID_ARG, "%s: misaligned buffer", fn);
  if (lf_status st = pooled_stride(g, n_kframes, &a.kf_stride, fn)) return st;
  a.kb_eff = k_b < n_bpf ? k_b : n_bpf;
  if (!fits_int(static_cast<long long>(g.B) * g.H * n_qb) || !fits_int(static_cast<long long>(W_f) * a.kb_eff) ||
      !fits_int(static_cast<long long>(g.B) * g.H * a.kf_stride * n_bpf))
    return fail(LF_ERR_INVALID_ARG, "%s: problem too large", fn);
  a.k_blk = k_blk;
  a.blocks_out = blocks_out;
  a.n_bpf = n_bpf;
  a.n_qb = n_qb;
  a.n_kframes = n_kframes;
  a.W_f = W_f;
  return LF_OK;
}

// Checks shared by the steady-state step calls: the cache geometry and the two frame
// ranges (new frames and lagged frames), both inside the cache and disjoint.
lf_status check_step_frames(const lf_geom& g, int32_t n_new, int32_t f_new, int32_t f_lag, int32_t n_lag, int* stride,
                            const char* fn) {
  if (n_new < 0 || f_new < 0 || f_lag < 0 || n_lag < 0)
    return fail(LF_ERR_INVALID_ARG, "%s: negative frame index or count", fn);
  if (g.frame_stride < 1) return fail(LF_ERR_INVALID_ARG, "%s: frame_stride must give the cache's frame count", fn);
  if (static_cast<long long>(f_new) + n_new > g.frame_stride || static_cast<long long>(f_lag) + n_lag > g.frame_stride)
    return fail(LF_ERR_INVALID_ARG, "%s: frames beyond the cache's %d frames", fn, g.frame_stride);
  if (n_new > 0 && n_lag > 0 && f_lag < f_new + n_new && f_new < f_lag + n_lag)
    return fail(LF_ERR_INVALID_ARG, "%s: lagged frames [%d, %d) overlap the new frames [%d, %d)", fn, f_lag,
                f_lag + n_lag, f_new, f_new + n_new);
  *stride = g.frame_stride;
  return LF_OK;
}

// The rotary turn (revolutions per unit of position) of each pair: pair k turns with the
// token's frame for the first d/2 - 2*floor(d/6) pairs, then its row, then its column;
// pair i of an axis with n pairs turns theta^(-i/n) radians per unit.
void rotary_turns(int d, float theta, float* rev) {
  const int n_hw = d / 6, n_t = d / 2 - 2 * n_hw;
  for (int k = 0; k < d / 2; ++k) {
    const int i = k < n_t ? k : (k < n_t + n_hw ? k - n_t : k - n_t - n_hw);
    const int n = k < n_t ? n_t : n_hw;
    rev[k] = static_cast<float>(std::pow(static_cast<double>(theta), -static_cast<double>(i) / n) /
                                (2.0 * 3.14159265358979323846));
  }
}

}  // namespace

extern "C" {

const char* lf_last_error(void) { return t_err; }

int32_t lf_abi_version(void) { return LF_ABI_VERSION; }

lf_status lf_cag_schedule(int32_t n_chunks, int32_t T, double s_base, double s_target,
                          const double* chunk_flops, const double* alpha, double* s_out,
                          double* beta_out) {
  const char* fn = "lf_cag_schedule";
  if (n_chunks < 2 || n_chunks > 4096) return fail(LF_ERR_INVALID_ARG, "%s: n_chunks must be in [2, 4096]", fn);
  if (T < 1) return fail(LF_ERR_INVALID_ARG, "%s: T must be >= 1", fn);
  if (!(s_base > 0.0 && s_base < 1.0)) return fail(LF_ERR_INVALID_ARG, "%s: s_base must be in (0, 1)", fn);
  if (!(s_target >= 0.0 && s_target < 1.0)) return fail(LF_ERR_INVALID_ARG, "%s: s_target must be in [0, 1)", fn);
  if (!chunk_flops || !s_out || !beta_out) return fail(LF_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  for (int i = 0; i < n_chunks; ++i) {
    if (!(std::isfinite(chunk_flops[i]) && chunk_flops[i] > 0.0))
      return fail(LF_ERR_INVALID_ARG, "%s: chunk_flops[%d] must be finite and > 0", fn, i);
    if (alpha && !(std::isfinite(alpha[i]) && alpha[i] >= 0.0))
      return fail(LF_ERR_INVALID_ARG, "%s: alpha[%d] must be finite and >= 0", fn, i);
  }
  // Total FLOP constraint sum_i F_i s_i = s_target sum_i F_i with s_1 = 0 and
  // s_i = s_base - alpha_i beta (i >= 2), solved for beta in closed form.
  double f_all = 0.0, f_sparse = 0.0, f_alpha = 0.0;
  for (int i = 0; i < n_chunks; ++i) {
    const double a = alpha ? alpha[i] : 1.0 / std::sqrt(static_cast<double>(i + 1) * T);
    f_all += chunk_flops[i];
    if (i > 0) {
      f_sparse += chunk_flops[i];
      f_alpha += chunk_flops[i] * a;
    }
  }
  if (!(f_alpha > 0.0)) return fail(LF_ERR_INVALID_ARG, "%s: alpha_i is zero for every sparse chunk", fn);
  const double beta = (s_base * f_sparse - s_target * f_all) / f_alpha;
  double s[4096];
  s[0] = 0.0;
  for (int i = 1; i < n_chunks; ++i) {
    const double a = alpha ? alpha[i] : 1.0 / std::sqrt(static_cast<double>(i + 1) * T);
    s[i] = s_base - a * beta;
  }
  if (beta < 0.0) return fail(LF_ERR_INFEASIBLE, "%s: target needs beta=%g < 0", fn, beta);
  for (int i = 1; i < n_chunks; ++i)
    if (!(s[i] >= 0.0 && s[i] < 1.0))
      return fail(LF_ERR_INFEASIBLE, "%s: s_%d=%g outside [0, 1)", fn, i + 1, s[i]);
  for (int i = 0; i < n_chunks; ++i) s_out[i] = s[i];
  *beta_out = beta;
  return LF_OK;
}

lf_status lf_block_budget(double s, int32_t n_kblocks, int32_t W_f, int32_t n_bpf, int32_t* k_b_out) {
  const char* fn = "lf_block_budget";
  if (!(s >= 0.0 && s <= 1.0)) return fail(LF_ERR_INVALID_ARG, "%s: s must be in [0, 1]", fn);
  if (n_kblocks < 1 || W_f < 1 || n_bpf < 1) return fail(LF_ERR_INVALID_ARG, "%s: sizes must be >= 1", fn);
  if (!k_b_out) return fail(LF_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  const double x = (1.0 - s) * static_cast<double>(n_kblocks) / static_cast<double>(W_f);
  double kb = std::floor(x + 0.5);
  if (kb < 1.0) kb = 1.0;
  if (kb > n_bpf) kb = n_bpf;
  *k_b_out = static_cast<int32_t>(kb);
  return LF_OK;
}

lf_status lf_pool(const void* x, lf_dtype dt, lf_geom g, int32_t n_frames, float* blk_out,
                  float* frm_out, void* stream) {
  const char* fn = "lf_pool";
  if (lf_status st = check_geom(g, fn)) return st;
  if (dt != LF_FP32 && dt != LF_BF16) return fail(LF_ERR_UNSUPPORTED, "%s: dtype %d unsupported", fn, (int)dt);
  if (n_frames < 1) return fail(LF_ERR_INVALID_ARG, "%s: n_frames must be >= 1", fn);
  if (!x || !blk_out) return fail(LF_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(x) || !aligned16(blk_out) || (frm_out && !aligned16(frm_out)))
    return fail(LF_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", fn);
  const int n_bpf = n_bpf_of(g);
  const long long BH = static_cast<long long>(g.B) * g.H;
  const long long len = static_cast<long long>(n_frames) * g.tokens_per_frame;
  if (!fits_int(BH * n_frames * n_bpf) || !fits_int(BH * n_frames * g.d) || !fits_int(len))
    return fail(LF_ERR_INVALID_ARG, "%s: problem too large", fn);
  if (g.head_stride != 0 && g.head_stride < len)
    return fail(LF_ERR_INVALID_ARG, "%s: head_stride %d < n_frames*tpf = %lld", fn, g.head_stride, len);
  const long long stride = g.head_stride ? g.head_stride : len;
  int out_stride = 0;
  if (lf_status st = pooled_stride(g, n_frames, &out_stride, fn)) return st;
  if (!fits_int(BH * out_stride * n_bpf)) return fail(LF_ERR_INVALID_ARG, "%s: problem too large", fn);
  pending_error();
  return hip_status(lf::launch_pool(x, dt == LF_BF16, g.d, static_cast<int>(BH), n_frames,
                                    g.tokens_per_frame, g.block_size, n_bpf, stride, out_stride, blk_out, frm_out,
                                    static_cast<hipStream_t>(stream)),
                    fn);
}

lf_status lf_pool_qk(const void* q, const void* k, lf_dtype dt, lf_geom g, int32_t n_qframes,
                     int32_t n_kframes, float* q_blk, float* k_blk, float* k_frm, void* stream) {
  const char* fn = "lf_pool_qk";
  if (lf_status st = check_geom(g, fn)) return st;
  if (dt != LF_FP32 && dt != LF_BF16) return fail(LF_ERR_UNSUPPORTED, "%s: dtype %d unsupported", fn, (int)dt);
  if (n_qframes < 1 || n_kframes < 1) return fail(LF_ERR_INVALID_ARG, "%s: n_qframes and n_kframes must be >= 1", fn);
  if (!q || !k || !q_blk || !k_blk || !k_frm) return fail(LF_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_blk) || !aligned16(k_blk) || !aligned16(k_frm))
    return fail(LF_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", fn);
  const int n_bpf = n_bpf_of(g);
  const long long BH = static_cast<long long>(g.B) * g.H;
  const long long lq = static_cast<long long>(n_qframes) * g.tokens_per_frame;
  const long long lk = static_cast<long long>(n_kframes) * g.tokens_per_frame;
  if (!fits_int(BH * (n_qframes + static_cast<long long>(n_kframes)) * n_bpf) || !fits_int(BH * n_kframes * g.d) ||
      !fits_int(lq) || !fits_int(lk))
    return fail(LF_ERR_INVALID_ARG, "%s: problem too large", fn);
  if (g.head_stride != 0 && g.head_stride < lq)
    return fail(LF_ERR_INVALID_ARG, "%s: head_stride %d < query token count %lld", fn, g.head_stride, lq);
  if (g.kv_head_stride != 0 && g.kv_head_stride < lk)
    return fail(LF_ERR_INVALID_ARG, "%s: kv_head_stride %d < key token count %lld", fn, g.kv_head_stride, lk);
  int k_out_stride = 0;
  if (lf_status st = pooled_stride(g, n_kframes, &k_out_stride, fn)) return st;
  if (!fits_int(BH * k_out_stride * n_bpf)) return fail(LF_ERR_INVALID_ARG, "%s: problem too large", fn);
  pending_error();
  return hip_status(lf::launch_pool_qk(q, k, dt == LF_BF16, g.d, static_cast<int>(BH), n_qframes, n_kframes,
                                       g.tokens_per_frame, g.block_size, n_bpf, g.head_stride ? g.head_stride : lq,
                                       g.kv_head_stride ? g.kv_head_stride : lk, k_out_stride, q_blk, k_blk, k_frm,
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

lf_status lf_qk_prologue(const void* x, void* x_out, const float* gamma, lf_dtype dt, lf_geom g, int32_t n_frames,
                         int32_t frame0, int32_t lat_w, float eps, float theta, float* blk_out, float* frm_out,
                         void* stream) {
  const char* fn = "lf_qk_prologue";
  if (lf_status st = check_geom(g, fn)) return st;
  if (dt != LF_FP32 && dt != LF_BF16) return fail(LF_ERR_UNSUPPORTED, "%s: dtype %d unsupported", fn, (int)dt);
  if (n_frames < 1 || frame0 < 0) return fail(LF_ERR_INVALID_ARG, "%s: n_frames must be >= 1 and frame0 >= 0", fn);
  if (lat_w < 1 || g.tokens_per_frame % lat_w != 0)
    return fail(LF_ERR_INVALID_ARG, "%s: lat_w=%d must divide tokens_per_frame=%d", fn, lat_w, g.tokens_per_frame);
  if (!(std::isfinite(eps) && eps > 0.f)) return fail(LF_ERR_INVALID_ARG, "%s: eps must be finite and > 0", fn);
  if (!(std::isfinite(theta) && theta > 1.f)) return fail(LF_ERR_INVALID_ARG, "%s: theta must be finite and > 1", fn);
  if (!x || !x_out || !gamma || !blk_out) return fail(LF_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(x) || !aligned16(x_out) || !aligned16(gamma) || !aligned16(blk_out) || (frm_out && !aligned16(frm_out)))
    return fail(LF_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", fn);
  if (x == x_out) return fail(LF_ERR_INVALID_ARG, "%s: x_out must not alias x", fn);
  const int n_bpf = n_bpf_of(g);
  const long long BH = static_cast<long long>(g.B) * g.H;
  const long long len = static_cast<long long>(n_frames) * g.tokens_per_frame;
  if (!fits_int(BH * n_frames * n_bpf) || !fits_int(BH * n_frames * g.d) || !fits_int(len) ||
      !fits_int(frame0 + static_cast<long long>(n_frames)))
    return fail(LF_ERR_INVALID_ARG, "%s: problem too large", fn);
  if (g.head_stride != 0 && g.head_stride < len)
    return fail(LF_ERR_INVALID_ARG, "%s: head_stride %d < n_frames*tpf = %lld", fn, g.head_stride, len);
  if (g.kv_head_stride != 0 && g.kv_head_stride < len)
    return fail(LF_ERR_INVALID_ARG, "%s: kv_head_stride %d < n_frames*tpf = %lld", fn, g.kv_head_stride, len);
  int out_stride = 0;
  if (lf_status st = pooled_stride(g, n_frames, &out_stride, fn)) return st;
  if (!fits_int(BH * out_stride * n_bpf)) return fail(LF_ERR_INVALID_ARG, "%s: problem too large", fn);
  lf::ProlArgs a;
  a.x = x;
  a.y = x_out;
  a.gamma = gamma;
  a.blk = blk_out;
  a.frm = frm_out;
  a.x_stride = g.head_stride ? g.head_stride : len;
  a.y_stride = g.kv_head_stride ? g.kv_head_stride : len;
  a.BH = static_cast<int>(BH);
  a.n_frames = n_frames;
  a.frame0 = frame0;
  a.out_stride = out_stride;
  a.tpf = g.tokens_per_frame;
  a.bs = g.block_size;
  a.n_bpf = n_bpf;
  a.lat_w = lat_w;
  a.eps = eps;
  rotary_turns(g.d, theta, a.rev);
  pending_error();
  return hip_status(lf::launch_prologue(a, dt == LF_BF16, g.d, static_cast<hipStream_t>(stream)), fn);
}

lf_status lf_pool_step(const void* q, const void* k_new, lf_dtype dt, lf_geom g, int32_t n_qframes, int32_t n_new,
                       int32_t f_new, int32_t f_lag, int32_t n_lag, float* q_blk, float* k_blk, float* k_frm,
                       void* stream) {
  const char* fn = "lf_pool_step";
  if (lf_status st = check_geom(g, fn)) return st;
  if (dt != LF_FP32 && dt != LF_BF16) return fail(LF_ERR_UNSUPPORTED, "%s: dtype %d unsupported", fn, (int)dt);
  if (n_qframes < 0) return fail(LF_ERR_INVALID_ARG, "%s: n_qframes must be >= 0", fn);
  int cs = 0;
  if (lf_status st = check_step_frames(g, n_new, f_new, f_lag, n_lag, &cs, fn)) return st;
  if ((n_qframes > 0 && (!q || !q_blk)) || (n_new > 0 && !k_new) || ((n_new > 0 || n_lag > 0) && !k_blk) ||
      (n_lag > 0 && !k_frm))
    return fail(LF_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if ((q && !aligned16(q)) || (k_new && !aligned16(k_new)) || (q_blk && !aligned16(q_blk)) ||
      (k_blk && !aligned16(k_blk)) || (k_frm && !aligned16(k_frm)))
    return fail(LF_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", fn);
  const int n_bpf = n_bpf_of(g);
  const long long BH = static_cast<long long>(g.B) * g.H;
  const long long lq = static_cast<long long>(n_qframes) * g.tokens_per_frame;
  const long long lk = static_cast<long long>(n_new) * g.tokens_per_frame;
  if (!fits_int(BH * (n_qframes + static_cast<long long>(n_new)) * n_bpf) || !fits_int(BH * cs * n_bpf) ||
      !fits_int(BH * cs * static_cast<long long>(g.d)) || !fits_int(lq) || !fits_int(lk))
    return fail(LF_ERR_INVALID_ARG, "%s: problem too large", fn);
  if (g.head_stride != 0 && g.head_stride < lq)
    return fail(LF_ERR_INVALID_ARG, "%s: head_stride %d < query token count %lld", fn, g.head_stride, lq);
  if (g.kv_head_stride != 0 && g.kv_head_stride < lk)
    return fail(LF_ERR_INVALID_ARG, "%s: kv_head_stride %d < new key token count %lld", fn, g.kv_head_stride, lk);
  if (n_qframes == 0 && n_new == 0 && n_lag == 0) return LF_OK;     // nothing to do
  lf::PoolStepArgs a;
  a.q = q;
  a.k = k_new;
  a.q_blk = q_blk;
  a.k_blk = k_blk;
  a.k_frm = k_frm;
  a.q_stride = g.head_stride ? g.head_stride : lq;
  a.k_stride = g.kv_head_stride ? g.kv_head_stride : lk;
  a.BH = static_cast<int>(BH);
  a.n_qframes = n_qframes;
  a.n_new = n_new;
  a.f_new = f_new;
  a.f_lag = f_lag;
  a.n_lag = n_lag;
  a.cache_stride = cs;
  a.tpf = g.tokens_per_frame;
  a.bs = g.block_size;
  a.n_bpf = n_bpf;
  pending_error();
  return hip_status(lf::launch_pool_step(a, dt == LF_BF16, g.d, static_cast<hipStream_t>(stream)), fn);
}

lf_status lf_qk_prologue_step(const void* q, const void* k_new, void* q_out, void* k_out, const float* gamma_q,
                              const float* gamma_k, lf_dtype dt, lf_geom g, int32_t n_frames, int32_t frame0,
                              int32_t lat_w, float eps, float theta, int32_t f_new, int32_t f_lag, int32_t n_lag,
                              float* q_blk, float* k_blk, float* k_frm, void* stream) {
  const char* fn = "lf_qk_prologue_step";
  if (lf_status st = check_geom(g, fn)) return st;
  if (dt != LF_FP32 && dt != LF_BF16) return fail(LF_ERR_UNSUPPORTED, "%s: dtype %d unsupported", fn, (int)dt);
  if (n_frames < 1 || frame0 < 0) return fail(LF_ERR_INVALID_ARG, "%s: n_frames must be >= 1 and frame0 >= 0", fn);
  if (lat_w < 1 || g.tokens_per_frame % lat_w != 0)
    return fail(LF_ERR_INVALID_ARG, "%s: lat_w=%d must divide tokens_per_frame=%d", fn, lat_w, g.tokens_per_frame);
  if (!(std::isfinite(eps) && eps > 0.f)) return fail(LF_ERR_INVALID_ARG, "%s: eps must be finite and > 0", fn);
  if (!(std::isfinite(theta) && theta > 1.f)) return fail(LF_ERR_INVALID_ARG, "%s: theta must be finite and > 1", fn);
  int cs = 0;
  if (lf_status st = check_step_frames(g, n_frames, f_new, f_lag, n_lag, &cs, fn)) return st;
  if (!q || !k_new || !q_out || !k_out || !gamma_q || !gamma_k || !q_blk || !k_blk || (n_lag > 0 && !k_frm))
    return fail(LF_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(q_out) || !aligned16(k_out) || !aligned16(gamma_q) ||
      !aligned16(gamma_k) || !aligned16(q_blk) || !aligned16(k_blk) || (k_frm && !aligned16(k_frm)))
    return fail(LF_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", fn);
  if (q == q_out || k_new == k_out) return fail(LF_ERR_INVALID_ARG, "%s: outputs must not alias inputs", fn);
  const int n_bpf = n_bpf_of(g);
  const long long BH = static_cast<long long>(g.B) * g.H;
  const long long len = static_cast<long long>(n_frames) * g.tokens_per_frame;
  if (!fits_int(BH * 2 * n_frames * n_bpf) || !fits_int(BH * cs * n_bpf) || !fits_int(BH * cs * static_cast<long long>(g.d)) ||
      !fits_int(len) || !fits_int(frame0 + static_cast<long long>(n_frames)))
    return fail(LF_ERR_INVALID_ARG, "%s: problem too large", fn);
  if (g.head_stride != 0 && g.head_stride < len)
    return fail(LF_ERR_INVALID_ARG, "%s: head_stride %d < n_frames*tpf = %lld", fn, g.head_stride, len);
  if (g.kv_head_stride != 0 && g.kv_head_stride < len)
    return fail(LF_ERR_INVALID_ARG, "%s: kv_head_stride %d < n_frames*tpf = %lld", fn, g.kv_head_stride, len);
  lf::ProlArgs a;
  a.x = q;
  a.y = q_out;
  a.gamma = gamma_q;
  a.blk = q_blk;
  a.frm = nullptr;
  a.x_stride = g.head_stride ? g.head_stride : len;
  a.y_stride = a.x_stride;
  a.BH = static_cast<int>(BH);
  a.n_frames = n_frames;
  a.frame0 = frame0;
  a.out_stride = n_frames;
  a.tpf = g.tokens_per_frame;
  a.bs = g.block_size;
  a.n_bpf = n_bpf;
  a.lat_w = lat_w;
  a.eps = eps;
  rotary_turns(g.d, theta, a.rev);
  lf::ProlStepArgs s;
  s.k = k_new;
  s.k_out = k_out;
  s.gamma_k = gamma_k;
  s.k_blk = k_blk;
  s.k_frm = k_frm;
  s.k_out_stride = g.kv_head_stride ? g.kv_head_stride : len;
  s.cache_stride = cs;
  s.f_new = f_new;
  s.f_lag = f_lag;
  s.n_lag = n_lag;
  pending_error();
  return hip_status(lf::launch_prologue_step(a, s, dt == LF_BF16, g.d, static_cast<hipStream_t>(stream)), fn);
}

lf_status lf_select_frames(const float* q_blk, const float* k_frm, lf_geom g, int32_t n_qb,
                           int32_t n_kframes, const int32_t* mem, int32_t n_mem,
                           const int32_t* forced, int32_t n_forced, int32_t k_f,
                           int32_t* frames_out, void* stream) {
  const char* fn = "lf_select_frames";
  lf::SelectArgs a = {};
  if (lf_status st = check_frame_stage(q_blk, k_frm, g, n_qb, n_kframes, mem, n_mem, forced, n_forced, k_f, a, fn))
    return st;
  if (!frames_out) return fail(LF_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (reinterpret_cast<uintptr_t>(frames_out) & 3u) return fail(LF_ERR_INVALID_ARG, "%s: misaligned buffer", fn);
  a.frames_out = frames_out;
  pending_error();
  return hip_status(lf::launch_select(a, g.d, g.B * g.H * n_qb, true, false, static_cast<hipStream_t>(stream)), fn);
}

lf_status lf_select_blocks(const float* q_blk, const float* k_blk, lf_geom g, int32_t n_qb,
                           int32_t n_kframes, const int32_t* frames, int32_t W_f, int32_t k_b,
                           int32_t* blocks_out, void* stream) {
  const char* fn = "lf_select_blocks";
  if (lf_status st = check_geom(g, fn)) return st;
  lf::SelectArgs a = {};
  if (lf_status st = check_block_stage(k_blk, g, n_qb, n_kframes, W_f, k_b, blocks_out, a, fn)) return st;
  if (!q_blk || !frames) return fail(LF_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(q_blk) || (reinterpret_cast<uintptr_t>(frames) & 3u))
    return fail(LF_ERR_INVALID_ARG, "%s: misaligned buffer", fn);
  a.q_blk = q_blk;
  a.frames_in = frames;
  pending_error();
  return hip_status(lf::launch_select(a, g.d, g.B * g.H * n_qb, false, true, static_cast<hipStream_t>(stream)), fn);
}

lf_status lf_select(const float* q_blk, const float* k_frm, const float* k_blk, lf_geom g, int32_t n_qb,
                    int32_t n_kframes, const int32_t* mem, int32_t n_mem, const int32_t* forced,
                    int32_t n_forced, int32_t k_f, int32_t k_b, int32_t* frames_out, int32_t* blocks_out,
                    void* stream) {
  const char* fn = "lf_select";
  lf::SelectArgs a = {};
  if (lf_status st = check_frame_stage(q_blk, k_frm, g, n_qb, n_kframes, mem, n_mem, forced, n_forced, k_f, a, fn))
    return st;
  if (lf_status st = check_block_stage(k_blk, g, n_qb, n_kframes, a.W_f, k_b, blocks_out, a, fn)) return st;
  if (frames_out && (reinterpret_cast<uintptr_t>(frames_out) & 3u))
    return fail(LF_ERR_INVALID_ARG, "%s: misaligned buffer", fn);
  a.frames_out = frames_out;
  pending_error();
  return hip_status(lf::launch_select(a, g.d, g.B * g.H * n_qb, true, true, static_cast<hipStream_t>(stream)), fn);
}

lf_status lf_select_blocks_1d(const float* q_blk, const float* k_blk, lf_geom g, int32_t n_qb,
                              int32_t n_kframes, int32_t K, int32_t* blocks_out, void* stream) {
  const char* fn = "lf_select_blocks_1d";
  if (lf_status st = check_geom(g, fn)) return st;
  if (n_qb < 1 || n_kframes < 1 || K < 1) return fail(LF_ERR_INVALID_ARG, "%s: n_qb, n_kframes and K must be >= 1", fn);
  const int n_bpf = n_bpf_of(g);
  const long long n_kb = static_cast<long long>(n_kframes) * n_bpf;
  if (n_kb > lf::kMax1DBlocks)
    return fail(LF_ERR_UNSUPPORTED, "%s: %lld key blocks > %d", fn, n_kb, lf::kMax1DBlocks);
  if (K > n_kb) return fail(LF_ERR_INVALID_ARG, "%s: K=%d > %lld key blocks", fn, K, n_kb);
  if (!q_blk || !k_blk || !blocks_out) return fail(LF_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(q_blk) || !aligned16(k_blk) || (reinterpret_cast<uintptr_t>(blocks_out) & 3u))
    return fail(LF_ERR_INVALID_ARG, "%s: misaligned buffer", fn);
  int fstride = 0;
  if (lf_status st = pooled_stride(g, n_kframes, &fstride, fn)) return st;
  const long long rows = static_cast<long long>(g.B) * g.H * n_qb;
  if (!fits_int(rows) || !fits_int(rows * K) || !fits_int(static_cast<long long>(g.B) * g.H * fstride * n_bpf))
    return fail(LF_ERR_INVALID_ARG, "%s: problem too large", fn);
  lf::Select1DArgs a;
  a.q_blk = q_blk;
  a.k_blk = k_blk;
  a.blocks_out = blocks_out;
  a.n_qb = n_qb;
  a.n_kb = static_cast<int>(n_kb);
  a.kb_stride = fstride * n_bpf;
  a.K = K;
  pending_error();
  return hip_status(lf::launch_select_1d(a, g.d, static_cast<int>(rows), static_cast<hipStream_t>(stream)), fn);
}

lf_status lf_sparse_attn(const void* q, const void* k, const void* v, void* o, lf_dtype dt,
                         lf_geom g, int32_t n_qframes, int32_t n_kframes, const int32_t* blocks,
                         int32_t W_b, float scale, void* stream) {
  const char* fn = "lf_sparse_attn";
  if (lf_status st = check_geom(g, fn)) return st;
  if (dt != LF_FP32 && dt != LF_BF16) return fail(LF_ERR_UNSUPPORTED, "%s: dtype %d unsupported", fn, (int)dt);
  if (dt == LF_BF16 && g.block_size > 64)
    return fail(LF_ERR_UNSUPPORTED, "%s: bf16 path needs block_size <= 64", fn);
  if (dt == LF_FP32 && g.block_size > 128)
    return fail(LF_ERR_UNSUPPORTED, "%s: fp32 path needs block_size <= 128", fn);
  if (n_qframes < 1 || n_kframes < 1 || W_b < 1)
    return fail(LF_ERR_INVALID_ARG, "%s: n_qframes, n_kframes and W_b must be >= 1", fn);
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(LF_ERR_INVALID_ARG, "%s: scale must be finite and > 0", fn);
  if (!q || !k || !v || !o || !blocks) return fail(LF_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(blocks) & 3u))
    return fail(LF_ERR_INVALID_ARG, "%s: misaligned buffer", fn);
  const int n_bpf = n_bpf_of(g);
  const long long BH = static_cast<long long>(g.B) * g.H;
  const long long n_qb = static_cast<long long>(n_qframes) * n_bpf;
  const long long n_kb = static_cast<long long>(n_kframes) * n_bpf;
  const long long lq = static_cast<long long>(n_qframes) * g.tokens_per_frame;
  const long long lk = static_cast<long long>(n_kframes) * g.tokens_per_frame;
  // the bf16 kernel addresses one (b, h) slice of K and V with 32-bit byte offsets
  if (!fits_int(BH * n_qb) || !fits_int(n_kb) || !fits_int(lq) || !fits_int(lk * g.d * 4))
    return fail(LF_ERR_INVALID_ARG, "%s: problem too large", fn);
  if (g.head_stride != 0 && g.head_stride < lq)
    return fail(LF_ERR_INVALID_ARG, "%s: head_stride %d < query token count %lld", fn, g.head_stride, lq);
  if (g.kv_head_stride != 0 && g.kv_head_stride < lk)
    return fail(LF_ERR_INVALID_ARG, "%s: kv_head_stride %d < key token count %lld", fn, g.kv_head_stride, lk);
  lf::AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.blocks = blocks;
  a.BH = static_cast<int>(BH); a.n_qb = static_cast<int>(n_qb); a.n_kb = static_cast<int>(n_kb);
  a.W_b = W_b; a.tpf = g.tokens_per_frame; a.bs = g.block_size; a.n_bpf = n_bpf;
  a.lq = static_cast<int>(lq); a.lk = static_cast<int>(lk);
  a.q_stride = g.head_stride ? g.head_stride : lq;
  a.kv_stride = g.kv_head_stride ? g.kv_head_stride : lk;
  a.scale_log2 = scale * 1.4426950408889634f;
  pending_error();
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(dt == LF_BF16 ? lf::launch_attn_bf16(a, g.d, st) : lf::launch_attn_f32(a, g.d, st), fn);
}

lf_status lf_probe_mfma_bf16(int32_t n_wg, int32_t iters, float* sink, int64_t* clocks, void* stream) {
  const char* fn = "lf_probe_mfma_bf16";
  if (n_wg < 1 || iters < 1) return fail(LF_ERR_INVALID_ARG, "%s: n_wg and iters must be >= 1", fn);
  if (!sink || !clocks) return fail(LF_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if ((reinterpret_cast<uintptr_t>(sink) & 3u) || (reinterpret_cast<uintptr_t>(clocks) & 7u))
    return fail(LF_ERR_INVALID_ARG, "%s: misaligned buffer", fn);
  pending_error();
  return hip_status(lf::launch_mfma_probe(n_wg, iters, sink, reinterpret_cast<long long*>(clocks),
                                          static_cast<hipStream_t>(stream)),
                    fn);
}

lf_status lf_probe_hbm_read(const void* x, int64_t bytes, int32_t n_wg, float* sink, void* stream) {
  const char* fn = "lf_probe_hbm_read";
  if (n_wg < 1) return fail(LF_ERR_INVALID_ARG, "%s: n_wg must be >= 1", fn);
  if (bytes <= 0 || (bytes % 16) != 0) return fail(LF_ERR_INVALID_ARG, "%s: bytes must be a positive multiple of 16", fn);
  if (!x || !sink) return fail(LF_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return fail(LF_ERR_INVALID_ARG, "%s: misaligned buffer", fn);
  pending_error();
  return hip_status(lf::launch_hbm_read(x, bytes, n_wg, sink, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
