/*
 * lf.h -- C ABI of the MI355X (gfx950) implementation of Light Forcing's Hierarchical
 * Sparse Attention (HSA) and Chunk-Aware Growth (CAG) schedule, for one chunk of an
 * autoregressive video-diffusion transformer.
 *
 * Citations name the page and its part:
 *   [S1]/[S2]/[S3]  Light Forcing summary (paper.rainbus.top/paper/2602.04789), the
 *                   execution-flow paragraph, stage 1 (CAG), stage 2 (token
 *                   compression), stage 3 (two-level mask selection + block-sparse
 *                   attention).
 *   [G2.1]/[G2.2]   Light Forcing technical summary (gist.science/paper/2602.04789),
 *                   section 2.1 (CAG) and section 2.2 (HSA).
 *
 * Conventions shared by every call
 *   - Return value: lf_status; LF_OK (0) on success. On failure nothing is enqueued,
 *     no output is written, and lf_last_error() returns a message for this thread.
 *   - Device calls are asynchronous on `stream` (a hipStream_t, e.g. the value of
 *     torch.cuda.current_stream().cuda_stream; NULL means the default stream). All
 *     tensors are caller-owned device buffers, row-major and contiguous, 16-byte
 *     aligned, and must stay alive until the stream work completes. The library
 *     allocates nothing, keeps no pointer after returning, and fully overwrites each
 *     output. No atomics are used: identical inputs give bitwise-identical outputs.
 *   - Precondition (not checked on the device): input values are finite.
 *   - Token geometry (frame-aligned blocks): frame f holds tokens [f*tpf, (f+1)*tpf);
 *     block j of a frame holds its tokens [j*bs, min((j+1)*bs, tpf)), so each frame has
 *     n_bpf = ceil(tpf/bs) blocks, the last one possibly shorter; the global block id of
 *     block j of frame f is f*n_bpf + j. Queries use the same rule on the chunk's own
 *     frames (query block r = frame r/n_bpf, block r%n_bpf).
 *   - Token tensors (x, q, k, v, o) are [B, H, tokens, d]: batch, head, token, channel,
 *     with each (b, h) slice contiguous. Two strides give the distance in tokens between
 *     consecutive (b, h) slices: g.head_stride for the query side (q, o, and lf_pool's
 *     x) and g.kv_head_stride for the key side (k, v). 0 means packed (the tensor's own
 *     token count); a larger value addresses a prefix or a window of a bigger
 *     allocation, such as an autoregressive KV cache sized for the whole video.
 *   - Pooled key tensors (k~ [B, H, frames*n_bpf, d], k^ [B, H, frames, d]) have their
 *     (b, h) slices g.frame_stride frames apart: 0 means packed (the call's key-frame
 *     count); a larger value addresses the first frames of a pooled-key cache sized for
 *     the whole video, so the keys of each frame are pooled once when it enters the KV
 *     cache and reused by every later chunk. Pooled queries and id lists are always
 *     packed.
 */
#ifndef LF_H
#define LF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LF_ABI_VERSION 4

typedef enum {
  LF_OK = 0,
  LF_ERR_INVALID_ARG = 1, /* a pointer, size, id or set violates the contract       */
  LF_ERR_UNSUPPORTED = 2, /* valid in principle, but not built for (dtype, d, sizes) */
  LF_ERR_INFEASIBLE = 3,  /* CAG target cannot be met without clamping               */
  LF_ERR_HIP = 4          /* the HIP runtime reported an error at launch             */
} lf_status;

typedef enum { LF_FP32 = 0, LF_BF16 = 1 } lf_dtype;

/* B batch, H heads, d head dim, tokens_per_frame (tpf), block_size (bs), head_stride
 * (tokens between (b, h) slices of q, o and lf_pool's x; 0 = packed), kv_head_stride
 * (the same for k and v; 0 = packed), frame_stride (frames between (b, h) slices of the
 * pooled key tensors; 0 = packed). */
typedef struct {
  int32_t B, H, d, tokens_per_frame, block_size;
  int32_t head_stride;
  int32_t kv_head_stride;
  int32_t frame_stride;
} lf_geom;

/* Message for the last failing call on the calling thread ("" if none). The pointer
 * stays valid until the next lf_* call on this thread. */
const char* lf_last_error(void);

/* LF_ABI_VERSION of the loaded library. */
int32_t lf_abi_version(void);

/* ---------------------------------------------------------------------------------
 * lf_cag_schedule -- [S1], [G2.1]: per-chunk sparsity s_1..s_n of Chunk-Aware Growth.
 * Host only, synchronous, no GPU needed.
 *   s_1 = 0 (the first chunk keeps dense attention); s_i = s_base - alpha_i * beta for
 *   i > 1, with beta chosen so that the attention FLOPs kept over all chunks,
 *   sum_i F_i (1 - s_i), equal (1 - s_target) * sum_i F_i.
 * n_chunks >= 2; T >= 1 denoising steps; 0 <= s_target < 1; 0 < s_base < 1.
 * chunk_flops[i] (host, n_chunks entries, > 0): dense attention FLOPs of chunk i+1 in
 *   any common unit (for equal chunks against a growing cache, F_i is proportional to i).
 * alpha (host, n_chunks entries, or NULL): the alpha_i weights. NULL selects
 *   alpha_i = 1/sqrt(i*T), this library's reading of "alpha_i proportional to 1/sqrt(T),
 *   the noise level reached by chunk i". alpha_1 is ignored. A constant alpha makes
 *   every s_i (i > 1) equal: the uniform allocation CAG is compared against, under the
 *   same FLOP budget (163.com article on Light Forcing, section 2).
 * Outputs (host): s_out[n_chunks], *beta_out.
 * Errors: LF_ERR_INVALID_ARG for bad sizes/pointers/values; LF_ERR_INFEASIBLE when the
 *   solution has beta < 0 or some s_i outside [0, 1) (nothing is clamped).
 * ------------------------------------------------------------------------------- */
lf_status lf_cag_schedule(int32_t n_chunks, int32_t T, double s_base, double s_target,
                          const double* chunk_flops, const double* alpha, double* s_out,
                          double* beta_out);

/* ---------------------------------------------------------------------------------
 * lf_block_budget -- turns a chunk sparsity s into the per-frame block top-k k_b.
 * The pages leave this step to a hyper-parameter table that is not available; this
 * library keeps round-half-up((1 - s) * n_kblocks / W_f) blocks per selected frame,
 * clamped to [1, n_bpf], so the W_f selected frames hold about (1 - s) of the
 * n_kblocks key blocks. Host only, synchronous.
 * Errors: LF_ERR_INVALID_ARG if s is not in [0, 1], n_kblocks < 1, W_f < 1, n_bpf < 1
 *   or k_b_out is NULL.
 * ------------------------------------------------------------------------------- */
lf_status lf_block_budget(double s, int32_t n_kblocks, int32_t W_f, int32_t n_bpf,
                          int32_t* k_b_out);

/* ---------------------------------------------------------------------------------
 * lf_pool -- [S2] token compression by mean pooling.
 * x: [B, H, n_frames*tpf, d] in dtype dt (LF_BF16 or LF_FP32); with a nonzero
 *   g.head_stride the (b, h) slice starts at x + (b*H + h)*head_stride*d
 *   (head_stride >= n_frames*tpf; g.kv_head_stride is not used).
 * blk_out: [B, H, n_frames*n_bpf, d] fp32, the mean of each block's tokens (q~ for the
 *   chunk's queries, k~ for keys), divided by the block's true token count.
 * frm_out: [B, H, n_frames, d] fp32, the mean of each frame's tpf tokens (k^), or NULL
 *   to skip (e.g. when pooling queries).
 * Both outputs have their (b, h) slices g.frame_stride frames apart (0 = packed,
 *   otherwise >= n_frames): pooling a chunk's new frames into a pooled-key cache passes
 *   the cache at the first new frame. Frame means are formed from the fp32 block
 *   means weighted by their token counts.
 * Limits: d in {64, 128}; 1 <= bs <= tpf; tpf <= 65536; n_frames >= 1; B, H >= 1;
 *   head_stride = 0 or >= n_frames*tpf.
 * Errors: LF_ERR_INVALID_ARG (NULL/unaligned pointers, bad sizes), LF_ERR_UNSUPPORTED
 *   (d or dtype), LF_ERR_HIP (launch).
 * ------------------------------------------------------------------------------- */
lf_status lf_pool(const void* x, lf_dtype dt, lf_geom g, int32_t n_frames, float* blk_out,
                  float* frm_out, void* stream);

/* ---------------------------------------------------------------------------------
 * lf_pool_qk -- [S2] both poolings of one chunk in one launch: the chunk's queries (block
 * means only) and all keys (block and frame means), with results bitwise equal to
 * lf_pool(q, ..., n_qframes, q_blk, NULL) followed by lf_pool(k, ..., n_kframes, k_blk,
 * k_frm).
 * q: [B, H, n_qframes*tpf, d], k: [B, H, n_kframes*tpf, d], both in dtype dt; their
 *   (b, h) slices are g.head_stride (q) and g.kv_head_stride (k) tokens apart, each
 *   0 (packed) or at least the tensor's token count.
 * q_blk: [B, H, n_qframes*n_bpf, d] fp32 (packed); k_blk: [B, H, n_kframes*n_bpf, d] fp32;
 *   k_frm: [B, H, n_kframes, d] fp32; the key outputs use g.frame_stride as lf_pool's do.
 * Limits and errors: those of lf_pool.
 * ------------------------------------------------------------------------------- */
lf_status lf_pool_qk(const void* q, const void* k, lf_dtype dt, lf_geom g, int32_t n_qframes,
                     int32_t n_kframes, float* q_blk, float* k_blk, float* k_frm, void* stream);

/* ---------------------------------------------------------------------------------
 * lf_qk_prologue -- the query/key prologue before attention (RMSNorm and rotary position
 * embedding, named among the released deployment kernels in the Light Forcing summary's
 * reproducibility paragraph and defined nowhere on the pages), fused with [S2] pooling so
 * the chunk's queries or keys are read from HBM once:
 *   y = RMSNorm(x) = x / sqrt(mean_c(x_c^2) + eps) * gamma       (over each token's d channels)
 *   x_out = RoPE(y): adjacent channel pairs (2k, 2k+1) rotate, (a, b) -> (a cos phi - b sin phi,
 *     a sin phi + b cos phi); of the d/2 pairs the first d/2 - 2*floor(d/6) turn with the
 *     token's frame (frame0 + frame within x), the next floor(d/6) with its row and the last
 *     floor(d/6) with its column in the latent frame (tokens_per_frame / lat_w rows of lat_w
 *     tokens, row-major); pair i of an axis with n pairs has phi = position * theta^(-i/n).
 *   blk_out, frm_out: the block and frame means of x_out exactly as lf_pool(x_out) would give
 *     them (bitwise), with g.frame_stride as for lf_pool; frm_out may be NULL.
 * x, x_out: [B, H, n_frames*tpf, d] in dtype dt; the (b, h) slices of x are g.head_stride
 *   tokens apart and those of x_out g.kv_head_stride apart (each 0 = packed), so a chunk's
 *   packed projection can be written into a KV cache sized for the clip; x_out is rounded
 *   to dt (round to nearest even) and must not alias x.
 * gamma: [d] fp32 (device). eps > 0; theta > 1 (10000 in the usual setting).
 * Numerics: fp32 arithmetic; the rotation uses hardware sine/cosine after reducing
 *   position * theta^(-i/n) / (2 pi) to [-1/2, 1/2] revolutions (about 1e-6 absolute
 *   error, far below one bf16 step).
 * Limits: those of lf_pool; lat_w divides tpf; frame0 >= 0.
 * Errors: LF_ERR_INVALID_ARG, LF_ERR_UNSUPPORTED (d, dtype), LF_ERR_HIP.
 * ------------------------------------------------------------------------------- */
lf_status lf_qk_prologue(const void* x, void* x_out, const float* gamma, lf_dtype dt, lf_geom g,
                         int32_t n_frames, int32_t frame0, int32_t lat_w, float eps, float theta,
                         float* blk_out, float* frm_out, void* stream);

/* ---------------------------------------------------------------------------------
 * lf_pool_step -- [S2] the pooling of one chunk in steady state, in one launch. A frame's
 * keys do not change once it is in the KV cache, so its block and frame means are kept in
 * a pooled-key cache; each call pools the chunk's queries and only its new key frames.
 * The chunk's own frames are always kept by [S3] (current-chunk frames), so their frame
 * means are first read by the next chunk's frame stage: this call leaves them out and
 * instead forms the frame means of n_lag earlier frames (normally the previous chunk's)
 * from block means that an earlier call wrote, in the same launch.
 *   q_blk  <- block means of q (n_qframes frames; packed [B, H, n_qframes*n_bpf, d] fp32)
 *   k_blk  <- block means of k_new at cache frames [f_new, f_new + n_new)
 *   k_frm  <- frame means of cache frames [f_lag, f_lag + n_lag), from k_blk
 * q: [B, H, n_qframes*tpf, d], slices g.head_stride tokens apart (0 = packed); k_new:
 *   [B, H, n_new*tpf, d], slices g.kv_head_stride apart (0 = packed); dtype dt.
 * k_blk, k_frm: the pooled-key cache at frame 0 ([B, H, frames*n_bpf, d] and
 *   [B, H, frames, d] fp32), slices g.frame_stride frames apart; g.frame_stride is the
 *   cache's frame count and must be >= 1 (no packed form here).
 * Results are bitwise those of lf_pool / lf_pool_qk over the same frames. n_qframes,
 * n_new and n_lag may each be 0 (the matching pointers may then be NULL); with all three 0
 * the call does nothing. The two frame ranges must lie in the cache and be disjoint.
 * Limits and errors: those of lf_pool_qk.
 * ------------------------------------------------------------------------------- */
lf_status lf_pool_step(const void* q, const void* k_new, lf_dtype dt, lf_geom g, int32_t n_qframes,
                       int32_t n_new, int32_t f_new, int32_t f_lag, int32_t n_lag, float* q_blk,
                       float* k_blk, float* k_frm, void* stream);

/* ---------------------------------------------------------------------------------
 * lf_qk_prologue_step -- lf_qk_prologue of a chunk's queries and of its new keys in one
 * launch, with the pooling of lf_pool_step: q_out = RoPE(RMSNorm(q; gamma_q)) and
 * k_out = RoPE(RMSNorm(k_new; gamma_k)) (both at clip frames frame0 .. frame0 +
 * n_frames - 1, lat_w tokens per latent row), q_blk <- block means of q_out, k_blk <-
 * block means of k_out at cache frames [f_new, f_new + n_frames), k_frm <- frame means of
 * cache frames [f_lag, f_lag + n_lag) from k_blk (n_lag may be 0, k_frm then NULL).
 * Every output is bitwise what lf_qk_prologue of each tensor (without frame means) gives.
 * q, k_new, q_out: [B, H, n_frames*tpf, d], slices g.head_stride tokens apart; k_out:
 *   the same shape, slices g.kv_head_stride apart (a KV cache view); dtype dt; outputs
 *   must not alias inputs. gamma_q, gamma_k: [d] fp32.
 * k_blk, k_frm, g.frame_stride: as for lf_pool_step. eps, theta, lat_w: as for
 *   lf_qk_prologue.
 * Errors: LF_ERR_INVALID_ARG, LF_ERR_UNSUPPORTED (d, dtype), LF_ERR_HIP.
 * ------------------------------------------------------------------------------- */
lf_status lf_qk_prologue_step(const void* q, const void* k_new, void* q_out, void* k_out,
                              const float* gamma_q, const float* gamma_k, lf_dtype dt, lf_geom g,
                              int32_t n_frames, int32_t frame0, int32_t lat_w, float eps, float theta,
                              int32_t f_new, int32_t f_lag, int32_t n_lag, float* q_blk, float* k_blk,
                              float* k_frm, void* stream);

/* ---------------------------------------------------------------------------------
 * lf_select_frames -- [S3] frame stage: for every row (b, h, query block r), the frame
 * relevance p_r(f) = <q~_r, k^_f> over the memory set M; the top-min(k_f, |M|)
 * frames of M ranked by (score descending, frame id ascending) join the always-kept
 * frames (sink, recent and current-chunk frames, passed as `forced`) to form T_r.
 * q_blk: [B, H, n_qb, d] fp32 (lf_pool of the queries). k_frm: [B, H, n_kframes, d]
 *   fp32 (frame means of all key frames; only those in M are read), (b, h) slices
 *   g.frame_stride frames apart (0 = packed).
 * mem, forced: HOST arrays of frame ids (n_mem, n_forced entries), each id in
 *   [0, n_kframes), no duplicates, the two sets disjoint; W_f (below) must be >= 1.
 * frames_out: [B, H, n_qb, W_f] int32, W_f = n_forced + min(k_f, n_mem), each row
 *   ascending.
 * Limits: d in {64, 128}; n_kframes <= 4096 (about 16 minutes of 480p latent frames);
 *   k_f >= 0. Up to 256 key frames the frame stage ranks by counting (one frame of M per
 *   thread); beyond, two rows of a head share each workgroup and each row takes its k_f
 *   best in k_f rounds of a wave-wide maximum (over the scores at or above the k_f-th
 *   largest lane maximum when at most 64 are), with the same result.
 * Errors: LF_ERR_INVALID_ARG, LF_ERR_UNSUPPORTED (d, n_kframes), LF_ERR_HIP.
 * ------------------------------------------------------------------------------- */
lf_status lf_select_frames(const float* q_blk, const float* k_frm, lf_geom g, int32_t n_qb,
                           int32_t n_kframes, const int32_t* mem, int32_t n_mem,
                           const int32_t* forced, int32_t n_forced, int32_t k_f,
                           int32_t* frames_out, void* stream);

/* ---------------------------------------------------------------------------------
 * lf_select_blocks -- [S3] block stage: for every row and every tau in T_r, the block
 * relevance o_r(tau, j) = <q~_r, k~_j^(tau)> over the frame's n_bpf blocks; the top
 * min(k_b, n_bpf) blocks J_r(tau) ranked by (score descending, j ascending). The mask
 * B_r(tau, j) = 1[tau in T_r, j in J_r(tau)] is emitted as an ascending list of global
 * block ids tau*n_bpf + j.
 * q_blk: [B, H, n_qb, d] fp32. k_blk: [B, H, n_kframes*n_bpf, d] fp32, (b, h) slices
 *   g.frame_stride frames apart (0 = packed).
 * frames: [B, H, n_qb, W_f] int32 device array, each row ascending and unique with ids
 *   in [0, n_kframes) (the output of lf_select_frames). A row breaking this gets
 *   unspecified list entries; nothing outside the buffers is read or written.
 * blocks_out: [B, H, n_qb, W_f*min(k_b, n_bpf)] int32.
 * Limits: d in {64, 128}; n_bpf <= 64; n_kframes <= 65535; k_b >= 1; W_f >= 1.
 * Errors: LF_ERR_INVALID_ARG, LF_ERR_UNSUPPORTED, LF_ERR_HIP.
 * ------------------------------------------------------------------------------- */
lf_status lf_select_blocks(const float* q_blk, const float* k_blk, lf_geom g, int32_t n_qb,
                           int32_t n_kframes, const int32_t* frames, int32_t W_f, int32_t k_b,
                           int32_t* blocks_out, void* stream);

/* ---------------------------------------------------------------------------------
 * lf_select -- [S3] both selection stages in one launch: lf_select_frames followed by
 * lf_select_blocks, with the same arguments, validation and results (bitwise), without
 * the round trip of T_r through memory between two launches.
 * q_blk, k_frm, k_blk: as above. mem, forced, k_f: as for lf_select_frames; W_f =
 *   n_forced + min(k_f, n_mem). k_b: as for lf_select_blocks.
 * frames_out: [B, H, n_qb, W_f] int32, or NULL to skip writing T_r.
 * blocks_out: [B, H, n_qb, W_f*min(k_b, n_bpf)] int32.
 * Limits: those of both calls (n_kframes <= 4096, n_bpf <= 64).
 * Errors: LF_ERR_INVALID_ARG, LF_ERR_UNSUPPORTED, LF_ERR_HIP.
 * ------------------------------------------------------------------------------- */
lf_status lf_select(const float* q_blk, const float* k_frm, const float* k_blk, lf_geom g,
                    int32_t n_qb, int32_t n_kframes, const int32_t* mem, int32_t n_mem,
                    const int32_t* forced, int32_t n_forced, int32_t k_f, int32_t k_b,
                    int32_t* frames_out, int32_t* blocks_out, void* stream);

/* ---------------------------------------------------------------------------------
 * lf_select_blocks_1d -- the single-granularity selection HSA is contrasted with (Light
 * Forcing summary, novelty paragraph; 163.com article, ablation section: "1D" sparse
 * attention): every key block j of the prefix is scored o_r(j) = <q~_r, k~_j>, and the
 * top K blocks ranked by (score descending, j ascending) form the row's list, ascending.
 * There is no frame stage and no always-kept frame; for a comparison at equal budget pass
 * K = the HSA list length W_f*min(k_b, n_bpf).
 * q_blk: [B, H, n_qb, d] fp32. k_blk: [B, H, n_kframes*n_bpf, d] fp32, (b, h) slices
 *   g.frame_stride frames apart (0 = packed).
 * blocks_out: [B, H, n_qb, K] int32, each row ascending; feed it to lf_sparse_attn with
 *   W_b = K.
 * Limits: d in {64, 128}; 1 <= K <= n_kframes*n_bpf <= 4096.
 * Errors: LF_ERR_INVALID_ARG, LF_ERR_UNSUPPORTED (d, block count), LF_ERR_HIP.
 * ------------------------------------------------------------------------------- */
lf_status lf_select_blocks_1d(const float* q_blk, const float* k_blk, lf_geom g, int32_t n_qb,
                              int32_t n_kframes, int32_t K, int32_t* blocks_out, void* stream);

/* ---------------------------------------------------------------------------------
 * lf_sparse_attn -- [S3], [G2.2] block-sparse attention: each query token t of query
 * block r attends only to the tokens of the blocks listed for r,
 *   o_t = sum_u softmax_u(scale * <q_t, k_u>) v_u   (softmax over the listed tokens).
 * With every block listed this is dense attention (CAG's first chunk).
 * q, o: [B, H, n_qframes*tpf, d]; k, v: [B, H, n_kframes*tpf, d]; all in dtype dt.
 *   The (b, h) slices of q and o are g.head_stride tokens apart, those of k and v
 *   g.kv_head_stride tokens apart; each 0 (packed) or at least the token count (so a
 *   chunk's packed queries can attend to a prefix of a KV cache sized for the video).
 * blocks: [B, H, n_qb, W_b] int32 device array, n_qb = n_qframes*n_bpf; ids should be
 *   unique (a repeated id is counted twice); ids outside [0, n_kframes*n_bpf) are
 *   skipped. A row with no valid id produces zeros.
 * scale: the softmax scale (usually 1/sqrt(d)); finite and > 0.
 * LF_BF16 runs on bf16 matrix cores (fp32 accumulate and softmax) and needs d = 128 or
 *   64 and bs <= 64; LF_FP32 runs in fp32 on the vector units and needs d in {64, 128}
 *   and bs <= 128.
 * Errors: LF_ERR_INVALID_ARG, LF_ERR_UNSUPPORTED, LF_ERR_HIP.
 * ------------------------------------------------------------------------------- */
lf_status lf_sparse_attn(const void* q, const void* k, const void* v, void* o, lf_dtype dt,
                         lf_geom g, int32_t n_qframes, int32_t n_kframes,
                         const int32_t* blocks, int32_t W_b, float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LF_H */
