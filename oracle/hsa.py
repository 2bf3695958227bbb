"""CPU oracle for Light Forcing's Hierarchical Sparse Attention (HSA) and Chunk-Aware
Growth (CAG). TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may import
this module. The product path (the HIP library and its Python binding) never calls it,
and it shares no code, table or helper with that path.

Plain, slow and fp64 throughout. Each function follows one step of the method in the
order and notation of the pages:

  [S1] Light Forcing summary (paper.rainbus.top/paper/2602.04789), execution-flow
       paragraph, stage 1: Chunk-Aware Growth. Chunk 1 stays dense; chunk i > 1 gets
       sparsity s_i = s_base - alpha_i * beta, alpha_i proportional to 1/sqrt(T), and
       beta is fixed by requiring the total FLOPs to meet the target sparsity.
  [S2] same paragraph, stage 2: token compression. Block-level mean pooling of the
       chunk's queries q^(i) and of all keys k_{:i} gives q~^(i), k~_{:i}; frame-level
       pooling of the keys of the memory set M gives k^_M.
  [S3] same paragraph, stage 3: two-level mask selection. Frame relevance
       p_r = <q~_r, k^_M>, top-k frames T_r per query block r (sink, recent and
       current-chunk frames always kept); block relevance o_r(tau, j) = <q~_r, k~_j^(tau)>
       with top-k blocks J_r(tau) inside each tau in T_r; block mask
       B_r(tau, j) = 1[tau in T_r, j in J_r(tau)]; block-sparse attention over it.
  [G2.1], [G2.2] Light Forcing technical summary (gist.science/paper/2602.04789),
       section 2.1 (CAG) and section 2.2 (HSA: attention only over the selected
       frame-block pairs, fixed cost independent of the number of history frames).
  [A2] 163.com article on Light Forcing, section 2 (片段感知增长): beta is solved from an
       equation making the FLOP-weighted sum of chunk sparsities equal the target.

Readings where the pages are silent (labelled R1..R20 throughout): alpha_i
= 1/sqrt(i*T) (R1); chunk FLOP weights F_i given by the caller (R2); the budget rule
turning s_i into a per-frame block count (R4, R17); frame-aligned ragged blocks (R5,
R6); memory set = key frames not forced (R7); per-head masks (R8); per-frame block
top-k also inside forced frames (R9); raw inner products (R10); ties broken toward the
lower index (R11); k >= candidates keeps all (R12); no causal mask (R13); softmax over
the selected tokens only, scale 1/sqrt(d) (R14); ascending fixed-width lists (R15); the
single-level comparison variant keeps no frame always (R23).

Parity status: the pages print no worked example and no reference output, so the
whole pipeline is pinned by closed forms, invariants, library special cases and brute
force (tests/test_oracle_*.py); CAG's alpha_i law and the budget rule are readings and
are "parity unpinned" by the pages beyond those invariants.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

# --------------------------------------------------------------------------- geometry


def block_geometry(tpf: int, bs: int):
    """Frame-aligned blocks (reading R5): block j of a frame covers its tokens
    [j*bs, min((j+1)*bs, tpf)). Returns (n_bpf, starts, lens) within one frame."""
    n_bpf = -(-tpf // bs)
    starts = [j * bs for j in range(n_bpf)]
    lens = [min(bs, tpf - s) for s in starts]
    return n_bpf, starts, lens


def block_tokens(g: int, tpf: int, bs: int) -> np.ndarray:
    """Token indices of global block id g = frame * n_bpf + j."""
    n_bpf, starts, lens = block_geometry(tpf, bs)
    f, j = divmod(g, n_bpf)
    a = f * tpf + starts[j]
    return np.arange(a, a + lens[j])


# --------------------------------------------------------------------------- [S1] CAG


def cag_alpha(n_chunks: int, T: int) -> np.ndarray:
    """alpha_i for i = 1..n: reading R1, alpha_i = 1/sqrt(i*T) (the pages give only
    alpha_i proportional to 1/sqrt(T), the noise level chunk i reaches)."""
    return np.array([1.0 / math.sqrt(i * T) for i in range(1, n_chunks + 1)])


def cag_schedule(n_chunks: int, T: int, s_base: float, s_target: float,
                 chunk_flops: Sequence[float], alpha: Optional[Sequence[float]] = None):
    """[S1], [G2.1], [A2]: per-chunk sparsities s_1..s_n and beta.

    s_1 = 0 (chunk 1 dense); s_i = s_base - alpha_i * beta for i > 1, with beta chosen
    so that the FLOPs kept, sum_i F_i (1 - s_i), equal (1 - s_target) sum_i F_i, i.e.
    the FLOP-weighted mean sparsity equals s_target. The constraint is affine in beta,
    so its root follows from two evaluations. Raises ValueError if beta < 0 or any
    s_i falls outside [0, 1) (reading R18: no clamping).
    """
    F = np.asarray(chunk_flops, dtype=np.float64)
    if F.shape != (n_chunks,) or n_chunks < 1:
        raise ValueError("chunk_flops must have n_chunks entries")
    a = cag_alpha(n_chunks, T) if alpha is None else np.asarray(alpha, dtype=np.float64)

    def sched(beta):
        s = s_base - a * beta
        s[0] = 0.0
        return s

    def excess(beta):  # FLOP-weighted sparsity minus its target
        return float(np.dot(F, sched(beta)) - s_target * F.sum())

    e0, e1 = excess(0.0), excess(1.0)
    if n_chunks < 2 or e1 == e0:
        raise ValueError("beta is undetermined (needs a sparse chunk with alpha > 0)")
    beta = -e0 / (e1 - e0)
    s = sched(beta)
    if beta < 0 or np.any(s < 0) or np.any(s >= 1):
        raise ValueError(f"infeasible CAG target: beta={beta}, s={s}")
    return s, beta


def uniform_schedule(n_chunks: int, s_target: float, chunk_flops: Sequence[float]):
    """The allocation Chunk-Aware Growth is compared against (163.com article, section 2:
    the same FLOP budget spread uniformly; gist.science technical summary, section 1: the
    isolated treatment of chunks): chunk 1 dense, every later chunk at one sparsity s',
    fixed by the same budget as CAG. Solving F_1 + (1 - s') * sum_{i>1} F_i =
    (1 - s_target) * sum_i F_i for s' gives s' = s_target * sum_i F_i / sum_{i>1} F_i.
    Raises ValueError if s' is not in [0, 1)."""
    F = np.asarray(chunk_flops, dtype=np.float64)
    if F.shape != (n_chunks,) or n_chunks < 2:
        raise ValueError("chunk_flops must have n_chunks >= 2 entries")
    sp = s_target * F.sum() / F[1:].sum()
    if not (0.0 <= sp < 1.0):
        raise ValueError(f"infeasible uniform target: s'={sp}")
    s = np.full(n_chunks, sp)
    s[0] = 0.0
    return s


def block_budget(s: float, n_kb: int, W_f: int, n_bpf: int) -> int:
    """Reading R4/R17 (the pages' per-chunk top-k table is not available): keep
    round-half-up((1 - s) * n_kb / W_f) blocks per selected frame, clamped to
    [1, n_bpf], so the W_f selected frames together hold about (1 - s) of all key
    blocks."""
    x = (1.0 - s) * n_kb / W_f
    return int(min(max(math.floor(x + 0.5), 1), n_bpf))


# --------------------------------------------------------------------------- [S2] pooling


def pool_blocks(x: np.ndarray, n_frames: int, tpf: int, bs: int) -> np.ndarray:
    """Block-level mean pooling: x [B,H,n_frames*tpf,d] -> [B,H,n_frames*n_bpf,d],
    each output the sum of the block's tokens divided by its true token count."""
    n_bpf, starts, lens = block_geometry(tpf, bs)
    B, H, L, d = x.shape
    assert L == n_frames * tpf
    out = np.empty((B, H, n_frames * n_bpf, d))
    for f in range(n_frames):
        for j in range(n_bpf):
            a = f * tpf + starts[j]
            out[:, :, f * n_bpf + j] = x[:, :, a:a + lens[j]].astype(np.float64).sum(axis=2) / lens[j]
    return out


def pool_frames(x: np.ndarray, n_frames: int, tpf: int) -> np.ndarray:
    """Frame-level mean pooling k^: the mean over all tpf tokens of each frame."""
    B, H, L, d = x.shape
    assert L == n_frames * tpf
    return x.astype(np.float64).reshape(B, H, n_frames, tpf, d).sum(axis=3) / tpf


# --------------------------------------------------------------------------- [S3] selection


def _top(scores: np.ndarray, ids: np.ndarray, k: int):
    """Rank candidates by (score descending, id ascending) -- reading R11 -- and keep
    the first k. Returns (kept ids, gap at the cut; inf when nothing is cut)."""
    order = np.lexsort((ids, -scores))
    k = min(k, len(ids))
    gap = math.inf
    if 0 < k < len(ids):
        gap = float(scores[order[k - 1]] - scores[order[k]])
    return ids[order[:k]], gap


def select_frames(q_blk: np.ndarray, k_frm: np.ndarray, mem: Sequence[int],
                  forced: Sequence[int], k_f: int):
    """Frame stage of [S3]: p_r(f) = <q~_r, k^_f> for f in M; the top-min(k_f, |M|) of
    M by (-p, f) join the always-kept frames; T_r is their union in ascending order.

    q_blk [B,H,n_qb,d], k_frm [B,H,n_frames,d]. Returns (frames [B,H,n_qb,W_f] int64,
    gaps [B,H,n_qb] of p at the cut) with W_f = |forced| + min(k_f, |M|)."""
    mem = np.asarray(sorted(mem), dtype=np.int64)
    forced = sorted(int(f) for f in forced)
    assert not set(forced) & set(mem.tolist())
    B, H, n_qb, d = q_blk.shape
    W_f = len(forced) + min(k_f, len(mem))
    frames = np.empty((B, H, n_qb, W_f), dtype=np.int64)
    gaps = np.full((B, H, n_qb), math.inf)
    for b in range(B):
        for h in range(H):
            for r in range(n_qb):
                chosen = np.empty(0, dtype=np.int64)
                if len(mem):
                    p_r = k_frm[b, h, mem] @ q_blk[b, h, r]
                    chosen, gaps[b, h, r] = _top(p_r, mem, k_f)
                frames[b, h, r] = sorted(forced + chosen.tolist())
    return frames, gaps


def select_blocks(q_blk: np.ndarray, k_blk: np.ndarray, frames: np.ndarray, n_bpf: int,
                  k_b: int):
    """Block stage of [S3]: for each tau in T_r, o_r(tau, j) = <q~_r, k~_j^(tau)> over the
    frame's n_bpf blocks; J_r(tau) = top-min(k_b, n_bpf) by (-o, j). The mask B_r is
    returned as the ascending list of global ids tau*n_bpf + j.

    Returns (blocks [B,H,n_qb,W_f*min(k_b,n_bpf)] int64, gaps [B,H,n_qb,W_f])."""
    B, H, n_qb, W_f = frames.shape
    kb = min(k_b, n_bpf)
    blocks = np.empty((B, H, n_qb, W_f * kb), dtype=np.int64)
    gaps = np.full((B, H, n_qb, W_f), math.inf)
    js = np.arange(n_bpf, dtype=np.int64)
    for b in range(B):
        for h in range(H):
            for r in range(n_qb):
                ids = []
                for t, tau in enumerate(frames[b, h, r]):
                    o_r = k_blk[b, h, tau * n_bpf + js] @ q_blk[b, h, r]
                    J, gaps[b, h, r, t] = _top(o_r, js, k_b)
                    ids.extend(int(tau) * n_bpf + np.sort(J))
                blocks[b, h, r] = ids
    return blocks, gaps


def select_blocks_1d(q_blk: np.ndarray, k_blk: np.ndarray, K: int):
    """The single-granularity selection HSA is contrasted with (Light Forcing summary,
    novelty paragraph: earlier dynamic sparse attention picks blocks at one level only;
    163.com article, ablation section: the "1D" variant): every key block j of the prefix
    is scored o_r(j) = <q~_r, k~_j>, and the top-min(K, n_kb) by (-o, j) form the row's
    list, ascending. There is no frame stage and no always-kept frame (reading R23).

    q_blk [B,H,n_qb,d], k_blk [B,H,n_kb,d]. Returns (blocks [B,H,n_qb,min(K,n_kb)] int64,
    gaps [B,H,n_qb] of o at the cut)."""
    B, H, n_qb, d = q_blk.shape
    n_kb = k_blk.shape[2]
    ke = min(K, n_kb)
    blocks = np.empty((B, H, n_qb, ke), dtype=np.int64)
    gaps = np.full((B, H, n_qb), math.inf)
    ids = np.arange(n_kb, dtype=np.int64)
    for b in range(B):
        for h in range(H):
            for r in range(n_qb):
                o_r = k_blk[b, h] @ q_blk[b, h, r]
                J, gaps[b, h, r] = _top(o_r, ids, K)
                blocks[b, h, r] = np.sort(J)
    return blocks, gaps


def block_mask(blocks: np.ndarray, n_kb: int) -> np.ndarray:
    """B_r(tau, j) = 1[tau in T_r, j in J_r(tau)] of [S3] as a dense boolean [B,H,n_qb,n_kb]
    over global block ids tau*n_bpf + j, from the per-row id lists (reading R15)."""
    B, H, n_qb, _ = blocks.shape
    m = np.zeros((B, H, n_qb, n_kb), dtype=bool)
    for b in range(B):
        for h in range(H):
            for r in range(n_qb):
                m[b, h, r, blocks[b, h, r]] = True
    return m


def frame_scores(q_blk: np.ndarray, k_frm: np.ndarray, b: int, h: int, r: int,
                 frames: Sequence[int]) -> np.ndarray:
    """Frame relevance of [S3], p_r(f) = <q~_r, k^_f>, of row (b, h, r) for each frame in
    `frames` (raw inner products, reading R10)."""
    return np.array([float(np.dot(q_blk[b, h, r], k_frm[b, h, int(f)])) for f in frames])


def block_scores(q_blk: np.ndarray, k_blk: np.ndarray, b: int, h: int, r: int, tau: int,
                 n_bpf: int) -> np.ndarray:
    """Block relevance of [S3], o_r(tau, j) = <q~_r, k~_j^(tau)>, of row (b, h, r) for the
    blocks j = 0..n_bpf-1 of frame tau."""
    return np.array([float(np.dot(q_blk[b, h, r], k_blk[b, h, int(tau) * n_bpf + j])) for j in range(n_bpf)])


# --------------------------------------------------------------------------- attention


def _softmax_rows(logits: np.ndarray) -> np.ndarray:
    z = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def sparse_attn(q: np.ndarray, k: np.ndarray, v: np.ndarray, blocks: np.ndarray,
                tpf: int, bs: int, scale: float, rows=None) -> np.ndarray:
    """Block-sparse attention ([S3], [G2.2]): each query token t of query block r attends
    to the tokens of the blocks listed for r only: o_t = sum_u softmax_u(scale q_t.k_u) v_u
    (readings R13, R14). q [B,H,Lq,d]; k, v [B,H,Lk,d]; blocks [B,H,n_qb,W_b].

    `rows` optionally restricts the work to a list of (b, h, r); the other output rows
    are left as NaN. Returns o [B,H,Lq,d] fp64."""
    B, H, Lq, d = q.shape
    o = np.full((B, H, Lq, d), np.nan)
    n_qb = blocks.shape[2]
    if rows is None:
        rows = [(b, h, r) for b in range(B) for h in range(H) for r in range(n_qb)]
    for b, h, r in rows:
        qt = block_tokens(r, tpf, bs)
        kt = np.concatenate([block_tokens(int(g), tpf, bs) for g in blocks[b, h, r]])
        P = _softmax_rows(scale * (q[b, h, qt].astype(np.float64) @ k[b, h, kt].astype(np.float64).T))
        o[b, h, qt] = P @ v[b, h, kt].astype(np.float64)
    return o


def dense_attn(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Full attention softmax(scale * Q K^T) V over all key tokens (chunk 1 under CAG)."""
    B, H, Lq, d = q.shape
    o = np.empty((B, H, Lq, d))
    for b in range(B):
        for h in range(H):
            P = _softmax_rows(scale * (q[b, h].astype(np.float64) @ k[b, h].astype(np.float64).T))
            o[b, h] = P @ v[b, h].astype(np.float64)
    return o


# --------------------------------------------------------------------------- pipeline


def hsa(q, k, v, *, tpf: int, bs: int, n_kframes: int, mem, forced, k_f: int, k_b: int,
        scale: float, attn_rows=None, with_attn: bool = True) -> dict:
    """One chunk of one layer through [S2] then [S3]. Returns every intermediate."""
    n_bpf, _, _ = block_geometry(tpf, bs)
    n_qframes = q.shape[2] // tpf
    q_blk = pool_blocks(q, n_qframes, tpf, bs)
    k_blk = pool_blocks(k, n_kframes, tpf, bs)
    k_frm = pool_frames(k, n_kframes, tpf)
    frames, fgaps = select_frames(q_blk, k_frm, mem, forced, k_f)
    blocks, bgaps = select_blocks(q_blk, k_blk, frames, n_bpf, k_b)
    out = dict(q_blk=q_blk, k_blk=k_blk, k_frm=k_frm, frames=frames, frame_gaps=fgaps,
               blocks=blocks, block_gaps=bgaps, n_bpf=n_bpf)
    if with_attn:
        out["o"] = sparse_attn(q, k, v, blocks, tpf, bs, scale, rows=attn_rows)
    return out


def attn_flops(blocks: np.ndarray, tpf: int, bs: int, n_kframes: int) -> tuple:
    """(dense, active) query-key token-pair counts over all heads: the sum over query
    blocks r of |r|*Lk, and of |r|*sum_{g in list_r}|g|. Times 4*d gives the FLOPs of
    the two products Q K^T and P V."""
    n_bpf, _, lens = block_geometry(tpf, bs)
    B, H, n_qb, _ = blocks.shape
    lk = n_kframes * tpf
    qlen = np.array([lens[r % n_bpf] for r in range(n_qb)])
    glen = np.array(lens)[blocks % n_bpf]                 # [B,H,n_qb,W_b]
    dense = B * H * qlen.sum() * lk
    active = float((qlen[None, None, :] * glen.sum(axis=-1)).sum())
    return float(dense), active
