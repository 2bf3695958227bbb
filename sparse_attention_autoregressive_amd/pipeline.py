"""One chunk of one layer through the whole HSA path, as a sequence of C-ABI calls.

Order (Light Forcing summary, execution flow, stages 2-3): pool the chunk's queries
(block means q~), pool all keys (block means k~ and frame means k^), frame top-k per
query block (T_r) and block top-k inside the chosen frames (the mask B_r as id lists)
in one selection launch, block-sparse attention. The two poolings share one launch.
All outputs are allocated once in a `Workspace`, so repeated calls (timing loops, the
per-layer sweep) allocate nothing.

Steady state (`PooledKeyCache`): a frame's keys do not change once the frame is in the
KV cache, so their block and frame means are computed once and kept; each later call
pools only the chunk's queries and its own key frames, and selection reads the cached
prefix. The chunk's own frames are always kept, so their frame means are first read by
the next chunk: each steady-state pooling launch forms the frame means of the previous
chunk's frames ("lagged") instead of its own, and `complete_cache` adds the last
chunk's. Results are bitwise those of the uncached path, since every frame's means are
computed by the same code from the same tokens.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Sequence

import torch

from . import (Geom, lf_block_budget, lf_cag_schedule, lf_pool, lf_pool_qk, lf_pool_step, lf_select,
               lf_select_blocks, lf_select_blocks_1d, lf_select_frames, lf_sparse_attn, n_bpf)


@dataclass
class ChunkPlan:
    """Static shape of one chunk's HSA call."""

    geom: Geom
    n_qframes: int
    n_kframes: int
    mem: Sequence[int]
    forced: Sequence[int]
    k_f: int
    k_b: int
    scale: float

    @property
    def n_bpf(self) -> int:
        return n_bpf(self.geom)

    @property
    def n_qb(self) -> int:
        return self.n_qframes * self.n_bpf

    @property
    def W_f(self) -> int:
        return len(self.forced) + min(self.k_f, len(self.mem))

    @property
    def W_b(self) -> int:
        return self.W_f * min(self.k_b, self.n_bpf)


class Workspace:
    """Preallocated intermediates and output for one ChunkPlan (the output is left out
    when the caller provides its own, as the sweep below does)."""

    def __init__(self, plan: ChunkPlan, dtype: torch.dtype, device, with_output: bool = True):
        g = plan.geom
        f32, i32 = torch.float32, torch.int32
        self.plan = plan
        self.q_blk = torch.empty((g.B, g.H, plan.n_qb, g.d), dtype=f32, device=device)
        self.k_blk = torch.empty((g.B, g.H, plan.n_kframes * plan.n_bpf, g.d), dtype=f32, device=device)
        self.k_frm = torch.empty((g.B, g.H, plan.n_kframes, g.d), dtype=f32, device=device)
        self.frames = torch.empty((g.B, g.H, plan.n_qb, plan.W_f), dtype=i32, device=device)
        self.blocks = torch.empty((g.B, g.H, plan.n_qb, plan.W_b), dtype=i32, device=device)
        self.o = (torch.empty((g.B, g.H, plan.n_qframes * g.tokens_per_frame, g.d), dtype=dtype, device=device)
                  if with_output else None)


def pool_q(ws: Workspace, q: torch.Tensor):
    p = ws.plan
    lf_pool(q, p.geom, p.n_qframes, blk_out=ws.q_blk, with_frames=False)


def pool_k(ws: Workspace, k: torch.Tensor):
    p = ws.plan
    lf_pool(k, p.geom, p.n_kframes, blk_out=ws.k_blk, frm_out=ws.k_frm)


def pool(ws: Workspace, q: torch.Tensor, k: torch.Tensor):
    """Both poolings in one launch (same results as pool_q + pool_k)."""
    p = ws.plan
    lf_pool_qk(q, k, p.geom, p.n_qframes, p.n_kframes, ws.q_blk, ws.k_blk, ws.k_frm)


def select_frames(ws: Workspace):
    p = ws.plan
    lf_select_frames(ws.q_blk, ws.k_frm, p.geom, p.n_qb, p.n_kframes, p.mem, p.forced, p.k_f,
                     out=ws.frames)


def select_blocks(ws: Workspace):
    p = ws.plan
    lf_select_blocks(ws.q_blk, ws.k_blk, p.geom, p.n_qb, p.n_kframes, ws.frames, p.k_b, out=ws.blocks)


def select(ws: Workspace):
    """Both selection stages in one launch (same results as select_frames + select_blocks)."""
    p = ws.plan
    lf_select(ws.q_blk, ws.k_frm, ws.k_blk, p.geom, p.n_qb, p.n_kframes, p.mem, p.forced, p.k_f, p.k_b,
              frames_out=ws.frames, blocks_out=ws.blocks)


def select_1d(ws: Workspace, out: torch.Tensor, K: int = 0) -> torch.Tensor:
    """The single-level comparison selection at the HSA budget (K = W_b unless given):
    top-K blocks over the whole prefix, written to `out` [B, H, n_qb, K]."""
    p = ws.plan
    return lf_select_blocks_1d(ws.q_blk, ws.k_blk, p.geom, p.n_qb, p.n_kframes, K or p.W_b, out=out)


def attend(ws: Workspace, q, k, v, out=None):
    p = ws.plan
    lf_sparse_attn(q, k, v, p.geom, p.n_qframes, p.n_kframes, ws.blocks, p.scale,
                   out=ws.o if out is None else out)


def hsa_chunk(ws: Workspace, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out=None) -> torch.Tensor:
    """Pool, select and attend for one chunk; returns the output (enqueued on the current
    stream). q, k, v and out may be token-range views of bigger per-head allocations."""
    pool(ws, q, k)
    select(ws)
    attend(ws, q, k, v, out)
    return ws.o if out is None else out


class PooledKeyCache:
    """Pooled keys of one layer for every frame of a clip: block means k~
    [B, H, n_frames*n_bpf, d] and frame means k^ [B, H, n_frames, d], fp32. Selection over
    the key prefix k_{:i} (Light Forcing summary, stage 3) reads the first frames; a
    frame's block means are written when its keys are pooled, its frame mean by the next
    chunk's pooling launch (or `complete_cache`). A steady-state chunk therefore expects
    the block means of every earlier frame and the frame means of all but the previous
    chunk's frames (filled by the earlier chunks, or by `lf_pool` for a history pooled at
    once)."""

    def __init__(self, g: Geom, n_frames: int, device):
        self.geom, self.n_frames, self.nb = g, n_frames, n_bpf(g)
        f32 = torch.float32
        self.k_blk = torch.empty((g.B, g.H, n_frames * self.nb, g.d), dtype=f32, device=device)
        self.k_frm = torch.empty((g.B, g.H, n_frames, g.d), dtype=f32, device=device)

    def blk(self, f0: int, f1: int) -> torch.Tensor:
        """Block means of frames [f0, f1) (a view)."""
        return self.k_blk[:, :, f0 * self.nb:f1 * self.nb]

    def frm(self, f0: int, f1: int) -> torch.Tensor:
        """Frame means of frames [f0, f1) (a view)."""
        return self.k_frm[:, :, f0:f1]


def new_frames(p: ChunkPlan) -> int:
    """First key frame of the chunk itself: its keys are the last n_qframes of the prefix."""
    return p.n_kframes - p.n_qframes


def _lag(p: ChunkPlan):
    """The previous chunk's frames: (first frame, count) of the lagged frame means."""
    f0 = new_frames(p)
    n = min(p.n_qframes, f0)
    return f0 - n, n


def pool_cached(ws: Workspace, cache: PooledKeyCache, q: torch.Tensor, k: torch.Tensor):
    """Pools the chunk's queries and only its own key frames (the last n_qframes of the
    key prefix k) into `cache`, plus the frame means of the previous chunk's frames from
    their cached block means, in one launch."""
    p = ws.plan
    f0, tpf = new_frames(p), p.geom.tokens_per_frame
    fl, nl = _lag(p)
    lf_pool_step(q, k[:, :, f0 * tpf:], p.geom, p.n_qframes, p.n_qframes, f0, fl, nl, ws.q_blk, cache.k_blk,
                 cache.k_frm)


def pool_keys_cached(p: ChunkPlan, cache: PooledKeyCache, k: torch.Tensor):
    """Pools only the chunk's own key frames into `cache` (a dense chunk needs no pooled
    queries, but later chunks select over its keys), with the lagged frame means."""
    f0, tpf = new_frames(p), p.geom.tokens_per_frame
    fl, nl = _lag(p)
    lf_pool_step(None, k[:, :, f0 * tpf:], p.geom, 0, p.n_qframes, f0, fl, nl, None, cache.k_blk, cache.k_frm)


def complete_cache(p: ChunkPlan, cache: PooledKeyCache):
    """The frame means of chunk p's own frames (which its pooling leaves to the next
    chunk), from their cached block means: for a cache no later chunk will extend."""
    lf_pool_step(None, None, p.geom, 0, 0, 0, new_frames(p), p.n_qframes, None, cache.k_blk, cache.k_frm)


def select_cached(ws: Workspace, cache: PooledKeyCache):
    """Both selection stages over the cached pooled keys of the key prefix."""
    p = ws.plan
    lf_select(ws.q_blk, cache.frm(0, p.n_kframes), cache.blk(0, p.n_kframes), p.geom, p.n_qb, p.n_kframes,
              p.mem, p.forced, p.k_f, p.k_b, frames_out=ws.frames, blocks_out=ws.blocks)


def hsa_chunk_cached(ws: Workspace, cache: PooledKeyCache, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     out=None) -> torch.Tensor:
    """hsa_chunk in steady state: the pooled keys of the earlier frames come from `cache`
    (filled by earlier chunks); the chunk's own key frames are pooled into it."""
    pool_cached(ws, cache, q, k)
    select_cached(ws, cache)
    attend(ws, q, k, v, out)
    return ws.o if out is None else out


def denoise_steps(ws: Workspace, cache: PooledKeyCache, k_cache: torch.Tensor, v_cache: torch.Tensor, steps):
    """The T denoising steps of one chunk in steady state (Light Forcing summary, execution
    flow: chunk i's sparsity is tied to the T steps it is denoised over, stage 1, and every
    step selects over the key prefix k_{:i}, stages 2-3). `steps` yields (q, k_chunk,
    v_chunk, out) per step: the step's queries, the chunk's own keys and values -- copied
    here into the KV caches at the chunk's frames -- and the output. The history's pooled
    keys in `cache` are read as they are (pooled once, by the earlier chunks; each step
    re-forms the previous chunk's lagged frame means, the same values); the chunk's own
    frames' block means are re-pooled at every step, since their keys change, and their
    frame means are left to the next chunk (or `complete_cache`). k_cache and v_cache
    hold the clip ([B, H, >= n_kframes * tpf, d]); returns the last step's output."""
    p = ws.plan
    tpf = p.geom.tokens_per_frame
    a, b = new_frames(p) * tpf, p.n_kframes * tpf
    out = None
    for q, k_new, v_new, out in steps:
        k_cache[:, :, a:b].copy_(k_new)
        v_cache[:, :, a:b].copy_(v_new)
        out = hsa_chunk_cached(ws, cache, q, k_cache[:, :, :b], v_cache[:, :, :b], out)
    return out


# ------------------------------------------------------------------ Chunk-Aware Growth sweep
@dataclass
class SweepPlan:
    """The schedule of one clip under Chunk-Aware Growth (Light Forcing summary,
    execution flow, stage 1; technical summary section 2.1): chunk i (1-based) queries
    its frames_per_chunk frames against the key prefix of frames_per_chunk*i frames, with
    sparsity s[i-1] from the CAG schedule and k_b from the block budget. A chunk with
    s = 0 (the first) runs dense attention over the full block list."""

    geom: Geom
    frames_per_chunk: int
    s: List[float]
    beta: float
    chunks: List[ChunkPlan] = field(default_factory=list)

    @property
    def n_chunks(self) -> int:
        return len(self.chunks)

    @property
    def n_frames(self) -> int:
        return self.frames_per_chunk * self.n_chunks

    def dense(self, i: int) -> bool:
        return self.s[i - 1] == 0.0


def plan_sweep(g: Geom, n_chunks: int, frames_per_chunk: int, k_f: int, T: int, s_base: float,
               s_target: float, scale: float, sink: Sequence[int] = (0,), schedule: str = "cag") -> SweepPlan:
    """Sparsity schedule (once per clip) and per-chunk plans. The FLOP weight of chunk i is
    its dense attention work, query tokens times key tokens (proportional to i).
    schedule "cag": Chunk-Aware Growth. "uniform": the allocation CAG is compared against
    (163.com article, section 2), chunk 1 dense and one sparsity for every later chunk
    under the same FLOP budget; it is the CAG solution for a constant alpha, so it comes
    from the same library call."""
    fpc, tpf, nb = frames_per_chunk, g.tokens_per_frame, n_bpf(g)
    flops = [float(fpc * tpf * fpc * i * tpf) for i in range(1, n_chunks + 1)]
    if schedule not in ("cag", "uniform"):
        raise ValueError(f"unknown schedule {schedule!r}")
    alpha = [1.0] * n_chunks if schedule == "uniform" else None
    s, beta = lf_cag_schedule(n_chunks, T, s_base, s_target, flops, alpha)
    sp = SweepPlan(g, fpc, s, beta)
    for i in range(1, n_chunks + 1):
        cur = list(range(fpc * (i - 1), fpc * i))
        forced = sorted(set(sink) | set(cur))
        mem = [f for f in range(fpc * (i - 1)) if f not in forced]
        W_f = len(forced) + min(k_f, len(mem))
        k_b = lf_block_budget(s[i - 1], fpc * i * nb, W_f, nb)
        sp.chunks.append(ChunkPlan(g, fpc, fpc * i, mem, forced, k_f, k_b, scale))
    return sp


class SweepWorkspace:
    """Per-chunk workspaces of a SweepPlan (reused by every layer), plus the full block
    lists of the dense chunks."""

    def __init__(self, sp: SweepPlan, dtype: torch.dtype, device):
        g = sp.geom
        self.plan = sp
        self.chunks = [Workspace(p, dtype, device, with_output=False) for p in sp.chunks]
        self.full = {}
        for i, p in enumerate(sp.chunks, 1):
            if sp.dense(i):
                n_kb = p.n_kframes * p.n_bpf
                ids = torch.arange(n_kb, dtype=torch.int32, device=device)
                self.full[i] = ids.expand(g.B, g.H, p.n_qb, n_kb).contiguous()


def sweep_layer(sw: SweepWorkspace, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                o: torch.Tensor, mark=None, cache: PooledKeyCache = None, complete: bool = True,
                stages: int = 3) -> torch.Tensor:
    """All chunks of one layer in order. q, k, v, o: [B, H, n_frames*tpf, d] holding the
    whole clip; chunk i reads its query frames and the key prefix as views and writes its
    frames of o. Enqueued on the current stream; returns o. `mark(i, stage)`, if given,
    is called before each stage ("pool", "select", "attn") and with stage
    "end" after chunk i (e.g. to record timing events). With a `cache` (this layer's,
    sized for the clip), every chunk pools only its own key frames into it, the dense
    first chunk included, and selection reads the cached prefix: the same outputs. The
    cache then holds every frame's means on return (the last chunk's frame means are
    formed after its attention, by `complete_cache`), unless `complete` is False.
    `stages` < 3 runs only the first stages of every chunk (1: pooling, 2: pooling and
    selection), for timing the stages apart; o is then not written."""
    sp = sw.plan
    tpf = sp.geom.tokens_per_frame
    tick = mark if mark is not None else (lambda i, stage: None)
    for i, (p, ws) in enumerate(zip(sp.chunks, sw.chunks), 1):
        a, b = (i - 1) * sp.frames_per_chunk * tpf, i * sp.frames_per_chunk * tpf
        qv, ov, kv, vv = q[:, :, a:b], o[:, :, a:b], k[:, :, :b], v[:, :, :b]
        if sp.dense(i):
            if cache is not None:
                tick(i, "pool")
                pool_keys_cached(p, cache, kv)
            if stages >= 3:
                tick(i, "attn")
                lf_sparse_attn(qv, kv, vv, p.geom, p.n_qframes, p.n_kframes, sw.full[i], p.scale, out=ov)
        else:
            tick(i, "pool")
            if cache is None:
                pool(ws, qv, kv)
            else:
                pool_cached(ws, cache, qv, kv)
            if stages >= 2:
                tick(i, "select")
                if cache is None:
                    select(ws)
                else:
                    select_cached(ws, cache)
            if stages >= 3:
                tick(i, "attn")
                attend(ws, qv, kv, vv, ov)
        tick(i, "end")
    if cache is not None and complete and sp.chunks:
        complete_cache(sp.chunks[-1], cache)
    return o
