"""One chunk of one layer through the whole HSA path, as a sequence of C-ABI calls.

Order (Light Forcing summary, execution flow, stages 2-3): pool the chunk's queries
(block means q~), pool all keys (block means k~ and frame means k^), frame top-k per
query block (T_r), block top-k inside the chosen frames (the mask B_r as id lists),
block-sparse attention. All outputs are allocated once in a `Workspace`, so repeated
calls (timing loops, the per-layer sweep) allocate nothing.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Sequence

import torch

from . import (Geom, lf_pool, lf_select_blocks, lf_select_frames, lf_sparse_attn, n_bpf)


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
    """Preallocated intermediates and output for one ChunkPlan."""

    def __init__(self, plan: ChunkPlan, dtype: torch.dtype, device):
        g = plan.geom
        f32, i32 = torch.float32, torch.int32
        self.plan = plan
        self.q_blk = torch.empty((g.B, g.H, plan.n_qb, g.d), dtype=f32, device=device)
        self.k_blk = torch.empty((g.B, g.H, plan.n_kframes * plan.n_bpf, g.d), dtype=f32, device=device)
        self.k_frm = torch.empty((g.B, g.H, plan.n_kframes, g.d), dtype=f32, device=device)
        self.frames = torch.empty((g.B, g.H, plan.n_qb, plan.W_f), dtype=i32, device=device)
        self.blocks = torch.empty((g.B, g.H, plan.n_qb, plan.W_b), dtype=i32, device=device)
        self.o = torch.empty((g.B, g.H, plan.n_qframes * g.tokens_per_frame, g.d), dtype=dtype, device=device)


def pool_q(ws: Workspace, q: torch.Tensor):
    p = ws.plan
    lf_pool(q, p.geom, p.n_qframes, blk_out=ws.q_blk, with_frames=False)


def pool_k(ws: Workspace, k: torch.Tensor):
    p = ws.plan
    lf_pool(k, p.geom, p.n_kframes, blk_out=ws.k_blk, frm_out=ws.k_frm)


def select_frames(ws: Workspace):
    p = ws.plan
    lf_select_frames(ws.q_blk, ws.k_frm, p.geom, p.n_qb, p.n_kframes, p.mem, p.forced, p.k_f,
                     out=ws.frames)


def select_blocks(ws: Workspace):
    p = ws.plan
    lf_select_blocks(ws.q_blk, ws.k_blk, p.geom, p.n_qb, p.n_kframes, ws.frames, p.k_b, out=ws.blocks)


def attend(ws: Workspace, q, k, v):
    p = ws.plan
    lf_sparse_attn(q, k, v, p.geom, p.n_qframes, p.n_kframes, ws.blocks, p.scale, out=ws.o)


def hsa_chunk(ws: Workspace, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> torch.Tensor:
    """Pool, select and attend for one chunk; returns ws.o (enqueued on the current stream)."""
    pool_q(ws, q)
    pool_k(ws, k)
    select_frames(ws)
    select_blocks(ws)
    attend(ws, q, k, v)
    return ws.o
