"""Seeded synthetic Q/K/V with planted frame/block relevance.

The pages measure on model activations (Self Forcing / LongLive / Infinite-Forcing on
VBench prompts) that are not available here; these tensors stand in for them with the
same shapes and an explicit relevance structure:

  frame codes   c_f ~ N(0, I_d)                      per (b, h, key frame)
  block codes   u   = c_f + 0.5 * N(0, I)            per (b, h, key frame, block)
  keys          K_t = u_(block of t) + N(0, I)       per token
  values        V_t = u_(block of t) + N(0, I)       per token
  query pairs   (a, b) drawn without replacement from the workload's history pool,
                one pair per (b, h, query block)
  queries       Q_t = (c_a + c_b) / 2 + N(0, I)      per token of that query block

Draw order (one numpy Generator(PCG64(seed)) per workload/layer): [planted frames],
c, block noise, K noise, V noise, pairs, Q noise. Everything is drawn in float32 and
then rounded once to the workload dtype (bf16 round-to-nearest-even via torch); both
the HIP path and the CPU oracle read those rounded values.

Blocks are frame-aligned: block j of a frame covers its tokens [j*bs, min((j+1)*bs, tpf)).
This module only builds inputs; it performs none of the method's computation.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Sequence

import numpy as np
import torch

from .configs import Sweep, Workload

_TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class Inputs:
    """Q [B,H,Lq,d], K/V [B,H,Lk,d] as CPU torch tensors in the workload dtype."""

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    pairs: np.ndarray          # [B,H,n_qb,2] frame ids planted into each query block
    planted: tuple             # the planting pool actually used

    def np64(self):
        """Float64 numpy copies of (q, k, v) holding exactly the rounded values."""
        return tuple(t.to(torch.float64).numpy() for t in (self.q, self.k, self.v))


def _block_lens(tpf: int, bs: int) -> np.ndarray:
    n = -(-tpf // bs)
    return np.array([min(bs, tpf - j * bs) for j in range(n)], dtype=np.int64)


def _draw_kv(rng, B, H, nf, tpf, bs, d):
    lens = _block_lens(tpf, bs)
    nb = len(lens)
    c = rng.standard_normal((B, H, nf, d), dtype=np.float32)
    u = c[:, :, :, None, :] + np.float32(0.5) * rng.standard_normal((B, H, nf, nb, d), dtype=np.float32)
    tok = np.repeat(u, lens, axis=3).reshape(B, H, nf * tpf, d)
    del u
    k = tok + rng.standard_normal(tok.shape, dtype=np.float32)
    v = tok + rng.standard_normal(tok.shape, dtype=np.float32)
    return c, k, v, lens


def _draw_q(rng, c, pool: Sequence[int], n_qframes, lens, tpf):
    B, H, _, d = c.shape
    nb = len(lens)
    n_qb = n_qframes * nb
    pool = np.asarray(pool, dtype=np.int64)
    if len(pool) < 2:
        raise ValueError("query planting needs at least two pool frames")
    order = rng.random((B, H, n_qb, len(pool))).argsort(axis=-1)[..., :2]
    pairs = pool[order]                                        # [B,H,n_qb,2]
    bi = np.arange(B)[:, None, None]
    hi = np.arange(H)[None, :, None]
    code = (c[bi, hi, pairs[..., 0]] + c[bi, hi, pairs[..., 1]]) * np.float32(0.5)
    q = np.repeat(code, np.tile(lens, n_qframes), axis=2)      # [B,H,Lq,d]
    q = q + rng.standard_normal(q.shape, dtype=np.float32)
    return q, pairs


def _to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(_TORCH_DTYPE[dtype]).contiguous()


def make(w: Workload) -> Inputs:
    """Inputs of one workload, from seed w.seed."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    if w.planted_from is not None:
        pool = tuple(sorted(int(x) for x in rng.choice(np.asarray(w.planted_from),
                                                        w.planted_count, replace=False)))
    else:
        pool = tuple(w.q_pool)
    c, k, v, lens = _draw_kv(rng, w.B, w.H, w.n_kframes, w.tpf, w.bs, w.d)
    q, pairs = _draw_q(rng, c, pool, w.n_qframes, lens, w.tpf)
    return Inputs(_to_dtype(q, w.dtype), _to_dtype(k, w.dtype), _to_dtype(v, w.dtype), pairs, pool)


def make_denoise_steps(w: Workload, T: int, step_noise: float = 0.5):
    """Inputs of the T denoising steps of one chunk: step 0 is `make(w)`; at each later step
    t the chunk's own frames (the last n_qframes key frames) get new keys and values and
    the chunk gets new queries -- step 0's tokens plus step_noise * N(0, I), drawn from
    Generator(PCG64(w.seed + 7919 t)) -- while the history frames' keys and values stay
    those of step 0. Returns a list of T Inputs."""
    base = make(w)
    q0, k0, v0 = (t.to(torch.float32).numpy() for t in (base.q, base.k, base.v))
    f0 = (w.n_kframes - w.n_qframes) * w.tpf
    steps = [base]
    for t in range(1, T):
        rng = np.random.Generator(np.random.PCG64(w.seed + 7919 * t))
        k, v = k0.copy(), v0.copy()
        k[:, :, f0:] += np.float32(step_noise) * rng.standard_normal(k[:, :, f0:].shape, dtype=np.float32)
        v[:, :, f0:] += np.float32(step_noise) * rng.standard_normal(v[:, :, f0:].shape, dtype=np.float32)
        q = q0 + np.float32(step_noise) * rng.standard_normal(q0.shape, dtype=np.float32)
        steps.append(Inputs(_to_dtype(q, w.dtype), _to_dtype(k, w.dtype), _to_dtype(v, w.dtype), base.pairs,
                            base.planted))
    return steps


def make_sweep_layer(s: Sweep, layer: int) -> Inputs:
    """Q/K/V of all 3*n_chunks frames of one sweep layer (seed s.seed(layer)).

    Chunk i's query blocks are planted from its own history pool (frames 0..3i-4; the
    first chunk, which has no history, from its own frames). Chunk i reads Q frames
    3i-3..3i-1 and the K/V prefix 0..3i-1.
    """
    rng = np.random.Generator(np.random.PCG64(s.seed(layer)))
    c, k, v, lens = _draw_kv(rng, s.B, s.H, s.n_frames, s.tpf, s.bs, s.d)
    qs, ps = [], []
    for i in range(1, s.n_chunks + 1):
        pool = s.chunk(i, layer).q_pool
        q, pairs = _draw_q(rng, c, pool, s.frames_per_chunk, lens, s.tpf)
        qs.append(q)
        ps.append(pairs)
    q = np.concatenate(qs, axis=2)
    pairs = np.concatenate(ps, axis=2)
    return Inputs(_to_dtype(q, s.dtype), _to_dtype(k, s.dtype), _to_dtype(v, s.dtype), pairs, ())


def make_on_device(B, H, n_qframes, n_kframes, tpf, bs, d, dtype, seed, device,
                   pools: Sequence[Sequence[int]]):
    """Timing-only inputs drawn on the device with torch's generator.

    Same recipe and distributions as `make`, but a different random stream, so the
    values are not those of `make` for the same seed. `pools` gives one planting pool
    per chunk of `n_qframes // len(pools)` query frames. Used where host generation of
    gigabytes of normals would dominate a run (the 30-layer sweep); never used for
    parity.
    """
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    lens = torch.as_tensor(_block_lens(tpf, bs), device=device)
    nb = lens.numel()
    f32 = torch.float32
    c = torch.randn((B, H, n_kframes, d), generator=g, device=device, dtype=f32)
    u = c[:, :, :, None, :] + 0.5 * torch.randn((B, H, n_kframes, nb, d), generator=g, device=device, dtype=f32)
    tok = torch.repeat_interleave(u, lens, dim=3).reshape(B, H, n_kframes * tpf, d)
    del u
    k = (tok + torch.randn(tok.shape, generator=g, device=device, dtype=f32)).to(_TORCH_DTYPE[dtype])
    v = (tok + torch.randn(tok.shape, generator=g, device=device, dtype=f32)).to(_TORCH_DTYPE[dtype])
    del tok
    fpc = n_qframes // len(pools)
    qs = []
    for pool in pools:
        pool_t = torch.as_tensor(list(pool), device=device)
        n_qb = fpc * nb
        order = torch.rand((B, H, n_qb, len(pool)), generator=g, device=device).argsort(dim=-1)[..., :2]
        pairs = pool_t[order]
        bi = torch.arange(B, device=device)[:, None, None]
        hi = torch.arange(H, device=device)[None, :, None]
        code = 0.5 * (c[bi, hi, pairs[..., 0]] + c[bi, hi, pairs[..., 1]])
        q = torch.repeat_interleave(code, lens.repeat(fpc), dim=2)
        qs.append(q + torch.randn(q.shape, generator=g, device=device, dtype=f32))
    q = torch.cat(qs, dim=2).to(_TORCH_DTYPE[dtype]).contiguous()
    return q, k.contiguous(), v.contiguous()
