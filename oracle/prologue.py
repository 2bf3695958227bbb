"""CPU oracle for the query/key prologue that feeds pooling: RMSNorm over each head's
channels, then a 3-D rotary position embedding over (frame, row, column). TEST
INFRASTRUCTURE ONLY (imported by tests/, the smoke check and the benchmark's
CPU-baseline leg; shares no code with the HIP library).

The pages name RoPE and RMSNorm only as deployment kernels shipped with the released code
(Light Forcing summary, reproducibility paragraph); they define neither. Every step below
is therefore a reading (R27-R29), and the function is "parity unpinned" by the pages: it
is pinned instead by closed forms, invariants and a hand-worked case
(tests/test_oracle_prologue.py).

  R27  RMSNorm per token over the head dimension d: y = x / sqrt(mean(x^2) + eps) * gamma,
       gamma a learned vector of length d shared by all heads.
  R28  Rotary pairs are adjacent channels (2k, 2k+1). Of the d/2 pairs the first
       d/2 - 2*floor(d/6) rotate with the token's frame index, the next floor(d/6) with its
       row and the last floor(d/6) with its column in the latent frame (lat_h x lat_w
       tokens, row-major). Within an axis with n pairs, pair i turns by
       pos * theta^(-i/n), theta = 10000.
  R29  The rotation of a pair (a, b) by angle phi is (a cos phi - b sin phi,
       a sin phi + b cos phi); the frame index is the token's absolute frame in the clip.
"""
from __future__ import annotations

import numpy as np


def rope_split(d: int):
    """(temporal, row, column) pair counts for head dimension d (reading R28)."""
    n_hw = d // 6
    return d // 2 - 2 * n_hw, n_hw, n_hw


def rope_angles(frames: np.ndarray, rows: np.ndarray, cols: np.ndarray, d: int, theta: float = 10000.0):
    """Angles [tokens, d/2] of every rotary pair for tokens at the given positions."""
    n_t, n_h, n_w = rope_split(d)
    parts = []
    for pos, n in ((frames, n_t), (rows, n_h), (cols, n_w)):
        inv = theta ** (-np.arange(n, dtype=np.float64) / n)
        parts.append(np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :])
    return np.concatenate(parts, axis=1)


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """Reading R27, over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps) * np.asarray(gamma, dtype=np.float64)


def rotate(y: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Reading R29 on adjacent channel pairs; y [..., tokens, d], angles [tokens, d/2]."""
    a, b = y[..., 0::2], y[..., 1::2]
    c, s = np.cos(angles), np.sin(angles)
    out = np.empty_like(y)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def qk_prologue(x: np.ndarray, gamma: np.ndarray, *, tpf: int, lat_w: int, frame0: int, eps: float = 1e-6,
                theta: float = 10000.0) -> np.ndarray:
    """x [B, H, n_frames*tpf, d] (the chunk's queries or keys; frame f of x is frame
    frame0 + f of the clip) -> RMSNorm then RoPE, fp64."""
    x = np.asarray(x, dtype=np.float64)
    L, d = x.shape[-2], x.shape[-1]
    t = np.arange(L)
    frames = frame0 + t // tpf
    p = t % tpf
    ang = rope_angles(frames, p // lat_w, p % lat_w, d, theta)
    return rotate(rmsnorm(x, gamma, eps), ang)
