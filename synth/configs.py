"""Workload table: the five seeded synthetic HSA workloads.

Pure data. Nothing here computes any part of the method (no pooling, scoring,
selection, schedule or attention arithmetic); the CPU oracle and the HIP path each
derive what they need from these parameters on their own.

Frame roles follow the Light Forcing summary (paper.rainbus.top, execution-flow
paragraph, stage 3): the sink frame(s), the most recent frame(s) and the current
chunk's frames are always kept; the remaining key frames form the memory set M from
which the top-k frames are retrieved per query block.

Shapes: 480p latent frames are 30x52 = 1560 tokens, a chunk is 3 latent frames, a
5-second clip is 7 chunks (21 latent frames); heads 12, head_dim 128, bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    """One chunk of one layer: queries of the current chunk against all key frames."""

    name: str
    B: int
    H: int
    d: int
    dtype: str                  # "fp32" or "bf16"
    tpf: int                    # tokens per latent frame
    bs: int                     # tokens per block (blocks are frame-aligned)
    n_kframes: int              # key/value frames (history + current chunk)
    current: Tuple[int, ...]    # the current chunk's frames (also the query frames)
    sink: Tuple[int, ...]
    recent: Tuple[int, ...]
    mem: Tuple[int, ...]        # memory set M (candidates for frame top-k)
    k_f: int                    # frames retrieved from M per query block
    k_b: Optional[int]          # blocks kept per selected frame; None -> from the CAG budget
    # Q planting: each query block's queries are the mean of the codes of two frames
    # drawn without replacement from this pool (None -> see planted_from).
    q_pool: Optional[Tuple[int, ...]] = None
    # Alternative planting: draw `planted_count` frames once from this range, then
    # draw each query block's pair from them.
    planted_from: Optional[Tuple[int, ...]] = None
    planted_count: int = 0
    # CAG parameters used when k_b is None (and reported otherwise).
    chunk_index: int = 1        # 1-based chunk number i
    n_chunks: int = 7
    T: int = 4                  # denoising steps
    s_base: float = 0.95
    s_target: float = 0.80
    seed: int = 0
    # Sparsity allocation over chunks: "cag" (Chunk-Aware Growth) or "uniform" (every
    # chunk after the first at one sparsity, same FLOP budget).
    schedule: str = "cag"

    @property
    def n_qframes(self) -> int:
        return len(self.current)

    @property
    def forced(self) -> Tuple[int, ...]:
        return tuple(sorted(set(self.sink) | set(self.recent) | set(self.current)))

    @property
    def scale(self) -> float:
        return 1.0 / float(self.d) ** 0.5

    @property
    def lq(self) -> int:
        return self.n_qframes * self.tpf

    @property
    def lk(self) -> int:
        return self.n_kframes * self.tpf


def _frames(a: int, b: int) -> Tuple[int, ...]:
    return tuple(range(a, b))


TINY = Workload(
    name="tiny_fp32", B=1, H=2, d=64, dtype="fp32", tpf=64, bs=32, n_kframes=7,
    current=(4, 5, 6), sink=(0,), recent=(3,), mem=(1, 2), k_f=1, k_b=1,
    q_pool=(0, 1, 2, 3), chunk_index=3, seed=1000,
)

CHUNK2 = Workload(
    name="480p_chunk2of7", B=1, H=12, d=128, dtype="bf16", tpf=1560, bs=64, n_kframes=6,
    current=(3, 4, 5), sink=(0,), recent=(), mem=(1, 2), k_f=4, k_b=None,
    q_pool=(0, 1, 2), chunk_index=2, s_target=0.80, seed=2000,
)

CHUNK7 = Workload(
    name="480p_chunk7of7", B=1, H=12, d=128, dtype="bf16", tpf=1560, bs=64, n_kframes=21,
    current=(18, 19, 20), sink=(0,), recent=(), mem=_frames(1, 18), k_f=4, k_b=8,
    q_pool=_frames(0, 18), chunk_index=7, s_target=0.80, seed=3000,
)

LONGLIVE = Workload(
    name="longlive_69f", B=1, H=12, d=128, dtype="bf16", tpf=1560, bs=64, n_kframes=69,
    current=(66, 67, 68), sink=(0, 1, 2), recent=(63, 64, 65), mem=_frames(3, 63),
    k_f=6, k_b=8, planted_from=_frames(3, 33), planted_count=6, chunk_index=7, seed=4000,
)


@dataclass(frozen=True)
class Sweep:
    """Full Chunk-Aware-Growth sweep: n_layers independent layers x n_chunks chunks.

    Each layer owns Q/K/V for all 3*n_chunks latent frames. Chunk i (1-based) queries
    frames 3i-3..3i-1 against the key prefix 0..3i-1; chunk 1 is dense.
    """

    name: str = "cag_sweep_7x30"
    n_layers: int = 30
    n_chunks: int = 7
    frames_per_chunk: int = 3
    B: int = 1
    H: int = 12
    d: int = 128
    dtype: str = "bf16"
    tpf: int = 1560
    bs: int = 64
    k_f: int = 4
    T: int = 4
    s_base: float = 0.95
    s_target: float = 0.85
    seed_base: int = 5000

    @property
    def n_frames(self) -> int:
        return self.n_chunks * self.frames_per_chunk

    def seed(self, layer: int) -> int:
        return self.seed_base + layer

    def chunk(self, i: int, layer: int = 0, schedule: str = "cag") -> Workload:
        """Workload of chunk i (1-based) in one layer; k_b left to the budget of the
        schedule ("cag" or "uniform")."""
        fpc = self.frames_per_chunk
        cur = _frames(fpc * (i - 1), fpc * i)
        mem = _frames(1, fpc * (i - 1)) if i > 1 else ()
        pool = _frames(0, fpc * (i - 1)) if i > 1 else cur
        return Workload(
            name=f"{self.name}_L{layer}_c{i}", B=self.B, H=self.H, d=self.d,
            dtype=self.dtype, tpf=self.tpf, bs=self.bs, n_kframes=fpc * i,
            current=cur, sink=(0,), recent=(), mem=mem, k_f=self.k_f, k_b=None,
            q_pool=pool, chunk_index=i, n_chunks=self.n_chunks, T=self.T,
            s_base=self.s_base, s_target=self.s_target, seed=self.seed(layer), schedule=schedule,
        )


SWEEP = Sweep()

WORKLOADS = {w.name: w for w in (TINY, CHUNK2, CHUNK7, LONGLIVE)}
