"""Host-side checks of the Chunk-Aware Growth sweep plan (30 layers x 7 chunks at 480p):
the library's schedule and per-chunk budgets equal the oracle's, the first chunk is
dense, and the realised block density meets the FLOP target."""
import numpy as np
import pytest

import oracle
import synth
import sparse_attention_autoregressive_amd as lf
from sparse_attention_autoregressive_amd.pipeline import plan_sweep

pytestmark = pytest.mark.skipif(not __import__("os").path.exists(lf.library_path()), reason="liblf.so not built")


def _plan():
    s = synth.SWEEP
    g = lf.Geom(s.B, s.H, s.d, s.tpf, s.bs)
    return s, plan_sweep(g, s.n_chunks, s.frames_per_chunk, s.k_f, s.T, s.s_base, s.s_target, s.d ** -0.5)


def test_schedule_and_budgets_match_oracle():
    s, sp = _plan()
    flops = [float(3 * s.tpf * 3 * i * s.tpf) for i in range(1, s.n_chunks + 1)]
    s_or, beta_or = oracle.cag_schedule(s.n_chunks, s.T, s.s_base, s.s_target, flops)
    assert np.allclose(sp.s, s_or, rtol=0, atol=1e-12) and abs(sp.beta - beta_or) < 1e-12
    nb = -(-s.tpf // s.bs)
    for i, p in enumerate(sp.chunks, 1):
        w = s.chunk(i)
        assert list(p.forced) == list(w.forced) and list(p.mem) == list(w.mem)
        W_f = len(w.forced) + min(w.k_f, len(w.mem))
        assert p.W_f == W_f
        assert p.k_b == oracle.block_budget(s_or[i - 1], w.n_kframes * nb, W_f, nb)


def test_first_chunk_dense_and_target_met():
    s, sp = _plan()
    assert sp.dense(1) and not any(sp.dense(i) for i in range(2, s.n_chunks + 1))
    p1 = sp.chunks[0]
    assert p1.W_b == p1.n_kframes * p1.n_bpf           # every key block listed
    # block-pair density over the schedule (every block of a frame counted once)
    pairs = sum(p.n_qb * p.W_b for p in sp.chunks)
    dense = sum(p.n_qb * p.n_kframes * p.n_bpf for p in sp.chunks)
    assert abs(1 - pairs / dense - s.s_target) < 5e-3, pairs / dense
    # budgets never shrink as the cache grows (CAG sparsity grows slower than the cache)
    kb = [p.k_b for p in sp.chunks[1:]]
    assert kb == sorted(kb)


def test_uniform_plan_matches_oracle_and_budget():
    """The uniform allocation (chunk 1 dense, one sparsity after it) from the library's
    CAG call with a constant alpha equals the oracle's closed form, keeps the same FLOP
    budget as CAG, and its per-chunk block budgets follow the same rule."""
    s = synth.SWEEP
    g = lf.Geom(s.B, s.H, s.d, s.tpf, s.bs)
    sp = plan_sweep(g, s.n_chunks, s.frames_per_chunk, s.k_f, s.T, s.s_base, s.s_target, s.d ** -0.5,
                    schedule="uniform")
    flops = np.array([float(3 * s.tpf * 3 * i * s.tpf) for i in range(1, s.n_chunks + 1)])
    s_or = oracle.uniform_schedule(s.n_chunks, s.s_target, flops)
    assert np.allclose(sp.s, s_or, rtol=0, atol=1e-12)
    assert sp.s[0] == 0.0 and np.ptp(sp.s[1:]) < 1e-12
    assert abs(np.dot(flops, 1 - np.asarray(sp.s)) - (1 - s.s_target) * flops.sum()) < 1e-9 * flops.sum()
    nb = -(-s.tpf // s.bs)
    for i, p in enumerate(sp.chunks, 1):
        w = s.chunk(i, schedule="uniform")
        W_f = len(w.forced) + min(w.k_f, len(w.mem))
        assert p.k_b == oracle.block_budget(s_or[i - 1], w.n_kframes * nb, W_f, nb)
    with pytest.raises(ValueError):
        plan_sweep(g, s.n_chunks, s.frames_per_chunk, s.k_f, s.T, s.s_base, s.s_target, s.d ** -0.5,
                   schedule="linear")
