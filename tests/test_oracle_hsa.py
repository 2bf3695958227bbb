"""Pins for the oracle's pooling, two-level selection and block-sparse attention.

Light Forcing summary (paper.rainbus.top), execution flow, stages 2-3: block-level mean
pooling of q and k, frame-level pooling of the memory-set keys, frame relevance
p_r = <q~_r, k^_M> with top-k frames (sink, recent and current frames always kept),
block relevance o_r(tau, j) = <q~_r, k~_j^(tau)> with top-k blocks per selected frame,
the block mask B_r and block-sparse attention over it.

Each pin is independent of the oracle's own code: a hand-worked example, brute-force
subset enumeration, torch's scaled_dot_product_attention (a library routine, fp64),
closed forms, and invariants the pages fix.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import synth


# ----------------------------------------------------------------------------- hand example
GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    for line in open(__import__("os").path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].split()
        if line:
            vals[line[0]] = [float(x) for x in line[1:]]
    return vals


def test_hand_worked_example():
    """The hand-derived example in tests/golden/hand_worked_hsa.txt: T_r, block lists and
    frame means, plus the attention outputs in closed form."""
    g = _golden("hand_worked_hsa.txt")
    d, tpf = int(g["d"][0]), int(g["tpf"][0])
    K = np.array(g["K"]).reshape(1, 1, -1, d)
    Q = np.array(g["Q"]).reshape(1, 1, -1, d)
    V = np.stack([np.arange(K.shape[2], dtype=float), np.ones(K.shape[2])], axis=1)[None, None]
    c = 1 / math.sqrt(2)
    out = oracle.hsa(Q, K, V, tpf=tpf, bs=int(g["bs"][0]), n_kframes=int(g["n_kframes"][0]),
                     mem=[int(x) for x in g["mem"]], forced=[int(x) for x in g["forced"]],
                     k_f=int(g["k_f"][0]), k_b=int(g["k_b"][0]), scale=c)
    n_q = Q.shape[2]
    assert out["frames"][0, 0].tolist() == np.array(g["frames"], int).reshape(n_q, -1).tolist()
    assert out["blocks"][0, 0].tolist() == np.array(g["blocks"], int).reshape(n_q, -1).tolist()
    assert np.allclose(out["k_frm"][0, 0], np.array(g["frame_means"]).reshape(-1, d), atol=0)
    # p_r over M = {1, 2}, o_r over each frame of T_r, and the dense mask B_r
    mem = [int(x) for x in g["mem"]]
    for r in range(n_q):
        assert oracle.frame_scores(out["q_blk"], out["k_frm"], 0, 0, r, mem).tolist() == g[f"frame_scores_r{r}"]
        got = [oracle.block_scores(out["q_blk"], out["k_blk"], 0, 0, r, tau, out["n_bpf"]).tolist()
               for tau in out["frames"][0, 0, r]]
        assert sum(got, []) == g[f"block_scores_r{r}"]
    n_kb = int(g["n_kframes"][0]) * out["n_bpf"]
    mask = oracle.block_mask(out["blocks"], n_kb)
    assert mask[0, 0].astype(int).reshape(-1).tolist() == [int(x) for x in g["mask"]]
    e1, e2 = math.exp(c), math.exp(2 * c)
    den = 2 * e1 + e2
    assert out["o"][0, 0, 0].tolist() == pytest.approx([(2 * e2 + 6 * e1) / den, 1.0], abs=1e-14)
    assert out["o"][0, 0, 1].tolist() == pytest.approx([(7 * e1 + 4 * e2) / den, 1.0], abs=1e-14)


# ----------------------------------------------------------------------------- pooling
def test_pool_closed_forms():
    rng = np.random.default_rng(1)
    tpf, bs, nf, d = 40, 16, 3, 5                  # blocks of 16, 16, 8 tokens
    x = np.broadcast_to(rng.standard_normal(d), (2, 3, nf * tpf, d)).copy()
    assert np.allclose(oracle.pool_blocks(x, nf, tpf, bs), x[:, :, :1], atol=1e-15)
    assert np.allclose(oracle.pool_frames(x, nf, tpf), x[:, :, :1], atol=1e-15)
    # a ramp x_t = t: block mean = start + (len - 1)/2
    ramp = np.arange(nf * tpf, dtype=float)[None, None, :, None]
    blk = oracle.pool_blocks(ramp, nf, tpf, bs)[0, 0, :, 0]
    want = [f * tpf + s + (l - 1) / 2 for f in range(nf) for s, l in ((0, 16), (16, 16), (32, 8))]
    assert np.allclose(blk, want, atol=1e-12)
    # frame mean = length-weighted mean of its block means (not their plain mean)
    y = rng.standard_normal((1, 2, nf * tpf, d))
    kb = oracle.pool_blocks(y, nf, tpf, bs).reshape(1, 2, nf, 3, d)
    w = np.array([16, 16, 8])[None, None, None, :, None]
    assert np.allclose((kb * w).sum(axis=3) / tpf, oracle.pool_frames(y, nf, tpf), atol=1e-13)
    assert not np.allclose(kb.mean(axis=3), oracle.pool_frames(y, nf, tpf), atol=1e-3)


def test_pool_brute_force_loops():
    rng = np.random.default_rng(2)
    tpf, bs, nf, d = 12, 5, 2, 3
    x = rng.standard_normal((1, 1, nf * tpf, d))
    blk = oracle.pool_blocks(x, nf, tpf, bs)
    g = 0
    for f in range(nf):
        t = 0
        while t < tpf:
            n = min(bs, tpf - t)
            acc = [0.0] * d
            for u in range(n):
                for c in range(d):
                    acc[c] += x[0, 0, f * tpf + t + u, c]
            assert blk[0, 0, g].tolist() == pytest.approx([a / n for a in acc], abs=1e-14)
            g += 1
            t += bs


# ----------------------------------------------------------------------------- selection
def _best_subset(scores, ids, k):
    """Lexicographically smallest k-subset maximising the summed score (= top-k with a
    lowest-index tie-break)."""
    best, best_sum = None, -math.inf
    for sub in itertools.combinations(sorted(ids), k):
        s = sum(scores[i] for i in sub)
        if s > best_sum + 1e-12:
            best, best_sum = sub, s
    return list(best)


def test_frame_and_block_selection_brute_force():
    rng = np.random.default_rng(3)
    d, tpf, bs, nf = 4, 12, 4, 7                    # n_bpf = 3
    n_bpf = 3
    for trial in range(20):
        q_blk = rng.standard_normal((1, 2, 4, d))
        k_blk = rng.standard_normal((1, 2, nf * n_bpf, d))
        k_frm = rng.standard_normal((1, 2, nf, d))
        if trial % 4 == 0:                          # exact ties
            k_frm[..., 2, :] = k_frm[..., 1, :]
            k_blk[..., 4, :] = k_blk[..., 3, :]
        mem, forced = [1, 2, 3, 4], [0, 5, 6]
        for k_f in range(0, 6):
            frames, gaps = oracle.select_frames(q_blk, k_frm, mem, forced, k_f)
            for h in range(2):
                for r in range(4):
                    p = {f: float(k_frm[0, h, f] @ q_blk[0, h, r]) for f in mem}
                    want = sorted(forced + _best_subset(p, mem, min(k_f, 4)))
                    assert frames[0, h, r].tolist() == want
        for k_b in (1, 2, 3, 9):
            frames, _ = oracle.select_frames(q_blk, k_frm, mem, forced, 2)
            blocks, _ = oracle.select_blocks(q_blk, k_blk, frames, n_bpf, k_b)
            for h in range(2):
                for r in range(4):
                    want = []
                    for tau in frames[0, h, r]:
                        o = {j: float(k_blk[0, h, tau * n_bpf + j] @ q_blk[0, h, r]) for j in range(n_bpf)}
                        want += [tau * n_bpf + j for j in _best_subset(o, range(n_bpf), min(k_b, n_bpf))]
                    assert blocks[0, h, r].tolist() == want


def test_selection_invariants_and_gaps():
    rng = np.random.default_rng(4)
    n_bpf = 5
    q_blk = rng.standard_normal((2, 3, 6, 8))
    k_frm = rng.standard_normal((2, 3, 12, 8))
    k_blk = rng.standard_normal((2, 3, 12 * n_bpf, 8))
    mem, forced = list(range(2, 9)), [0, 1, 9, 10, 11]
    frames, fg = oracle.select_frames(q_blk, k_frm, mem, forced, 3)
    assert frames.shape[-1] == 5 + 3
    for row in frames.reshape(-1, 8):
        assert set(forced) <= set(row.tolist())          # always-kept frames present
        assert list(row) == sorted(set(row.tolist()))    # ascending, unique
    assert np.all(fg > 0)                                # distinct random scores
    blocks, bg = oracle.select_blocks(q_blk, k_blk, frames, n_bpf, 2)
    assert blocks.shape[-1] == 8 * 2                     # |J_r(tau)| = min(k_b, n_bpf)
    for row, fr in zip(blocks.reshape(-1, 16), frames.reshape(-1, 8)):
        assert list(row) == sorted(set(row.tolist()))
        assert sorted(set((row // n_bpf).tolist())) == fr.tolist()
    # k_b >= n_bpf keeps every block of each selected frame; gaps are then infinite
    blocks, bg = oracle.select_blocks(q_blk, k_blk, frames, n_bpf, 7)
    assert np.all(np.isinf(bg))
    for row, fr in zip(blocks.reshape(-1, 40), frames.reshape(-1, 8)):
        assert row.tolist() == [f * n_bpf + j for f in fr for j in range(n_bpf)]
    # k_f >= |M| keeps every frame
    frames, fg = oracle.select_frames(q_blk, k_frm, mem, forced, 50)
    assert np.all(frames == np.arange(12)) and np.all(np.isinf(fg))


def test_fixed_width_independent_of_history_length():
    # Per-row cost is fixed for fixed k_f, k_b and forced frames, whatever |M| is
    # (gist.science technical summary, section 2.2).
    rng = np.random.default_rng(5)
    widths = set()
    for n_hist in (6, 20, 60):
        nf = n_hist + 3
        q_blk = rng.standard_normal((1, 1, 3, 4))
        k_frm = rng.standard_normal((1, 1, nf, 4))
        k_blk = rng.standard_normal((1, 1, nf * 4, 4))
        forced = [0, nf - 3, nf - 2, nf - 1]
        frames, _ = oracle.select_frames(q_blk, k_frm, list(range(1, nf - 3)), forced, 4)
        blocks, _ = oracle.select_blocks(q_blk, k_blk, frames, 4, 2)
        widths.add(blocks.shape[-1])
    assert widths == {16}


def test_planted_frames_are_retrieved():
    """Planted relevance on the LongLive-like recipe (2 heads to stay quick): each query
    block is built from two planted frames' codes, whose frame scores sit about d/2
    above the rest, so both must be in T_r for >= 99% of rows. A sign or operand slip
    in the frame stage fails this."""
    w = synth.LONGLIVE
    w2 = type(w)(**{**w.__dict__, "H": 2})
    x = synth.make(w2)
    q, k, _ = x.np64()
    out = oracle.hsa(q, k, k, tpf=w2.tpf, bs=w2.bs, n_kframes=w2.n_kframes, mem=w2.mem,
                     forced=w2.forced, k_f=w2.k_f, k_b=w2.k_b, scale=w2.scale, with_attn=False)
    fr = out["frames"]
    hit = [set(x.pairs[0, h, r].tolist()) <= set(fr[0, h, r].tolist())
           for h in range(2) for r in range(fr.shape[2])]
    assert np.mean(hit) >= 0.99


# ----------------------------------------------------------------------------- attention
def _sdpa64(q, k, v, mask=None, scale=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else t(mask), scale=scale).numpy()


def test_dense_equals_library_sdpa():
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((1, 2, n, 16)) for n in (24, 40, 40))
    assert np.abs(oracle.dense_attn(q, k, v, 0.25) - _sdpa64(q, k, v, scale=0.25)).max() < 1e-12


def test_zero_sparsity_selection_equals_dense():
    # k_f >= |M| and k_b >= n_bpf select every block: HSA must then equal dense attention.
    rng = np.random.default_rng(7)
    tpf, bs, nf, d = 20, 8, 5, 16
    q = rng.standard_normal((1, 2, 2 * tpf, d))
    k = rng.standard_normal((1, 2, nf * tpf, d))
    v = rng.standard_normal((1, 2, nf * tpf, d))
    out = oracle.hsa(q, k, v, tpf=tpf, bs=bs, n_kframes=nf, mem=[1, 2], forced=[0, 3, 4],
                     k_f=9, k_b=9, scale=0.25)
    assert np.abs(out["o"] - _sdpa64(q, k, v, scale=0.25)).max() < 1e-12


def test_sparse_equals_library_masked_sdpa():
    # B_r expanded to a token mask as a boolean attn_mask of the library routine.
    w = synth.TINY
    x = synth.make(w)
    q, k, v = x.np64()
    out = oracle.hsa(q, k, v, tpf=w.tpf, bs=w.bs, n_kframes=w.n_kframes, mem=w.mem,
                     forced=w.forced, k_f=w.k_f, k_b=w.k_b, scale=w.scale)
    n_kb = w.n_kframes * out["n_bpf"]
    bmask = oracle.block_mask(out["blocks"], n_kb)
    tok_mask = np.zeros((1, w.H, w.lq, w.lk), dtype=bool)
    for h in range(w.H):
        for r in range(out["blocks"].shape[2]):
            qt = oracle.block_tokens(r, w.tpf, w.bs)
            for g in range(n_kb):
                if bmask[0, h, r, g]:
                    kt = oracle.block_tokens(g, w.tpf, w.bs)
                    tok_mask[0, h, qt[:, None], kt[None, :]] = True
    assert tok_mask.sum() < tok_mask.size                              # really sparse
    ref = _sdpa64(q, k, v, mask=tok_mask, scale=w.scale)
    assert np.abs(out["o"] - ref).max() < 1e-12


def test_block_mask_round_trip():
    """B_r as a dense mask holds exactly the listed ids: per row, its set positions are the
    row's (ascending, unique) list and its count is the list width."""
    rng = np.random.default_rng(9)
    n_kb, W = 40, 7
    lists = np.sort(np.stack([rng.choice(n_kb, W, replace=False) for _ in range(2 * 3 * 5)]), axis=1)
    blocks = lists.reshape(2, 3, 5, W)
    m = oracle.block_mask(blocks, n_kb)
    assert m.shape == (2, 3, 5, n_kb) and (m.sum(axis=-1) == W).all()
    for b in range(2):
        for h in range(3):
            for r in range(5):
                assert np.nonzero(m[b, h, r])[0].tolist() == blocks[b, h, r].tolist()


def test_attention_closed_forms():
    rng = np.random.default_rng(8)
    tpf, bs, d = 16, 4, 8
    q = rng.standard_normal((1, 1, tpf, d))
    k = rng.standard_normal((1, 1, 3 * tpf, d))
    blocks = np.array([[[[0, 5, 9]] * 4]])                            # 4 query blocks
    kt = np.concatenate([oracle.block_tokens(g, tpf, bs) for g in (0, 5, 9)])
    # constant V -> that constant
    v = np.broadcast_to(rng.standard_normal(d), (1, 1, 3 * tpf, d)).copy()
    o = oracle.sparse_attn(q, k, v, blocks, tpf, bs, 0.3)
    assert np.allclose(o, v[:, :, :tpf], atol=1e-14)
    # Q = 0 -> uniform weights: the mean of the selected values
    v = rng.standard_normal((1, 1, 3 * tpf, d))
    o = oracle.sparse_attn(np.zeros_like(q), k, v, blocks, tpf, bs, 0.3)
    assert np.allclose(o[0, 0], v[0, 0, kt].mean(axis=0), atol=1e-14)
    # one selected key token -> its value (1-token blocks)
    o = oracle.sparse_attn(q[:, :, :2], k, v, np.array([[[[7], [30]]]]), 1, 1, 0.3)
    assert np.allclose(o[0, 0, 0], v[0, 0, 7]) and np.allclose(o[0, 0, 1], v[0, 0, 30])


def test_attn_flops_counts():
    n_bpf = 3   # tpf 10, bs 4 -> 4, 4, 2
    blocks = np.array([[[[0, 2], [1, 5], [3, 4]]]])                   # 3 query blocks
    dense, active = oracle.attn_flops(blocks, 10, 4, 2)
    assert dense == 10 * 20
    assert active == 4 * (4 + 2) + 4 * (4 + 2) + 2 * (4 + 4)


def test_one_level_selection_pins():
    """Single-level block top-k: a worked case by hand (ties to the lower id), K at or
    above the block count keeps everything, brute force over all K-subsets on tiny
    inputs, and the reduction to HSA's block stage when the prefix is one frame."""
    q = np.zeros((1, 1, 1, 2))
    q[..., 0] = 1.0
    kb = np.zeros((1, 1, 4, 2))
    kb[0, 0, :, 0] = [0.5, 2.0, -1.0, 2.0]            # scores 0.5, 2, -1, 2
    blocks, gaps = oracle.select_blocks_1d(q, kb, 2)
    assert blocks.tolist() == [[[[1, 3]]]] and gaps[0, 0, 0] == 1.5
    assert oracle.select_blocks_1d(q, kb, 3)[0].tolist() == [[[[0, 1, 3]]]]
    assert oracle.select_blocks_1d(q, kb, 9)[0].tolist() == [[[[0, 1, 2, 3]]]]
    rng = np.random.default_rng(11)
    for _ in range(20):
        n_kb, d, K = int(rng.integers(3, 8)), 4, int(rng.integers(1, 5))
        q = rng.standard_normal((1, 1, 1, d))
        kb = rng.standard_normal((1, 1, n_kb, d))
        got = oracle.select_blocks_1d(q, kb, K)[0][0, 0, 0].tolist()
        s = kb[0, 0] @ q[0, 0, 0]
        best = max(itertools.combinations(range(n_kb), min(K, n_kb)), key=lambda c: (sum(s[list(c)]), [-i for i in c]))
        assert got == sorted(best)
    # one frame of n_bpf blocks: the same list as the block stage with T_r = {0}
    n_bpf, d = 6, 8
    q = rng.standard_normal((1, 2, 3, d))
    kb = rng.standard_normal((1, 2, n_bpf, d))
    frames = np.zeros((1, 2, 3, 1), dtype=np.int64)
    for K in (1, 3, 6):
        two, _ = oracle.select_blocks(q, kb, frames, n_bpf, K)
        one, _ = oracle.select_blocks_1d(q, kb, K)
        assert np.array_equal(one, two)
