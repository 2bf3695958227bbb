"""GPU parity of the whole HSA path (C ABI -> HIP kernels) against the CPU oracle.

Workloads: the tiny fp32 case (every row, every output), the 480p chunk-2 and chunk-7
layers and the 69-frame LongLive-like layer at full size (masks on every row; attention
on a sample of rows that covers two whole heads, every ragged query block and random
rows), plus edge cases (ragged and 1-token blocks, d=64, dense lists, skipped ids,
empty memory set, k >= candidates) and bitwise determinism.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_attention_autoregressive_amd as lf
from support import (NEAR_TIE, compare_attention, compare_masks, lib_k_b, log, oracle_k_b, run_gpu,
                     run_oracle_masks, sample_rows)

pytestmark = pytest.mark.gpu

_cache = {}


def _case(name):
    """(workload, inputs, fp64 arrays, gpu results, oracle masks, k_b) -- computed once."""
    if name in _cache:
        return _cache[name]
    w = synth.WORKLOADS[name]
    log(f"[case] {name}: generating inputs")
    x = synth.make(w)
    q64, k64, v64 = x.np64()
    k_b = lib_k_b(w)
    assert k_b == oracle_k_b(w)
    gpu = run_gpu(w, x, k_b)
    log(f"[case] {name}: oracle masks")
    ref = run_oracle_masks(w, q64, k64, k_b)
    _cache[name] = (w, x, (q64, k64, v64), gpu, ref, k_b)
    return _cache[name]


ALL = ["tiny_fp32", "480p_chunk2of7", "480p_chunk7of7", "longlive_69f"]


@pytest.mark.parametrize("name", ALL)
def test_pool_parity(name):
    w, x, (q64, k64, v64), gpu, ref, k_b = _case(name)
    for key in ("q_blk", "k_blk", "k_frm"):
        e = ref[key]
        err = np.abs(gpu[key].astype(np.float64) - e).max() / np.abs(e).max()
        log(f"[pool] {name} {key}: max rel err {err:.2e}")
        assert err <= 2e-6, (key, err)


@pytest.mark.parametrize("name", ALL)
def test_mask_parity(name):
    w, x, (q64, k64, v64), gpu, ref, k_b = _case(name)
    nb = ref["n_bpf"]
    stats = compare_masks(gpu, ref, min(k_b, nb))
    log(f"[mask] {name}: {stats}")
    W_f = len(w.forced) + min(w.k_f, len(w.mem))
    assert gpu["frames"].shape[-1] == W_f
    # forced frames always present; every row's count is the budget
    fr = gpu["frames"].reshape(-1, W_f)
    for f in w.forced:
        assert (fr == f).any(axis=1).all()
    assert gpu["blocks"].shape[-1] == W_f * min(k_b, nb)
    assert stats["frame_ties"] + stats["block_ties"] <= max(2, stats["rows"] // 100)


@pytest.mark.parametrize("name", ALL)
def test_attention_parity(name):
    w, x, (q64, k64, v64), gpu, ref, k_b = _case(name)
    rows = sample_rows(w, gpu["frames"].shape[2], full=(w.H * gpu["frames"].shape[2] <= 1000 and w.n_kframes <= 8))
    res = compare_attention(w, gpu, q64, k64, v64, rows, w.dtype)
    log(f"[attn] {name}: {res}")


def test_planted_frames_recovered_on_gpu():
    w, x, _, gpu, _, _ = _case("longlive_69f")
    fr = gpu["frames"][0]
    hit = [set(x.pairs[0, h, r].tolist()) <= set(fr[h, r].tolist())
           for h in range(w.H) for r in range(fr.shape[1])]
    assert np.mean(hit) >= 0.99


def test_determinism_bitwise():
    w = synth.CHUNK7
    x = synth.make(w)
    dev = torch.device("cuda")
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    a = run_gpu(w, x, w.k_b, q, k, v)
    b = run_gpu(w, x, w.k_b, q, k, v)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


# ------------------------------------------------------------------------------ edge cases
def _edge(w, k_b=None, full=True):
    x = synth.make(w)
    q64, k64, v64 = x.np64()
    k_b = w.k_b if k_b is None else k_b
    gpu = run_gpu(w, x, k_b)
    ref = run_oracle_masks(w, q64, k64, k_b)
    stats = compare_masks(gpu, ref, min(k_b, ref["n_bpf"]))
    rows = sample_rows(w, gpu["frames"].shape[2], full=full)
    res = compare_attention(w, gpu, q64, k64, v64, rows, w.dtype)
    log(f"[edge] {w.name}: {stats} {res}")
    return x, gpu, ref


def _base(**kw):
    from dataclasses import replace
    w = replace(synth.CHUNK7, H=2, tpf=200, n_kframes=9, current=(6, 7, 8), sink=(0,), recent=(5,),
                mem=(1, 2, 3, 4), k_f=2, k_b=2, q_pool=(0, 1, 2, 3, 4), name="edge_base", seed=7001)
    return replace(w, **kw)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_edge_ragged_blocks(dtype):
    # 200 tokens per frame in blocks of 64 -> 64, 64, 64, 8; several tiles and a ragged tail
    _edge(_base(dtype=dtype, name=f"ragged_{dtype}"))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_edge_one_token_blocks(dtype):
    # 17 tokens per frame in blocks of 16 -> 16 + 1: 1-token query and key blocks
    _edge(_base(dtype=dtype, tpf=17, bs=16, k_b=1, name=f"onetoken_{dtype}", seed=7002))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_edge_head_dim_64(dtype):
    _edge(_base(dtype=dtype, d=64, bs=32, k_b=3, name=f"d64_{dtype}", seed=7003))


def test_edge_all_candidates_kept_equals_dense():
    # k_f >= |M| and k_b >= n_bpf: every block listed -> dense attention
    w = _base(k_f=9, k_b=9, name="dense_lists", seed=7004)
    x, gpu, ref = _edge(w)
    q64, k64, v64 = x.np64()
    dense = oracle.dense_attn(q64, k64, v64, w.scale)
    err = np.abs(gpu["o"] - dense).max()
    assert err <= 2e-2, err


def test_edge_first_chunk_no_memory():
    # chunk 1 under CAG: no history, the chunk's own frames forced, dense within them
    w = _base(n_kframes=3, current=(0, 1, 2), sink=(0,), recent=(), mem=(), k_f=4, k_b=25,
              q_pool=(0, 1, 2), name="first_chunk", seed=7005)
    _edge(w)


def test_edge_k_f_zero_and_batch():
    w = _base(B=2, k_f=0, name="kf0_batch2", seed=7006)
    _edge(w)


def test_edge_skipped_ids():
    # ids outside [0, n_kb) in a list are skipped: same as the list without them
    w = _base(name="skipped_ids", seed=7007)
    x = synth.make(w)
    dev = torch.device("cuda")
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    g = lf.Geom(w.B, w.H, w.d, w.tpf, w.bs)
    nb = lf.n_bpf(g)
    n_qb, n_kb = 3 * nb, w.n_kframes * nb
    rng = np.random.default_rng(0)
    lists = np.sort(np.stack([rng.choice(n_kb, 6, replace=False) for _ in range(w.H * n_qb)]), axis=1)
    noisy = lists.copy()
    noisy[:, 0] = -5
    noisy[:, 3] = n_kb + 7
    blk = torch.as_tensor(noisy.reshape(1, w.H, n_qb, 6), dtype=torch.int32, device=dev)
    o = lf.lf_sparse_attn(q, k, v, g, 3, w.n_kframes, blk, w.scale)
    keep = np.concatenate([lists[:, 1:3], lists[:, 4:]], axis=1).reshape(1, w.H, n_qb, 4)
    q64, k64, v64 = x.np64()
    ref = oracle.sparse_attn(q64, k64, v64, keep, w.tpf, w.bs, w.scale)
    assert np.abs(o.float().cpu().numpy() - ref).max() <= 2e-2


@pytest.mark.parametrize("hot_key", [8.0, 32.0])
def test_edge_fixed_reference_redo(hot_key):
    # The attention kernel first weights a row against each query's maximum over the row's
    # first tile. Here one listed block scores far above that. Queries 0.5 and the block's
    # keys 8.0 give 0.5 * 8 * 128 / sqrt(128) ~ 45 nats (~65 log2 units: a row sum near
    # 2^68, past the fixed-reference limit of 2^64); keys 32.0 give ~260 log2 units (the
    # fixed-reference weights overflow fp32). Either way the row is redone with the running
    # maximum. Head 0's rows list that block after an ordinary one; head 1's rows do not.
    # Both match the oracle.
    w = _base(name=f"redo_{hot_key:g}", seed=7012)
    x = synth.make(w)
    dev = torch.device("cuda")
    g = lf.Geom(w.B, w.H, w.d, w.tpf, w.bs)
    nb = lf.n_bpf(g)
    n_qb = 3 * nb
    hot = 5 * nb + 1                                   # a full 64-token block of frame 5
    tok0 = 5 * w.tpf + w.bs
    q = torch.full_like(x.q, 0.5)
    k = x.k.clone()
    k[:, :, tok0:tok0 + w.bs] = hot_key
    lists = np.zeros((1, w.H, n_qb, 3), dtype=np.int32)
    lists[0, 0] = [0, 3, hot]
    lists[0, 1] = [1, 2, 7]
    blk = torch.as_tensor(lists, device=dev)
    o = lf.lf_sparse_attn(q.to(dev), k.to(dev), x.v.to(dev), g, 3, w.n_kframes, blk, w.scale)
    q64 = q.double().numpy()
    k64 = k.double().numpy()
    v64 = x.v.double().numpy()
    ref = oracle.sparse_attn(q64, k64, v64, lists, w.tpf, w.bs, w.scale)
    got = o.float().cpu().numpy()
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max()
    log(f"[edge] fixed-reference redo (keys {hot_key:g}): max abs err {err:.3e}")
    assert err <= 2e-2, err


def test_edge_constant_values():
    # constant V -> every output equals that constant, up to one bf16 ulp (P is rounded
    # to bf16 for the matrix cores, the normaliser is summed in fp32)
    w = _base(name="constV", seed=7008)
    x = synth.make(w)
    dev = torch.device("cuda")
    v = torch.full_like(x.v, 0.8125).to(dev)           # exactly representable in bf16
    gpu = run_gpu(w, x, w.k_b, v=v)
    assert np.abs(gpu["o"] - 0.8125).max() <= 2.0 ** -8


@pytest.mark.parametrize("name", ["tiny_fp32", "480p_chunk7of7", "longlive_69f"])
def test_separate_select_calls_equal_fused(name):
    """lf_select_frames then lf_select_blocks give bitwise the lists of the fused lf_select
    (which the pipeline runs), with and without writing T_r."""
    w, x, _, gpu, _, k_b = _case(name)
    dev = torch.device("cuda")
    g = lf.Geom(w.B, w.H, w.d, w.tpf, w.bs)
    nb = lf.n_bpf(g)
    n_qb = w.n_qframes * nb
    q_blk, k_frm = (torch.from_numpy(gpu[k]).to(dev) for k in ("q_blk", "k_frm"))
    k_blk = torch.from_numpy(gpu["k_blk"]).to(dev)
    frames = lf.lf_select_frames(q_blk, k_frm, g, n_qb, w.n_kframes, w.mem, w.forced, w.k_f)
    blocks = lf.lf_select_blocks(q_blk, k_blk, g, n_qb, w.n_kframes, frames, k_b)
    _, blocks2 = lf.lf_select(q_blk, k_frm, k_blk, g, n_qb, w.n_kframes, w.mem, w.forced, w.k_f, k_b,
                              with_frames=False)
    torch.cuda.synchronize()
    assert np.array_equal(frames.cpu().numpy(), gpu["frames"])
    assert np.array_equal(blocks.cpu().numpy(), gpu["blocks"])
    assert np.array_equal(blocks2.cpu().numpy(), gpu["blocks"])


def test_select_blocks_malformed_frames_stay_in_bounds():
    """Frame ids outside [0, n_kframes) in the input of lf_select_blocks are clamped by the
    kernel: the call completes and every listed id is a valid block id (the contract only
    promises in-bounds behaviour for such rows)."""
    w, x, _, gpu, _, k_b = _case("480p_chunk7of7")
    dev = torch.device("cuda")
    g = lf.Geom(w.B, w.H, w.d, w.tpf, w.bs)
    nb = lf.n_bpf(g)
    frames = torch.from_numpy(gpu["frames"]).to(dev)
    frames[..., 0] = -5
    frames[..., -1] = 10 ** 6
    q_blk, k_blk = (torch.from_numpy(gpu[k]).to(dev) for k in ("q_blk", "k_blk"))
    blocks = lf.lf_select_blocks(q_blk, k_blk, g, w.n_qframes * nb, w.n_kframes, frames.contiguous(), k_b)
    torch.cuda.synchronize()
    b = blocks.cpu().numpy()
    assert b.min() >= 0 and b.max() < w.n_kframes * nb


@pytest.mark.parametrize("name", ["tiny_fp32", "480p_chunk2of7"])
def test_pool_qk_equals_separate_pools(name):
    """The combined query + key pooling launch (the pipeline's) gives bitwise the block and
    frame means of two lf_pool calls."""
    w, x, _, gpu, _, k_b = _case(name)
    dev = torch.device("cuda")
    g = lf.Geom(w.B, w.H, w.d, w.tpf, w.bs)
    q, k = x.q.to(dev), x.k.to(dev)
    q_blk, _ = lf.lf_pool(q, g, w.n_qframes, with_frames=False)
    k_blk, k_frm = lf.lf_pool(k, g, w.n_kframes)
    q2, k2, f2 = lf.lf_pool_qk(q, k, g, w.n_qframes, w.n_kframes)
    torch.cuda.synchronize()
    assert torch.equal(q_blk, q2) and torch.equal(k_blk, k2) and torch.equal(k_frm, f2)
    assert np.array_equal(q2.cpu().numpy(), gpu["q_blk"]) and np.array_equal(f2.cpu().numpy(), gpu["k_frm"])


@pytest.mark.parametrize("name", ALL)
def test_one_level_selection_parity(name):
    """Single-level block top-K over the whole prefix at the HSA budget (K = W_b): every
    row's list equals the oracle's (fp64 scores of the oracle's pooling) except where the
    oracle's cut is a near-tie, lists are ascending, and attention over the GPU's lists
    matches the oracle's attention over the same lists."""
    w, x, (q64, k64, v64), gpu, ref, k_b = _case(name)
    dev = torch.device("cuda")
    g = lf.Geom(w.B, w.H, w.d, w.tpf, w.bs)
    nb = lf.n_bpf(g)
    n_qb = w.n_qframes * nb
    K = gpu["blocks"].shape[-1]
    q_blk, k_blk = (torch.from_numpy(gpu[k]).to(dev) for k in ("q_blk", "k_blk"))
    got = lf.lf_select_blocks_1d(q_blk, k_blk, g, n_qb, w.n_kframes, K)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    want, gaps = oracle.select_blocks_1d(ref["q_blk"], ref["k_blk"], K)
    rows_g, rows_w = got.reshape(-1, K), want.reshape(-1, K)
    diff = ~(rows_g == rows_w).all(axis=1)
    bad = np.nonzero(diff & ~(gaps.reshape(-1) < NEAR_TIE))[0]
    log(f"[1d] {name}: K={K}, {int(diff.sum())} near-tie rows of {len(rows_g)}")
    assert len(bad) == 0, (bad[:5], rows_g[bad[0]], rows_w[bad[0]])
    assert (np.diff(rows_g, axis=1) > 0).all() and rows_g.min() >= 0 and rows_g.max() < w.n_kframes * nb
    x_dev = [t.to(dev) for t in (x.q, x.k, x.v)]
    o = lf.lf_sparse_attn(*x_dev, g, w.n_qframes, w.n_kframes, torch.from_numpy(got).to(dev), w.scale)
    torch.cuda.synchronize()
    rows = sample_rows(w, n_qb, full=(name == "tiny_fp32"))
    st = compare_attention(w, dict(blocks=got, o=o.float().cpu().numpy()), q64, k64, v64, rows, w.dtype)
    log(f"[1d] {name}: attention {st}")


@pytest.mark.parametrize("name,frame0,lat_w", [("tiny_fp32", 4, 8), ("tiny_fp32", 4, 2), ("480p_chunk2of7", 3, 52),
                                               ("480p_chunk7of7", 18, 52)])
def test_prologue_parity(name, frame0, lat_w):
    """RMSNorm + rotary prologue fused with pooling, on the chunk's queries: the output
    against the oracle (within one step of the stored type, plus fp32 error), and the fused
    block and frame means equal lf_pool of the output bitwise (and the oracle's pooling of
    it within the pooling bound)."""
    from oracle.prologue import qk_prologue
    w = synth.WORKLOADS[name]
    x = synth.make(w)
    dev = torch.device("cuda")
    g = lf.Geom(w.B, w.H, w.d, w.tpf, w.bs)
    rng = np.random.default_rng(77)
    gamma_np = (1.0 + 0.1 * rng.standard_normal(w.d)).astype(np.float32)
    gamma = torch.from_numpy(gamma_np).to(dev)
    q = x.q.to(dev)
    log(f"[prologue] {name}: frame0 {frame0}, lat_w {lat_w}")
    y, blk, frm = lf.lf_qk_prologue(q, gamma, g, w.n_qframes, frame0, lat_w)
    blk2, frm2 = lf.lf_pool(y, g, w.n_qframes)
    torch.cuda.synchronize()
    assert torch.equal(blk, blk2) and torch.equal(frm, frm2)
    q64, _, _ = x.np64()
    ref = qk_prologue(q64, gamma_np.astype(np.float64), tpf=w.tpf, lat_w=lat_w, frame0=frame0, eps=1e-6)
    got = y.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    if w.dtype == "bf16":
        # one bf16 step of the value: the fp32 result (within ~1e-6 of exact) rounds to the
        # nearest bf16, or to the next one when it lies within that error of a midpoint
        bound = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7) + 1e-5
    else:
        bound = 1e-5 * np.maximum(np.abs(ref), 1.0)
    log(f"[prologue] {name}: max abs err {err.max():.3e}, worst err/bound {(err / bound).max():.3f}")
    assert (err <= bound).all()
    pooled = oracle.pool_blocks(got, w.n_qframes, w.tpf, w.bs)
    rel = np.abs(blk.cpu().numpy() - pooled).max() / np.abs(pooled).max()
    assert rel <= 2e-6, rel


def test_prologue_into_cache_view_equals_packed():
    """The prologue reading a token-range view and writing into a token-range view of a
    larger cache (different head strides on the two sides) gives bitwise the packed
    results, and writes nothing outside its frames."""
    w = synth.WORKLOADS["480p_chunk2of7"]
    x = synth.make(w)
    dev = torch.device("cuda")
    g = lf.Geom(w.B, w.H, w.d, w.tpf, w.bs)
    gamma = torch.from_numpy((1.0 + 0.1 * np.random.default_rng(5).standard_normal(w.d)).astype(np.float32)).to(dev)
    k = x.k.to(dev)                                       # 6 frames; prologue of frames 3..5
    f0, n = 3, 3
    src = k[:, :, f0 * w.tpf:]
    y, blk, frm = lf.lf_qk_prologue(src.contiguous(), gamma, g, n, f0, 52)
    cache = torch.full((w.B, w.H, 10 * w.tpf, w.d), float("nan"), dtype=k.dtype, device=dev)
    view = cache[:, :, f0 * w.tpf:(f0 + n) * w.tpf]
    y2, blk2, frm2 = lf.lf_qk_prologue(src, gamma, g, n, f0, 52, x_out=view)
    torch.cuda.synchronize()
    assert torch.equal(y, view) and torch.equal(blk, blk2) and torch.equal(frm, frm2)
    assert torch.isnan(cache[:, :, :f0 * w.tpf]).all() and torch.isnan(cache[:, :, (f0 + n) * w.tpf:]).all()


def test_edge_lists_longer_than_one_segment():
    # 312 listed blocks per row (13 per frame x 24 frames, every candidate kept): the
    # attention kernel stages lists 256 blocks at a time, so this walks two segments;
    # with every block listed the result is dense attention
    w = _base(tpf=200, bs=16, n_kframes=24, current=(21, 22, 23), sink=(0,), recent=(20,),
              mem=tuple(range(1, 20)), k_f=19, k_b=13, q_pool=tuple(range(0, 20)), name="two_segments", seed=7010)
    x, gpu, ref = _edge(w, full=False)
    assert gpu["blocks"].shape[-1] == 24 * 13
    q64, k64, v64 = x.np64()
    dense = oracle.dense_attn(q64, k64, v64, w.scale)
    assert np.abs(gpu["o"] - dense).max() <= 2e-2


def test_edge_maximum_frame_count():
    # 256 key frames (the most the listed frame stage takes; beyond, the long-history path,
    # tests/test_gpu_long_history.py) of one 16-token block each; 252 memory frames ranked
    # per row
    w = _base(tpf=16, bs=16, n_kframes=256, current=(253, 254, 255), sink=(0,), recent=(252,),
              mem=tuple(range(1, 252)), k_f=8, k_b=1, q_pool=tuple(range(0, 252)), name="max_frames", seed=7011)
    _edge(w)
