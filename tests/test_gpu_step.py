"""GPU checks of the one-launch steady-state pooling calls against the separate calls they
fuse, bitwise: lf_pool_step against lf_pool of the queries, of the new key frames and of
the lagged frames (whose frame means it forms from the cached block means), and
lf_qk_prologue_step against two lf_qk_prologue calls (queries, new keys). Nothing of the
cache outside the new block means and the lagged frame means may be written."""
import numpy as np
import pytest
import torch

import synth
import sparse_attention_autoregressive_amd as lf
from support import log

pytestmark = pytest.mark.gpu


def _same(a, b):
    """Bitwise equal, NaN where the other is NaN."""
    return bool(((a == b) | (a.isnan() & b.isnan())).all())


def _setup(name, cap_extra=2):
    w = synth.WORKLOADS[name]
    x = synth.make(w)
    dev = torch.device("cuda")
    g = lf.Geom(w.B, w.H, w.d, w.tpf, w.bs)
    cap = w.n_kframes + cap_extra
    nb = lf.n_bpf(g)
    k_blk = torch.full((w.B, w.H, cap * nb, w.d), float("nan"), dtype=torch.float32, device=dev)
    k_frm = torch.full((w.B, w.H, cap, w.d), float("nan"), dtype=torch.float32, device=dev)
    return w, x, dev, g, nb, k_blk, k_frm


@pytest.mark.parametrize("name", ["tiny_fp32", "480p_chunk2of7", "480p_chunk7of7"])
def test_pool_step_equals_separate_calls(name):
    w, x, dev, g, nb, k_blk, k_frm = _setup(name)
    q, k = x.q.to(dev), x.k.to(dev)
    tpf, nq = w.tpf, w.n_qframes
    f_new = w.n_kframes - nq
    n_lag = min(nq, f_new)
    f_lag = f_new - n_lag
    # the lagged frames' block means come from an earlier step
    k_blk[:, :, f_lag * nb:f_new * nb] = lf.lf_pool(k[:, :, f_lag * tpf:f_new * tpf], g, n_lag)[0]
    before = k_blk.clone()
    log(f"[step] {name}: lf_pool_step, new frames [{f_new}, {w.n_kframes}), lagged [{f_lag}, {f_new})")
    q_blk = lf.lf_pool_step(q, k[:, :, f_new * tpf:], g, nq, nq, f_new, f_lag, n_lag, None, k_blk, k_frm)
    ref_q, _ = lf.lf_pool(q, g, nq, with_frames=False)
    ref_kb, ref_kf = lf.lf_pool(k[:, :, f_new * tpf:], g, nq)
    _, ref_lag = lf.lf_pool(k[:, :, f_lag * tpf:f_new * tpf], g, n_lag)
    torch.cuda.synchronize()
    assert torch.equal(q_blk, ref_q)
    assert torch.equal(k_blk[:, :, f_new * nb:w.n_kframes * nb], ref_kb)
    assert _same(k_blk[:, :, :f_new * nb], before[:, :, :f_new * nb]), "the history's block means changed"
    assert torch.isnan(k_blk[:, :, w.n_kframes * nb:]).all()
    if n_lag:
        assert torch.equal(k_frm[:, :, f_lag:f_new], ref_lag)
    assert torch.isnan(k_frm[:, :, :f_lag]).all() and torch.isnan(k_frm[:, :, f_new:]).all()
    # the frame means of the new frames, by a call with lagged frames only
    lf.lf_pool_step(None, None, g, 0, 0, 0, f_new, nq, None, k_blk, k_frm)
    torch.cuda.synchronize()
    assert torch.equal(k_frm[:, :, f_new:w.n_kframes], ref_kf)
    assert torch.isnan(k_frm[:, :, w.n_kframes:]).all()


def test_pool_step_keys_only_and_empty():
    """Keys only (a dense chunk: no pooled queries), and a call with nothing to do."""
    w, x, dev, g, nb, k_blk, k_frm = _setup("480p_chunk2of7")
    k = x.k.to(dev)
    tpf = w.tpf
    lf.lf_pool_step(None, k[:, :, :3 * tpf], g, 0, 3, 0, 0, 0, None, k_blk, k_frm)
    lf.lf_pool_step(None, None, g, 0, 0, 0, 0, 0, None, k_blk, k_frm)
    lf.lf_pool_step(None, k[:, :, 3 * tpf:6 * tpf], g, 0, 3, 3, 0, 3, None, k_blk, k_frm)
    ref_kb, ref_kf = lf.lf_pool(k[:, :, :6 * tpf], g, 6)
    torch.cuda.synchronize()
    assert torch.equal(k_blk[:, :, :6 * nb], ref_kb)
    assert torch.equal(k_frm[:, :, :3], ref_kf[:, :, :3])
    assert torch.isnan(k_frm[:, :, 3:]).all() and torch.isnan(k_blk[:, :, 6 * nb:]).all()


@pytest.mark.parametrize("name,lat_w", [("tiny_fp32", 8), ("480p_chunk2of7", 52), ("480p_chunk7of7", 52)])
def test_prologue_step_equals_separate_calls(name, lat_w):
    w, x, dev, g, nb, k_blk, k_frm = _setup(name)
    q, k = x.q.to(dev), x.k.to(dev)
    tpf, nq = w.tpf, w.n_qframes
    f_new = w.n_kframes - nq
    n_lag = min(nq, f_new)
    f_lag = f_new - n_lag
    rng = np.random.default_rng(91)
    gq = torch.from_numpy((1.0 + 0.1 * rng.standard_normal(w.d)).astype(np.float32)).to(dev)
    gk = torch.from_numpy((1.0 + 0.1 * rng.standard_normal(w.d)).astype(np.float32)).to(dev)
    k_new = k[:, :, f_new * tpf:].contiguous()               # the chunk's raw keys (pre-norm)
    # a KV cache with room for 2 more frames: the keys go to the chunk's frames
    kv = torch.full((w.B, w.H, (w.n_kframes + 2) * tpf, w.d), float("nan"), dtype=q.dtype, device=dev)
    kv[:, :, :f_new * tpf] = k[:, :, :f_new * tpf]
    k_blk[:, :, f_lag * nb:f_new * nb] = lf.lf_pool(k[:, :, f_lag * tpf:f_new * tpf], g, n_lag)[0]
    log(f"[step] {name}: lf_qk_prologue_step, frame0 {f_new}, lat_w {lat_w}")
    q_out, q_blk = lf.lf_qk_prologue_step(q, k_new, gq, gk, g, nq, f_new, lat_w, f_new, f_lag, n_lag,
                                          kv[:, :, f_new * tpf:w.n_kframes * tpf], k_blk, k_frm)
    ref_q, ref_qb, _ = lf.lf_qk_prologue(q, gq, g, nq, f_new, lat_w, with_frames=False)
    ref_k, ref_kb, ref_kf = lf.lf_qk_prologue(k_new, gk, g, nq, f_new, lat_w)
    _, ref_lag = lf.lf_pool(k[:, :, f_lag * tpf:f_new * tpf], g, n_lag)
    torch.cuda.synchronize()
    assert torch.equal(q_out, ref_q) and torch.equal(q_blk, ref_qb)
    assert torch.equal(kv[:, :, f_new * tpf:w.n_kframes * tpf], ref_k)
    assert torch.isnan(kv[:, :, w.n_kframes * tpf:]).all()
    assert torch.equal(k_blk[:, :, f_new * nb:w.n_kframes * nb], ref_kb)
    if n_lag:
        assert torch.equal(k_frm[:, :, f_lag:f_new], ref_lag)
    assert torch.isnan(k_frm[:, :, :f_lag]).all() and torch.isnan(k_frm[:, :, f_new:]).all()
    lf.lf_pool_step(None, None, g, 0, 0, 0, f_new, nq, None, k_blk, k_frm)
    torch.cuda.synchronize()
    assert torch.equal(k_frm[:, :, f_new:w.n_kframes], ref_kf)
