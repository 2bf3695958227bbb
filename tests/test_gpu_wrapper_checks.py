"""The Python binding rejects id lists and pooled tensors of the wrong dtype or shape on
the host, before anything is enqueued: an int64 list (the oracle's own output dtype) or a
list, pooled-query tensor or output too short for the geometry would otherwise be read or
written past its end by the kernels."""
import pytest
import torch

import synth
import sparse_attention_autoregressive_amd as lf

pytestmark = pytest.mark.gpu


def _setup():
    w = synth.TINY
    dev = torch.device("cuda")
    g = lf.Geom(w.B, w.H, w.d, w.tpf, w.bs)
    nb = lf.n_bpf(g)
    n_qb, n_kb = w.n_qframes * nb, w.n_kframes * nb
    f32 = torch.float32
    q = torch.zeros((w.B, w.H, w.lq, w.d), dtype=f32, device=dev)
    kv = torch.zeros((w.B, w.H, w.lk, w.d), dtype=f32, device=dev)
    q_blk = torch.zeros((w.B, w.H, n_qb, w.d), dtype=f32, device=dev)
    k_blk = torch.zeros((w.B, w.H, n_kb, w.d), dtype=f32, device=dev)
    k_frm = torch.zeros((w.B, w.H, w.n_kframes, w.d), dtype=f32, device=dev)
    return w, g, n_qb, q, kv, q_blk, k_blk, k_frm


def test_sparse_attn_rejects_bad_lists():
    w, g, n_qb, q, kv, *_ = _setup()
    good = torch.zeros((w.B, w.H, n_qb, 4), dtype=torch.int32, device=q.device)
    out = torch.full_like(q, 7.0)
    for bad in (good.to(torch.int64),                       # the oracle's dtype
                good[:, :, :-1].contiguous(),                # one query block short
                good.reshape(w.B, w.H, -1),                  # flattened
                good[:, :1].contiguous()):                   # one head only
        with pytest.raises(ValueError):
            lf.lf_sparse_attn(q, kv, kv, g, w.n_qframes, w.n_kframes, bad, w.scale, out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a rejected call wrote its output"


def test_select_rejects_bad_buffers():
    w, g, n_qb, q, kv, q_blk, k_blk, k_frm = _setup()
    dev = q.device
    W_f = len(w.forced) + min(w.k_f, len(w.mem))
    W_b = W_f * min(w.k_b, lf.n_bpf(g))
    i32 = torch.int32
    with pytest.raises(ValueError):                          # pooled queries too short
        lf.lf_select(q_blk[:, :, :-1].contiguous(), k_frm, k_blk, g, n_qb, w.n_kframes, w.mem, w.forced,
                     w.k_f, w.k_b)
    with pytest.raises(ValueError):                          # list output one slot short
        lf.lf_select(q_blk, k_frm, k_blk, g, n_qb, w.n_kframes, w.mem, w.forced, w.k_f, w.k_b,
                     blocks_out=torch.zeros((w.B, w.H, n_qb, W_b - 1), dtype=i32, device=dev))
    with pytest.raises(ValueError):                          # frame output of the wrong dtype
        lf.lf_select(q_blk, k_frm, k_blk, g, n_qb, w.n_kframes, w.mem, w.forced, w.k_f, w.k_b,
                     frames_out=torch.zeros((w.B, w.H, n_qb, W_f), dtype=torch.int64, device=dev))
    with pytest.raises(ValueError):                          # frame lists as int64
        lf.lf_select_blocks(q_blk, k_blk, g, n_qb, w.n_kframes,
                            torch.zeros((w.B, w.H, n_qb, W_f), dtype=torch.int64, device=dev), w.k_b)
    with pytest.raises(ValueError):                          # frame-stage output too short
        lf.lf_select_frames(q_blk, k_frm, g, n_qb, w.n_kframes, w.mem, w.forced, w.k_f,
                            out=torch.zeros((w.B, w.H, n_qb - 1, W_f), dtype=i32, device=dev))
    with pytest.raises(ValueError):                          # single-level output too short
        lf.lf_select_blocks_1d(q_blk, k_blk, g, n_qb, w.n_kframes, 5,
                               out=torch.zeros((w.B, w.H, n_qb, 4), dtype=i32, device=dev))
    with pytest.raises(ValueError):                          # pooled queries of the wrong dtype
        lf.lf_pool_qk(q, kv, g, w.n_qframes, w.n_kframes, q_blk=q_blk.double())
