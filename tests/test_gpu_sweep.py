"""GPU parity of the Chunk-Aware Growth sweep (7 chunks of a 480p clip, 30 layers), run as
the sweep driver runs it: token-range views of per-layer Q/K/V/O tensors that hold the
whole clip.

Every layer runs twice: uncached (each chunk pools its whole key prefix) and in steady
state (a per-layer pooled-key cache: each chunk pools only its own key frames). For every
sparse chunk of every layer both runs' masks are compared with the oracle on every row;
the steady-state lists, pooled keys and outputs must equal the uncached ones bitwise.
Attention is compared with the oracle run on the GPU's own lists: every head of layers 0
and 29, one seeded head (all its rows) of every other layer; the dense first chunk is
checked to list every block. Layer 3 also runs the uniform allocation CAG is compared
against."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_attention_autoregressive_amd as lf
from sparse_attention_autoregressive_amd.pipeline import PooledKeyCache, SweepWorkspace, plan_sweep, sweep_layer
from support import compare_attention, compare_masks, log, oracle_k_b, oracle_masks_from_pools

pytestmark = pytest.mark.gpu

S = synth.SWEEP


def _plan(schedule="cag"):
    g = lf.Geom(S.B, S.H, S.d, S.tpf, S.bs)
    return g, plan_sweep(g, S.n_chunks, S.frames_per_chunk, S.k_f, S.T, S.s_base, S.s_target, S.d ** -0.5,
                         schedule=schedule)


def _attn_rows(layer, n_qb):
    if layer in (0, S.n_layers - 1):
        return [(0, h, r) for h in range(S.H) for r in range(n_qb)]
    h = int(np.random.default_rng(S.seed(layer)).integers(0, S.H))
    return [(0, h, r) for r in range(n_qb)]


def _check_layer(layer, schedule, cached):
    g, sp = _plan(schedule)
    log(f"[sweep] layer {layer} ({schedule}): generating inputs")
    x = synth.make_sweep_layer(S, layer)
    dev = torch.device("cuda")
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    o = torch.full_like(q, float("nan"))
    sw = SweepWorkspace(sp, q.dtype, dev)
    log(f"[sweep] layer {layer}: 7 chunks on the GPU")
    sweep_layer(sw, q, k, v, o)
    if cached:
        o_c = torch.full_like(q, float("nan"))
        sw_c = SweepWorkspace(sp, q.dtype, dev)
        cache = PooledKeyCache(g, sp.n_frames, dev)
        cache.k_blk.fill_(float("nan"))
        cache.k_frm.fill_(float("nan"))
        stages = []
        sweep_layer(sw_c, q, k, v, o_c, mark=lambda i, st: stages.append((i, st)), cache=cache)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any(), "some output token was not written"
    if cached:
        assert (1, "pool") in stages and (1, "select") not in stages
        assert torch.equal(o, o_c), "steady-state outputs differ from the uncached sweep"
        last = sw.chunks[-1]
        assert torch.equal(last.k_blk, cache.k_blk) and torch.equal(last.k_frm, cache.k_frm)
    q64, k64, v64 = x.np64()
    o_np = o.float().cpu().numpy()
    tpf, fpc, nb = S.tpf, S.frames_per_chunk, lf.n_bpf(g)
    kb_all = oracle.pool_blocks(k64, S.n_frames, tpf, S.bs)       # every frame pooled once
    kf_all = oracle.pool_frames(k64, S.n_frames, tpf)
    for i, p in enumerate(sp.chunks, 1):
        w = S.chunk(i, layer, schedule)
        assert p.k_b == oracle_k_b(w)
        a, b = (i - 1) * fpc * tpf, i * fpc * tpf
        qi, ki, vi = q64[:, :, a:b], k64[:, :, :b], v64[:, :, :b]
        q_blk = oracle.pool_blocks(qi, fpc, tpf, S.bs)
        ref = oracle_masks_from_pools(w, q_blk, kb_all[:, :, :i * fpc * nb], kf_all[:, :, :i * fpc], p.k_b)
        if sp.dense(i):
            blocks = sw.full[i].cpu().numpy()
            assert np.array_equal(ref["blocks"], blocks), "dense chunk: oracle lists are not the full lists"
        else:
            ws = sw.chunks[i - 1]
            gpu = dict(frames=ws.frames.cpu().numpy(), blocks=ws.blocks.cpu().numpy())
            stats = compare_masks(gpu, ref, min(p.k_b, p.n_bpf))
            if cached:
                wc = sw_c.chunks[i - 1]
                assert torch.equal(ws.q_blk, wc.q_blk) and torch.equal(ws.frames, wc.frames) \
                    and torch.equal(ws.blocks, wc.blocks), f"chunk {i}: steady-state lists differ"
                compare_masks(dict(frames=wc.frames.cpu().numpy(), blocks=wc.blocks.cpu().numpy()), ref,
                              min(p.k_b, p.n_bpf))
            log(f"[sweep] layer {layer} chunk {i}: masks {stats}")
            blocks = gpu["blocks"]
        rows = _attn_rows(layer, p.n_qb)
        st = compare_attention(w, dict(blocks=blocks, o=o_np[:, :, a:b]), qi, ki, vi, rows, "bf16")
        log(f"[sweep] layer {layer} chunk {i} (k_b={p.k_b}, W_b={p.W_b}): attention {st}")


@pytest.mark.parametrize("layer", range(S.n_layers))
def test_sweep_layer_parity(layer):
    _check_layer(layer, "cag", cached=True)


def test_sweep_uniform_allocation_parity():
    _check_layer(3, "uniform", cached=False)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_token_range_views_equal_packed(dtype):
    """The whole path on token-range views of a larger allocation (head stride > token
    count) gives bitwise the same pooled tensors, lists and outputs as on packed copies."""
    from dataclasses import replace
    from sparse_attention_autoregressive_amd.pipeline import Workspace, hsa_chunk
    from support import plan_of, lib_k_b
    w = replace(synth.TINY, dtype=dtype, name=f"tiny_views_{dtype}")
    x = synth.make(w)
    dev = torch.device("cuda")
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    plan = plan_of(w, lib_k_b(w))
    packed = Workspace(plan, q.dtype, dev)
    hsa_chunk(packed, q, k, v)
    cap = w.lk + 3 * w.tpf                                   # room for 3 more frames per head
    big = {n: torch.full((w.B, w.H, cap, w.d), float("nan"), dtype=q.dtype, device=dev) for n in "qkvo"}
    off = 2 * w.tpf                                          # queries start 2 frames in
    big["q"][:, :, off:off + w.lq] = q
    big["k"][:, :, :w.lk] = k
    big["v"][:, :, :w.lk] = v
    views = Workspace(plan, q.dtype, dev)
    hsa_chunk(views, big["q"][:, :, off:off + w.lq], big["k"][:, :, :w.lk], big["v"][:, :, :w.lk],
              out=big["o"][:, :, off:off + w.lq])
    torch.cuda.synchronize()
    for name in ("q_blk", "k_blk", "k_frm", "frames", "blocks"):
        assert torch.equal(getattr(packed, name), getattr(views, name)), name
    assert torch.equal(packed.o, big["o"][:, :, off:off + w.lq])
    assert torch.isnan(big["o"][:, :, :off]).all() and torch.isnan(big["o"][:, :, off + w.lq:]).all()


@pytest.mark.parametrize("name", ["tiny_fp32", "480p_chunk2of7"])
def test_steady_state_chunk_equals_uncached(name):
    """One chunk in steady state: packed queries and output, keys and values a prefix of a
    KV cache with room for more frames (so the query-side and key-side head strides
    differ), the history's pooled keys in a cache filled beforehand. Pooled queries, the
    cache's new frames, lists and output equal the uncached call on packed tensors
    bitwise; the chunk's own frame means are written by `complete_cache` only."""
    from sparse_attention_autoregressive_amd.pipeline import (Workspace, complete_cache, hsa_chunk, hsa_chunk_cached,
                                                              new_frames)
    from support import lib_k_b, plan_of
    w = synth.WORKLOADS[name]
    x = synth.make(w)
    dev = torch.device("cuda")
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    plan = plan_of(w, lib_k_b(w))
    g = plan.geom
    ref = Workspace(plan, q.dtype, dev)
    hsa_chunk(ref, q, k, v)
    cap_frames = w.n_kframes + 4
    kc = torch.full((w.B, w.H, cap_frames * w.tpf, w.d), float("nan"), dtype=q.dtype, device=dev)
    vc = torch.full_like(kc, float("nan"))
    kc[:, :, :w.lk] = k
    vc[:, :, :w.lk] = v
    cache = PooledKeyCache(g, cap_frames, dev)
    cache.k_blk.fill_(float("nan"))
    cache.k_frm.fill_(float("nan"))
    f0 = new_frames(plan)
    lf.lf_pool(kc[:, :, :f0 * w.tpf], g, f0, blk_out=cache.blk(0, f0), frm_out=cache.frm(0, f0))
    ws = Workspace(plan, q.dtype, dev)
    hsa_chunk_cached(ws, cache, q, kc[:, :, :w.lk], vc[:, :, :w.lk])
    torch.cuda.synchronize()
    assert torch.equal(ref.q_blk, ws.q_blk)
    assert torch.equal(ref.k_blk, cache.blk(0, w.n_kframes)) and torch.equal(ref.k_frm[:, :, :f0], cache.frm(0, f0))
    assert torch.isnan(cache.k_frm[:, :, f0:]).all(), "the chunk's own frame means are left to the next chunk"
    assert torch.equal(ref.frames, ws.frames) and torch.equal(ref.blocks, ws.blocks)
    assert torch.equal(ref.o, ws.o)
    complete_cache(plan, cache)
    torch.cuda.synchronize()
    assert torch.equal(ref.k_frm, cache.frm(0, w.n_kframes))
    assert torch.isnan(cache.k_frm[:, :, w.n_kframes:]).all() and torch.isnan(cache.k_blk[:, :, ref.k_blk.shape[2]:]).all()
