"""The T denoising steps of one chunk in steady state (pipeline.denoise_steps) at full size
(480p chunk 7 of 7: 18 history frames, the chunk's 3 frames, 4 steps): the history's keys
and values sit in a KV cache and their pooled keys in a pooled-key cache filled once; each
step writes the chunk's new keys and values into the cache, re-pools only the chunk's
frames' block means (their frame means are first read by the next chunk) and attends over
the cached prefix.

Every step's pooled queries, lists and output equal the uncached path on that step's
packed inputs bitwise; the history's cached means never change; the last step's masks
(every row) and sampled outputs match the oracle run on that step's inputs."""
import numpy as np
import pytest
import torch

import synth
import sparse_attention_autoregressive_amd as lf
from sparse_attention_autoregressive_amd.pipeline import (PooledKeyCache, Workspace, complete_cache, denoise_steps,
                                                          hsa_chunk, new_frames)
from support import compare_attention, compare_masks, lib_k_b, log, plan_of, run_oracle_masks, sample_rows

pytestmark = pytest.mark.gpu

T = 4


def test_denoise_steps_chunk7():
    w = synth.CHUNK7
    log(f"[steps] {w.name}: generating {T} steps")
    steps = synth.make_denoise_steps(w, T)
    dev = torch.device("cuda")
    plan = plan_of(w, lib_k_b(w))
    g = plan.geom
    f0 = new_frames(plan)
    a, b = f0 * w.tpf, w.lk
    cap = w.n_kframes + 3                                   # room for the next chunk
    k_cache = torch.full((w.B, w.H, cap * w.tpf, w.d), float("nan"), dtype=torch.bfloat16, device=dev)
    v_cache = torch.full_like(k_cache, float("nan"))
    k_cache[:, :, :a] = steps[0].k[:, :, :a].to(dev)        # the history, written by earlier chunks
    v_cache[:, :, :a] = steps[0].v[:, :, :a].to(dev)
    cache = PooledKeyCache(g, cap, dev)
    cache.k_blk.fill_(float("nan"))
    cache.k_frm.fill_(float("nan"))
    lf.lf_pool(k_cache[:, :, :a], g, f0, blk_out=cache.blk(0, f0), frm_out=cache.frm(0, f0))
    hist_blk, hist_frm = cache.blk(0, f0).clone(), cache.frm(0, f0).clone()
    ws = Workspace(plan, torch.bfloat16, dev)
    outs = [torch.empty((w.B, w.H, w.lq, w.d), dtype=torch.bfloat16, device=dev) for _ in range(T)]
    dev_steps = [(s.q.to(dev), s.k.to(dev), s.v.to(dev)) for s in steps]
    seen = []

    def feed():
        for t, (q, k, v) in enumerate(dev_steps):
            yield q, k[:, :, a:], v[:, :, a:], outs[t]
            torch.cuda.synchronize()                          # step t has run: keep its lists
            seen.append((ws.q_blk.clone(), ws.frames.clone(), ws.blocks.clone()))

    log(f"[steps] {w.name}: {T} steady-state steps on the GPU")
    last = denoise_steps(ws, cache, k_cache, v_cache, feed())
    torch.cuda.synchronize()
    assert len(seen) == T and last is outs[-1]
    assert torch.equal(cache.blk(0, f0), hist_blk) and torch.equal(cache.frm(0, f0), hist_frm)
    assert torch.isnan(cache.k_frm[:, :, f0:]).all() and torch.isnan(k_cache[:, :, b:]).all()
    complete_cache(plan, cache)                             # the chunk's frame means, left to the next chunk
    torch.cuda.synchronize()
    for t, (q, k, v) in enumerate(dev_steps):
        ref = Workspace(plan, torch.bfloat16, dev)
        hsa_chunk(ref, q, k, v)
        torch.cuda.synchronize()
        q_blk, frames, blocks = seen[t]
        assert torch.equal(ref.q_blk, q_blk), f"step {t}: pooled queries"
        assert torch.equal(ref.frames, frames) and torch.equal(ref.blocks, blocks), f"step {t}: lists"
        assert torch.equal(ref.o, outs[t]), f"step {t}: output"
        if t == T - 1:
            assert torch.equal(ref.k_blk, cache.blk(0, w.n_kframes)) and torch.equal(ref.k_frm, cache.frm(0, w.n_kframes))
    log(f"[steps] {w.name}: oracle on the last step")
    q64, k64, v64 = steps[-1].np64()
    ref = run_oracle_masks(w, q64, k64, plan.k_b)
    gpu = dict(frames=seen[-1][1].cpu().numpy(), blocks=seen[-1][2].cpu().numpy(), o=outs[-1].float().cpu().numpy())
    stats = compare_masks(gpu, ref, min(plan.k_b, plan.n_bpf))
    res = compare_attention(w, gpu, q64, k64, v64, sample_rows(w, plan.n_qb, full=False), "bf16")
    log(f"[steps] {w.name} step {T - 1}: masks {stats}, attention {res}")
    # the steps really differ: the chunk's lists change from step to step
    assert not all(torch.equal(seen[0][2], s[2]) for s in seen[1:])
