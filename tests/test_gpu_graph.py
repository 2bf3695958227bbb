"""HIP-graph replay of one chunk (pipeline.ChunkGraph) against eager calls, bitwise.

The graph is captured once on fixed tensors; two different input sets are written into
them in turn and the graph replayed, three rounds, with eager library work on other
tensors and host synchronisations between the replays. Every replay's T_r, block lists
and attention output must equal the eager results of the same inputs bit for bit, for
the uncached path and for the steady-state path over a pooled-key cache.
"""
import pytest
import torch

import synth
from sparse_attention_autoregressive_amd import lf_pool
from sparse_attention_autoregressive_amd.pipeline import (ChunkGraph, PooledKeyCache, Workspace, hsa_chunk,
                                                           hsa_chunk_cached, new_frames)
from support import lib_k_b, log, plan_of

pytestmark = pytest.mark.gpu


def _inputs(w, dev):
    x = synth.make(w)
    pool = [w.q_pool if w.q_pool is not None else x.planted]
    y = synth.make_on_device(w.B, w.H, w.n_qframes, w.n_kframes, w.tpf, w.bs, w.d, w.dtype, w.seed + 7,
                             dev, pool)
    return [(x.q.to(dev), x.k.to(dev), x.v.to(dev)), y]


def _outputs(ws):
    return ws.frames.clone(), ws.blocks.clone(), ws.o.clone()


@pytest.mark.parametrize("cached", [False, True])
def test_chunk_graph_replays_equal_eager(cached):
    w = synth.WORKLOADS["480p_chunk2of7"]
    dev = torch.device("cuda")
    log(f"[graph] {w.name} cached={cached}: inputs")
    sets = _inputs(w, dev)
    plan = plan_of(w, lib_k_b(w))
    f0 = new_frames(plan)

    def fill_history(c, k):
        """The history frames' means, as earlier chunks would have left them in the cache."""
        lf_pool(k[:, :, :f0 * w.tpf], plan.geom, f0, blk_out=c.blk(0, f0), frm_out=c.frm(0, f0))
        return c

    def cache_for(k):
        return fill_history(PooledKeyCache(plan.geom, w.n_kframes, dev), k)

    # eager references, one workspace (and cache) per input set
    refs = []
    for q, k, v in sets:
        ws = Workspace(plan, q.dtype, dev)
        if cached:
            hsa_chunk_cached(ws, cache_for(k), q, k, v)
        else:
            hsa_chunk(ws, q, k, v)
        torch.cuda.synchronize()
        refs.append(_outputs(ws))
    assert not torch.equal(refs[0][2], refs[1][2])      # the two sets really differ

    # the captured tensors: inputs copied in place before each replay
    q, k, v = (t.clone() for t in sets[0])
    ws = Workspace(plan, q.dtype, dev)
    cache = cache_for(k) if cached else None
    log(f"[graph] {w.name} cached={cached}: capture")
    g = ChunkGraph(ws, q, k, v, cache=cache)
    other = Workspace(plan, q.dtype, dev)
    for rnd in range(3):
        for i, (qi, ki, vi) in enumerate(sets):
            q.copy_(qi)
            k.copy_(ki)
            v.copy_(vi)
            if cached:   # the history part of the cache belongs to the input set
                fill_history(cache, k)
            g.replay()
            torch.cuda.synchronize()
            got = _outputs(ws)
            for name, a, b in zip(("frames", "blocks", "o"), got, refs[i]):
                assert torch.equal(a, b), (rnd, i, name)
            # eager work between replays, on other tensors
            hsa_chunk(other, *sets[1 - i])
            torch.cuda.synchronize()
        log(f"[graph] {w.name} cached={cached}: round {rnd} equal")
