"""GPU parity of selection over long histories: more key frames than fit the frame stage's
one-frame-per-thread ranking (256), up to the 4096-frame limit. Frame ids then reach the
kernel as bit masks and the frame top-k is taken in k_f rounds of a workgroup-wide
maximum. Masks are compared with the oracle's on every row, attention on sampled rows,
and the separate selection calls with the fused one bitwise.

At 480p a latent frame holds 1560 tokens; these cases keep the frame count and shrink
the frame (64 tokens, 32-token blocks) so the oracle finishes in seconds."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
import sparse_attention_autoregressive_amd as lf
from support import compare_attention, compare_masks, fp32_logit_tol, log, run_gpu, run_oracle_masks, sample_rows

pytestmark = pytest.mark.gpu


def _long(n, **kw):
    base = dict(name=f"long_history_{n}", B=1, H=2, d=128, dtype="bf16", tpf=64, bs=32, n_kframes=n,
                current=(n - 3, n - 2, n - 1), sink=(0,), recent=(), mem=tuple(range(1, n - 3)), k_f=6, k_b=1,
                q_pool=tuple(range(0, n - 3)), seed=7100 + n % 97)
    base.update(kw)
    return replace(synth.CHUNK7, **base)


def _check(w, wide=False):
    x = synth.make(w)
    q64, k64, v64 = x.np64()
    log(f"[long] {w.name}: {w.n_kframes} key frames, |M| = {len(w.mem)}, k_f = {w.k_f}")
    gpu = run_gpu(w, x, w.k_b)
    ref = run_oracle_masks(w, q64, k64, w.k_b)
    stats = compare_masks(gpu, ref, min(w.k_b, ref["n_bpf"]))
    rows = sample_rows(w, gpu["frames"].shape[2], full=True)
    res = compare_attention(w, gpu, q64, k64, v64, rows, w.dtype,
                            tol=fp32_logit_tol(w, q64, k64, v64) if wide else None)
    log(f"[long] {w.name}: masks {stats}, attention {res}")
    return x, gpu


@pytest.mark.parametrize("n, tpf", [(257, 64), (700, 96), (1200, 64)])
def test_long_history_masks_and_attention(n, tpf):
    # 8, 16 and 32 scores per lane in the top-k rounds; tpf = 96 gives 3 blocks per frame,
    # 9 query blocks per head, so the last workgroup of each head holds a single row
    w = _long(n, tpf=tpf, name=f"long_history_{n}_tpf{tpf}")
    x, gpu = _check(w)
    # the planted frames are among the retrieved ones for most rows (the scores work)
    pairs, frames = x.pairs.reshape(-1, 2), gpu["frames"].reshape(-1, gpu["frames"].shape[-1])
    hit = np.mean([len(set(p) & set(f)) for p, f in zip(pairs, frames)])
    assert hit > 1.0, hit


def test_long_history_480p_block_geometry():
    # 300 key frames at the 480p frame and block sizes (1560 tokens, 25 blocks per frame
    # with a 24-token tail, 75 query blocks), one head, k_f = 4 and k_b = 8 as at chunk 7
    _check(_long(300, H=1, d=128, tpf=1560, bs=64, k_f=4, k_b=8, name="long_history_480p"))


def test_long_history_two_batches():
    # B = 2: the (b, h) slices of q~, k^ and k~ and the rows' workgroups across the batch
    _check(_long(300, B=2, H=2, d=64, dtype="fp32", k_f=5, name="long_history_batch2"))


def test_long_history_max_frames_fp32():
    # the 4096-frame limit: 4092 memory frames, the dynamic LDS at its largest
    _check(_long(4096, H=1, d=64, dtype="fp32", k_f=8, name="long_history_4096_fp32"))


def test_long_history_max_frames_wide_fp32():
    # 4096 frames with k_f = 4000 of the 4092 memory frames: T_r at its widest, the
    # selection's LDS past 64 KB per workgroup; each row attends over 4004 blocks, so the
    # output tolerance follows the fp32 logit error bound
    _check(_long(4096, H=1, d=64, dtype="fp32", k_f=4000, name="long_history_4096_wide"), wide=True)


def test_long_history_keep_all():
    # k_f >= |M| over 300 frames: every memory frame kept without scores, W_f = 300
    _check(_long(300, H=1, d=64, dtype="fp32", k_f=400, name="long_history_keep_all"))


def test_long_history_separate_calls_equal_fused():
    w = _long(1200, H=1, name="long_history_calls")
    x = synth.make(w)
    gpu = run_gpu(w, x, w.k_b)
    dev = torch.device("cuda")
    g = lf.Geom(w.B, w.H, w.d, w.tpf, w.bs)
    n_qb = w.n_qframes * lf.n_bpf(g)
    q_blk, k_frm, k_blk = (torch.from_numpy(gpu[k]).to(dev) for k in ("q_blk", "k_frm", "k_blk"))
    frames = lf.lf_select_frames(q_blk, k_frm, g, n_qb, w.n_kframes, w.mem, w.forced, w.k_f)
    blocks = lf.lf_select_blocks(q_blk, k_blk, g, n_qb, w.n_kframes, frames, w.k_b)
    _, blocks2 = lf.lf_select(q_blk, k_frm, k_blk, g, n_qb, w.n_kframes, w.mem, w.forced, w.k_f, w.k_b,
                              with_frames=False)
    torch.cuda.synchronize()
    assert np.array_equal(frames.cpu().numpy(), gpu["frames"])
    assert np.array_equal(blocks.cpu().numpy(), gpu["blocks"])
    assert np.array_equal(blocks2.cpu().numpy(), gpu["blocks"])


def test_long_history_equal_scores_take_lowest_ids():
    # zero queries: every frame score is exactly 0, so each row's top k_f of M are its
    # k_f lowest frame ids (the pages' ranking with ties to the lower id), and each
    # frame's top k_b blocks its k_b lowest block indices
    w = _long(700, H=1, d=64, dtype="fp32", k_f=20, k_b=1, name="long_history_ties")
    x = synth.make(w)
    x = replace(x, q=torch.zeros_like(x.q))
    gpu = run_gpu(w, x, w.k_b)
    want = sorted(set(w.forced) | set(sorted(w.mem)[:w.k_f]))
    frames = gpu["frames"].reshape(-1, gpu["frames"].shape[-1])
    assert all(list(f) == want for f in frames)
    blocks = gpu["blocks"].reshape(-1, gpu["blocks"].shape[-1])
    nb = lf.n_bpf(lf.Geom(w.B, w.H, w.d, w.tpf, w.bs))
    assert all(list(b) == [f * nb for f in want] for b in blocks)
