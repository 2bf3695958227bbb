"""Host-side checks of the C ABI (no GPU): the library loads, exports every symbol the
header declares, solves the CAG schedule and the block budget like the oracle, and
rejects bad arguments before anything is launched."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle
import sparse_attention_autoregressive_amd as lf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
lib_missing = not os.path.exists(lf.library_path())
pytestmark = pytest.mark.skipif(lib_missing, reason="liblf.so not built")


def _declared():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            names |= set(re.findall(r"\b(lf_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(lf.library_path())
    names = _declared()
    assert {"lf_pool", "lf_pool_qk", "lf_select_frames", "lf_select_blocks", "lf_select", "lf_sparse_attn",
            "lf_cag_schedule", "lf_block_budget", "lf_last_error", "lf_abi_version",
            "lf_probe_mfma_bf16", "lf_probe_hbm_read", "lf_pool_step", "lf_qk_prologue_step"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lf.lf_abi_version() == 4


@pytest.mark.parametrize("n,T,s_base,s_t", [(7, 4, 0.95, 0.8), (7, 4, 0.95, 0.85), (5, 2, 0.9, 0.6),
                                            (12, 8, 0.97, 0.75), (2, 4, 0.95, 0.4)])
def test_cag_matches_oracle(n, T, s_base, s_t):
    rng = np.random.default_rng(n + T)
    for F in (list(range(1, n + 1)), rng.uniform(0.5, 3, n).cumsum().tolist()):
        s_lib, b_lib = lf.lf_cag_schedule(n, T, s_base, s_t, F)
        s_or, b_or = oracle.cag_schedule(n, T, s_base, s_t, F)
        assert b_lib == pytest.approx(b_or, rel=1e-12, abs=1e-14)
        assert np.allclose(s_lib, s_or, rtol=0, atol=1e-12)
        alpha = rng.uniform(0.1, 0.5, n).tolist()
        try:
            s_or, b_or = oracle.cag_schedule(n, T, s_base, s_t, F, alpha=alpha)
        except ValueError:
            with pytest.raises(lf.LfError):
                lf.lf_cag_schedule(n, T, s_base, s_t, F, alpha=alpha)
            continue
        s_lib, b_lib = lf.lf_cag_schedule(n, T, s_base, s_t, F, alpha=alpha)
        assert b_lib == pytest.approx(b_or, rel=1e-12, abs=1e-14)
        assert np.allclose(s_lib, s_or, rtol=0, atol=1e-12)


@pytest.mark.parametrize("s_t", [0.93, 0.2])
def test_cag_infeasible(s_t):
    with pytest.raises(lf.LfError) as e:
        lf.lf_cag_schedule(7, 4, 0.95, s_t, list(range(1, 8)))
    assert e.value.status == lf.LF_ERR_INFEASIBLE


@pytest.mark.parametrize("args", [(1, 4, 0.95, 0.8), (7, 0, 0.95, 0.8), (7, 4, 1.5, 0.8),
                                  (7, 4, 0.95, 1.0), (7, 4, 0.95, -0.1)])
def test_cag_invalid(args):
    n = max(args[0], 1)
    with pytest.raises(lf.LfError) as e:
        lf.lf_cag_schedule(*args, list(range(1, n + 1)))
    assert e.value.status == lf.LF_ERR_INVALID_ARG
    with pytest.raises(lf.LfError):
        lf.lf_cag_schedule(3, 4, 0.95, 0.5, [1.0, -2.0, 3.0])


def test_block_budget_matches_oracle():
    rng = np.random.default_rng(0)
    for _ in range(2000):
        s = float(rng.uniform(0, 1))
        n_kb, W_f, n_bpf = int(rng.integers(1, 3000)), int(rng.integers(1, 30)), int(rng.integers(1, 64))
        assert lf.lf_block_budget(s, n_kb, W_f, n_bpf) == oracle.block_budget(s, n_kb, W_f, n_bpf)
    # exact half-way points round up
    assert lf.lf_block_budget(0.5, 10, 2, 25) == 3
    with pytest.raises(lf.LfError):
        lf.lf_block_budget(1.5, 10, 2, 25)


# --------------------------------------------------------------------- argument validation
_lib = None


def _c():
    global _lib
    if _lib is None:
        lf._load()
        _lib = lf._lib
    return _lib


FAKE = 0x10000            # 16-byte aligned, never dereferenced: every call below fails validation


def _err(status, want):
    assert status == want, (status, _c().lf_last_error().decode())
    assert _c().lf_last_error().decode() != ""


def test_pool_validation():
    c = _c()
    good = lf.Geom(1, 2, 128, 1560, 64)
    _err(c.lf_pool(FAKE, 1, lf.Geom(1, 2, 96, 1560, 64), 3, FAKE, None, None), lf.LF_ERR_UNSUPPORTED)
    _err(c.lf_pool(FAKE, 7, good, 3, FAKE, None, None), lf.LF_ERR_UNSUPPORTED)
    _err(c.lf_pool(None, 1, good, 3, FAKE, None, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_pool(FAKE + 4, 1, good, 3, FAKE, None, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_pool(FAKE, 1, good, 0, FAKE, None, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_pool(FAKE, 1, lf.Geom(0, 2, 128, 1560, 64), 3, FAKE, None, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_pool(FAKE, 1, lf.Geom(1, 2, 128, 64, 65), 3, FAKE, None, None), lf.LF_ERR_INVALID_ARG)


def test_select_frames_validation():
    c = _c()
    g = lf.Geom(1, 2, 128, 1560, 64)
    arr = lf._i32_array

    def call(mem, forced, k_f=2, n_kf=10, out=FAKE):
        return c.lf_select_frames(FAKE, FAKE, g, 75, n_kf, arr(mem), len(mem), arr(forced),
                                  len(forced), k_f, out, None)

    _err(call([1, 2], [2, 9]), lf.LF_ERR_INVALID_ARG)          # overlap
    _err(call([1, 1], [0]), lf.LF_ERR_INVALID_ARG)             # duplicate
    _err(call([1, 12], [0]), lf.LF_ERR_INVALID_ARG)            # out of range
    _err(call([], [], k_f=3), lf.LF_ERR_INVALID_ARG)           # empty T_r
    _err(call([1], [0], k_f=-1), lf.LF_ERR_INVALID_ARG)
    _err(call([1], [0], n_kf=4097), lf.LF_ERR_UNSUPPORTED)              # beyond the 4096-frame limit
    _err(call([1, 4000], [0], n_kf=3000), lf.LF_ERR_INVALID_ARG)        # long history: id out of range
    _err(call([1], [0], out=FAKE + 2), lf.LF_ERR_INVALID_ARG)


def test_select_blocks_validation():
    c = _c()
    g = lf.Geom(1, 2, 128, 1560, 64)
    _err(c.lf_select_blocks(FAKE, FAKE, g, 75, 21, FAKE, 8, 0, FAKE, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_select_blocks(FAKE, FAKE, g, 75, 21, FAKE, 0, 8, FAKE, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_select_blocks(FAKE, FAKE, lf.Geom(1, 2, 128, 1560, 16), 75, 21, FAKE, 8, 8, FAKE, None),
         lf.LF_ERR_UNSUPPORTED)                                 # 98 blocks per frame
    _err(c.lf_select_blocks(None, FAKE, g, 75, 21, FAKE, 8, 8, FAKE, None), lf.LF_ERR_INVALID_ARG)


def test_select_fused_validation():
    c = _c()
    g = lf.Geom(1, 2, 128, 1560, 64)
    arr = lf._i32_array

    def call(mem, forced, k_f=2, k_b=8, n_kf=10, frames=FAKE, blocks=FAKE, gg=g):
        return c.lf_select(FAKE, FAKE, FAKE, gg, 75, n_kf, arr(mem), len(mem), arr(forced), len(forced),
                           k_f, k_b, frames, blocks, None)

    _err(call([1, 2], [2, 9]), lf.LF_ERR_INVALID_ARG)          # overlap
    _err(call([1], [0], k_b=0), lf.LF_ERR_INVALID_ARG)
    _err(call([1], [0], blocks=None), lf.LF_ERR_INVALID_ARG)
    _err(call([1], [0], frames=FAKE + 2), lf.LF_ERR_INVALID_ARG)
    _err(call([1], [0], n_kf=4097), lf.LF_ERR_UNSUPPORTED)              # beyond the 4096-frame limit
    _err(call([1, 4000], [0], n_kf=3000), lf.LF_ERR_INVALID_ARG)        # long history: id out of range
    _err(call([1], [0], gg=lf.Geom(1, 2, 128, 1560, 16)), lf.LF_ERR_UNSUPPORTED)   # 98 blocks per frame


def test_sparse_attn_validation():
    c = _c()
    g = lf.Geom(1, 2, 128, 1560, 64)
    F = FAKE
    _err(c.lf_sparse_attn(F, F, F, F, 1, lf.Geom(1, 2, 128, 1560, 128), 3, 21, F, 64, 0.1, None),
         lf.LF_ERR_UNSUPPORTED)                                 # bf16 path needs bs <= 64
    _err(c.lf_sparse_attn(F, F, F, F, 1, g, 3, 21, F, 0, 0.1, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_sparse_attn(F, F, F, F, 1, g, 3, 21, F, 64, math.inf, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_sparse_attn(F, F, F, F, 1, g, 3, 21, F, 64, -0.1, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_sparse_attn(F, F, None, F, 1, g, 3, 21, F, 64, 0.1, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_sparse_attn(F, F, F, F + 8, 1, g, 3, 21, F, 64, 0.1, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_sparse_attn(F, F, F, F, 3, g, 3, 21, F, 64, 0.1, None), lf.LF_ERR_UNSUPPORTED)
    _err(c.lf_sparse_attn(F, F, F, F, 1, lf.Geom(1, 2, 80, 1560, 64), 3, 21, F, 64, 0.1, None),
         lf.LF_ERR_UNSUPPORTED)


def test_pool_qk_validation():
    c = _c()
    F = FAKE
    g = lf.Geom(1, 2, 128, 1560, 64)
    _err(c.lf_pool_qk(F, F, 1, g, 0, 21, F, F, F, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_pool_qk(F, None, 1, g, 3, 21, F, F, F, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_pool_qk(F, F, 1, g, 3, 21, F, F, F + 4, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_pool_qk(F, F, 7, g, 3, 21, F, F, F, None), lf.LF_ERR_UNSUPPORTED)
    # query stride below the 3-frame query range, key stride below the 21-frame key range
    _err(c.lf_pool_qk(F, F, 1, lf.Geom(1, 2, 128, 1560, 64, 4679), 3, 21, F, F, F, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_pool_qk(F, F, 1, lf.Geom(1, 2, 128, 1560, 64, 0, 21 * 1560 - 1), 3, 21, F, F, F, None),
         lf.LF_ERR_INVALID_ARG)
    # pooled-key outputs: frame stride below the 21 pooled frames
    _err(c.lf_pool_qk(F, F, 1, lf.Geom(1, 2, 128, 1560, 64, 0, 0, 20), 3, 21, F, F, F, None), lf.LF_ERR_INVALID_ARG)


def test_head_stride_validation():
    c = _c()
    F = FAKE
    # pooling 3 frames of 1560 tokens needs a head stride of 0 or >= 4680
    _err(c.lf_pool(F, 1, lf.Geom(1, 2, 128, 1560, 64, 4679), 3, F, None, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_pool(F, 1, lf.Geom(1, 2, 128, 1560, 64, -1), 3, F, None, None), lf.LF_ERR_INVALID_ARG)
    # attention: the query stride covers the 3 query frames, the key stride the 21 key frames
    _err(c.lf_sparse_attn(F, F, F, F, 1, lf.Geom(1, 2, 128, 1560, 64, 3 * 1560 - 1), 3, 21, F, 64, 0.1, None),
         lf.LF_ERR_INVALID_ARG)
    _err(c.lf_sparse_attn(F, F, F, F, 1, lf.Geom(1, 2, 128, 1560, 64, 0, 21 * 1560 - 1), 3, 21, F, 64, 0.1,
                          None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_sparse_attn(F, F, F, F, 1, lf.Geom(1, 2, 128, 1560, 64, 0, -5), 3, 21, F, 64, 0.1, None),
         lf.LF_ERR_INVALID_ARG)
    g = lf.Geom(1, 2, 128, 1560, 64)
    assert g.head_stride == 0 and g.kv_head_stride == 0 and g.frame_stride == 0
    g2 = g.with_stride(7, 9).with_frame_stride(21)
    assert (g2.head_stride, g2.kv_head_stride, g2.frame_stride) == (7, 9, 21)
    assert g2.with_stride(8).kv_head_stride == 9


def test_frame_stride_validation():
    c = _c()
    F = FAKE
    arr = lf._i32_array
    # lf_pool outputs: 0 or at least n_frames
    _err(c.lf_pool(F, 1, lf.Geom(1, 2, 128, 1560, 64, 0, 0, 2), 3, F, F, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_pool(F, 1, lf.Geom(1, 2, 128, 1560, 64, 0, 0, -1), 3, F, F, None), lf.LF_ERR_INVALID_ARG)
    # selection reads n_kframes pooled frames per (b, h) slice
    short = lf.Geom(1, 2, 128, 1560, 64, 0, 0, 9)
    _err(c.lf_select_frames(F, F, short, 75, 10, arr([1]), 1, arr([0]), 1, 1, F, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_select_blocks(F, F, short, 75, 10, F, 2, 8, F, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_select(F, F, F, short, 75, 10, arr([1]), 1, arr([0]), 1, 1, 8, F, F, None), lf.LF_ERR_INVALID_ARG)
    assert "frame_stride" in c.lf_last_error().decode()


def test_error_message_is_per_thread():
    import threading
    c = _c()
    _err(c.lf_pool(None, 1, lf.Geom(1, 2, 128, 1560, 64), 3, FAKE, None, None), lf.LF_ERR_INVALID_ARG)
    seen = {}

    def other():
        seen["msg"] = c.lf_last_error().decode()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "lf_pool" in c.lf_last_error().decode()


def test_probe_validation():
    c = _c()
    _err(c.lf_probe_mfma_bf16(0, 10, FAKE, FAKE, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_probe_mfma_bf16(4, 0, FAKE, FAKE, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_probe_mfma_bf16(4, 10, FAKE, FAKE + 4, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_probe_mfma_bf16(4, 10, None, FAKE, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_probe_hbm_read(FAKE, 1 << 20, 0, FAKE, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_probe_hbm_read(FAKE, 1000, 4, FAKE, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_probe_hbm_read(FAKE, 0, 4, FAKE, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_probe_hbm_read(FAKE + 8, 1 << 20, 4, FAKE, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_probe_hbm_read(None, 1 << 20, 4, FAKE, None), lf.LF_ERR_INVALID_ARG)


def test_select_1d_validation():
    c = _c()
    F = FAKE
    g = lf.Geom(1, 2, 128, 1560, 64)                      # 25 blocks per frame
    _err(c.lf_select_blocks_1d(F, F, g, 75, 21, 0, F, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_select_blocks_1d(F, F, g, 75, 21, 526, F, None), lf.LF_ERR_INVALID_ARG)     # K > 525 blocks
    _err(c.lf_select_blocks_1d(F, F, g, 75, 164, 64, F, None), lf.LF_ERR_UNSUPPORTED)    # 4100 blocks
    _err(c.lf_select_blocks_1d(F, None, g, 75, 21, 64, F, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_select_blocks_1d(F, F, g, 75, 21, 64, F + 2, None), lf.LF_ERR_INVALID_ARG)
    _err(c.lf_select_blocks_1d(F, F, lf.Geom(1, 2, 128, 1560, 64, 0, 0, 20), 75, 21, 64, F, None),
         lf.LF_ERR_INVALID_ARG)                                                            # frame stride < 21


def test_prologue_validation():
    c = _c()
    F = FAKE
    g = lf.Geom(1, 2, 128, 1560, 64)
    call = lambda gg=g, n=3, f0=0, lw=52, eps=1e-6, th=1e4, x=F, y=F + 4096, gm=F: c.lf_qk_prologue(
        x, y, gm, 1, gg, n, f0, lw, eps, th, F, None, None)
    _err(call(lw=50), lf.LF_ERR_INVALID_ARG)             # 50 does not divide 1560
    _err(call(lw=0), lf.LF_ERR_INVALID_ARG)
    _err(call(eps=0.0), lf.LF_ERR_INVALID_ARG)
    _err(call(eps=math.nan), lf.LF_ERR_INVALID_ARG)
    _err(call(th=1.0), lf.LF_ERR_INVALID_ARG)
    _err(call(f0=-1), lf.LF_ERR_INVALID_ARG)
    _err(call(n=0), lf.LF_ERR_INVALID_ARG)
    _err(call(y=F), lf.LF_ERR_INVALID_ARG)               # output aliases input
    _err(call(gm=None), lf.LF_ERR_INVALID_ARG)
    _err(call(gm=F + 4), lf.LF_ERR_INVALID_ARG)
    _err(call(gg=lf.Geom(1, 2, 96, 1560, 64)), lf.LF_ERR_UNSUPPORTED)
    _err(call(gg=lf.Geom(1, 2, 128, 1560, 64, 4679)), lf.LF_ERR_INVALID_ARG)
    _err(call(gg=lf.Geom(1, 2, 128, 1560, 64, 0, 0, 2)), lf.LF_ERR_INVALID_ARG)


def test_prologue_output_stride_validation():
    c = _c()
    F = FAKE
    _err(c.lf_qk_prologue(F, F + 4096, F, 1, lf.Geom(1, 2, 128, 1560, 64, 0, 4679), 3, 0, 52, 1e-6, 1e4, F, None,
                          None), lf.LF_ERR_INVALID_ARG)   # output stride below 3 frames


def test_pool_step_validation():
    c = _c()
    F = FAKE
    g = lf.Geom(1, 2, 128, 1560, 64, 0, 0, 24)            # a 24-frame pooled-key cache
    call = lambda gg=g, q=F, k=F, nq=3, nn=3, fn=18, fl=15, nl=3, qb=F, kb=F, kf=F, dt=1: c.lf_pool_step(
        q, k, dt, gg, nq, nn, fn, fl, nl, qb, kb, kf, None)
    _err(call(gg=lf.Geom(1, 2, 128, 1560, 64)), lf.LF_ERR_INVALID_ARG)          # no cache frame count
    _err(call(fn=22), lf.LF_ERR_INVALID_ARG)                                     # new frames past the cache
    _err(call(fl=22), lf.LF_ERR_INVALID_ARG)                                     # lagged frames past the cache
    _err(call(fl=16), lf.LF_ERR_INVALID_ARG)                                     # lagged overlaps new
    _err(call(nq=-1), lf.LF_ERR_INVALID_ARG)
    _err(call(nl=-1), lf.LF_ERR_INVALID_ARG)
    _err(call(q=None), lf.LF_ERR_INVALID_ARG)
    _err(call(qb=None), lf.LF_ERR_INVALID_ARG)
    _err(call(k=None), lf.LF_ERR_INVALID_ARG)
    _err(call(kf=None), lf.LF_ERR_INVALID_ARG)
    _err(call(kb=F + 4), lf.LF_ERR_INVALID_ARG)
    _err(call(dt=7), lf.LF_ERR_UNSUPPORTED)
    _err(call(gg=lf.Geom(1, 2, 128, 1560, 64, 4679, 0, 24)), lf.LF_ERR_INVALID_ARG)    # query stride < 3 frames
    _err(call(gg=lf.Geom(1, 2, 128, 1560, 64, 0, 4679, 24)), lf.LF_ERR_INVALID_ARG)    # key stride < 3 frames
    # nothing to do: accepted without touching any pointer
    assert c.lf_pool_step(None, None, 1, g, 0, 0, 0, 0, 0, None, None, None, None) == lf.LF_OK


def test_prologue_step_validation():
    c = _c()
    F = FAKE
    g = lf.Geom(1, 2, 128, 1560, 64, 0, 0, 24)
    call = lambda gg=g, n=3, f0=18, lw=52, eps=1e-6, th=1e4, x=F, y=F + 4096, fn=18, fl=15, nl=3, kf=F: \
        c.lf_qk_prologue_step(x, F + 8192, y, F + 12288, F, F, 1, gg, n, f0, lw, eps, th, fn, fl, nl, F, F, kf, None)
    _err(call(lw=50), lf.LF_ERR_INVALID_ARG)
    _err(call(eps=0.0), lf.LF_ERR_INVALID_ARG)
    _err(call(th=1.0), lf.LF_ERR_INVALID_ARG)
    _err(call(n=0), lf.LF_ERR_INVALID_ARG)
    _err(call(f0=-1), lf.LF_ERR_INVALID_ARG)
    _err(call(y=F), lf.LF_ERR_INVALID_ARG)                                       # output aliases input
    _err(call(fn=22), lf.LF_ERR_INVALID_ARG)
    _err(call(fl=17), lf.LF_ERR_INVALID_ARG)                                     # lagged overlaps new
    _err(call(kf=None), lf.LF_ERR_INVALID_ARG)
    _err(call(gg=lf.Geom(1, 2, 128, 1560, 64)), lf.LF_ERR_INVALID_ARG)
    _err(call(gg=lf.Geom(1, 2, 96, 1560, 64, 0, 0, 24)), lf.LF_ERR_UNSUPPORTED)
    _err(call(gg=lf.Geom(1, 2, 128, 1560, 64, 0, 4679, 24)), lf.LF_ERR_INVALID_ARG)
