"""Light Forcing Hierarchical Sparse Attention (HSA) + Chunk-Aware Growth on MI355X.

Thin Python binding of the C ABI in include/lf.h (liblf.so, built by
`python -m sparse_attention_autoregressive_amd._build`). The functions carry the C
names and only marshal arguments: torch tensors provide device memory and the current
HIP stream; every step of the computation runs in the library's HIP kernels. There is
no fallback: if the library is missing, importing a function raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = ["Geom", "LfError", "lf_abi_version", "lf_cag_schedule", "lf_block_budget",
           "lf_pool", "lf_pool_qk", "lf_pool_step", "lf_qk_prologue", "lf_qk_prologue_step", "lf_select_frames", "lf_select_blocks", "lf_select", "lf_select_blocks_1d", "lf_sparse_attn",
           "lf_probe_mfma_bf16", "lf_probe_hbm_read", "library_path", "n_bpf"]

LF_OK, LF_ERR_INVALID_ARG, LF_ERR_UNSUPPORTED, LF_ERR_INFEASIBLE, LF_ERR_HIP = range(5)
LF_FP32, LF_BF16 = 0, 1
_STATUS = {1: "LF_ERR_INVALID_ARG", 2: "LF_ERR_UNSUPPORTED", 3: "LF_ERR_INFEASIBLE", 4: "LF_ERR_HIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "liblf.so")


class Geom(ctypes.Structure):
    """lf_geom: batch, heads, head dim, tokens per frame, tokens per block, the token
    strides between (b, h) slices of the query-side (q, o, lf_pool's x) and key-side (k, v)
    token tensors, and the frame stride between (b, h) slices of the pooled key tensors
    (0 = packed for each; the wrappers below fill them in from the tensors they are
    given)."""

    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32),
                ("tokens_per_frame", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("head_stride", ctypes.c_int32), ("kv_head_stride", ctypes.c_int32),
                ("frame_stride", ctypes.c_int32)]

    def __repr__(self):
        return (f"Geom(B={self.B}, H={self.H}, d={self.d}, tpf={self.tokens_per_frame}, "
                f"bs={self.block_size}, head_stride={self.head_stride}, kv_head_stride={self.kv_head_stride}, "
                f"frame_stride={self.frame_stride})")

    def _copy(self, **kw) -> "Geom":
        f = {n: getattr(self, n) for n, _ in self._fields_}
        f.update(kw)
        return Geom(**f)

    def with_stride(self, head_stride: int, kv_head_stride: Optional[int] = None) -> "Geom":
        return self._copy(head_stride=head_stride,
                          kv_head_stride=self.kv_head_stride if kv_head_stride is None else kv_head_stride)

    def with_frame_stride(self, frame_stride: int) -> "Geom":
        return self._copy(frame_stride=frame_stride)


def n_bpf(g: Geom) -> int:
    return -(-g.tokens_per_frame // g.block_size)


class LfError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m sparse_attention_autoregressive_amd._build`")
    lib = ctypes.CDLL(path)
    i32, f64, f32, vp = ctypes.c_int32, ctypes.c_double, ctypes.c_float, ctypes.c_void_p
    pf64 = ctypes.POINTER(ctypes.c_double)
    pi32 = ctypes.POINTER(ctypes.c_int32)
    lib.lf_last_error.restype = ctypes.c_char_p
    lib.lf_last_error.argtypes = []
    lib.lf_abi_version.restype = i32
    lib.lf_abi_version.argtypes = []
    sig = {
        "lf_cag_schedule": [i32, i32, f64, f64, pf64, pf64, pf64, pf64],
        "lf_block_budget": [f64, i32, i32, i32, pi32],
        "lf_pool": [vp, i32, Geom, i32, vp, vp, vp],
        "lf_pool_qk": [vp, vp, i32, Geom, i32, i32, vp, vp, vp, vp],
        "lf_select_frames": [vp, vp, Geom, i32, i32, pi32, i32, pi32, i32, i32, vp, vp],
        "lf_select_blocks": [vp, vp, Geom, i32, i32, vp, i32, i32, vp, vp],
        "lf_select": [vp, vp, vp, Geom, i32, i32, pi32, i32, pi32, i32, i32, i32, vp, vp, vp],
        "lf_sparse_attn": [vp, vp, vp, vp, i32, Geom, i32, i32, vp, i32, f32, vp],
        "lf_select_blocks_1d": [vp, vp, Geom, i32, i32, i32, vp, vp],
        "lf_qk_prologue": [vp, vp, vp, i32, Geom, i32, i32, i32, f32, f32, vp, vp, vp],
        "lf_pool_step": [vp, vp, i32, Geom, i32, i32, i32, i32, i32, vp, vp, vp, vp],
        "lf_qk_prologue_step": [vp, vp, vp, vp, vp, vp, i32, Geom, i32, i32, i32, f32, f32, i32, i32, i32, vp, vp,
                                vp, vp],
        "lf_probe_mfma_bf16": [i32, i32, vp, vp, vp],
        "lf_probe_hbm_read": [vp, ctypes.c_int64, i32, vp, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != LF_OK:
        raise LfError(status, _load().lf_last_error().decode())


def _stream(t: torch.Tensor) -> Optional[int]:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a tensor on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _exact(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple) -> int:
    """Checks a packed device tensor of one dtype and one exact shape (id lists, pooled
    queries); returns its data pointer. Raises ValueError before anything is enqueued."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a tensor on the GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _tokens(t: torch.Tensor, name: str, g: Geom, n_tokens: int) -> int:
    """Checks a [B, H, n_tokens, d] token tensor whose (b, h) slices are contiguous and
    evenly spaced (a packed tensor, or a token-range view of a bigger one); returns its
    head stride in tokens."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a tensor on the GPU")
    if tuple(t.shape) != (g.B, g.H, n_tokens, g.d):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(g.B, g.H, n_tokens, g.d)}")
    sb, sh, st, sc = t.stride()
    if sc != 1 or st != g.d or sh % g.d != 0 or (g.B > 1 and sb != g.H * sh):
        raise ValueError(f"{name}: each (b, h) slice must be contiguous and the slices evenly spaced")
    return sh // g.d


def _pooled(t: torch.Tensor, name: str, g: Geom, n_frames: int, per_frame: int) -> int:
    """Checks a pooled key tensor [B, H, n_frames*per_frame, d] fp32 (per_frame = blocks per
    frame for block means, 1 for frame means) whose (b, h) slices are contiguous and evenly
    spaced (packed, or the first frames of a cache sized for more); returns its frame
    stride."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a tensor on the GPU")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    if tuple(t.shape) != (g.B, g.H, n_frames * per_frame, g.d):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(g.B, g.H, n_frames * per_frame, g.d)}")
    sb, sh, sr, sc = t.stride()
    unit = per_frame * g.d
    if sc != 1 or sr != g.d or sh % unit != 0 or (g.B > 1 and sb != g.H * sh):
        raise ValueError(f"{name}: each (b, h) slice must be contiguous and the slices evenly spaced")
    return sh // unit


def _frame_geom(g: Geom, n_frames: int, strides: Sequence[int]) -> Geom:
    """g with the frame stride of the pooled key tensors of one call (0 when packed)."""
    if len(set(strides)) != 1:
        raise ValueError(f"pooled key tensors of one call must share their frame stride, got {strides}")
    return g.with_frame_stride(0 if strides[0] == n_frames else strides[0])


def _shared(names: str, strides: Sequence[int], n_tokens: int) -> int:
    """The head stride that tensors `names` share (0 when packed)."""
    if len(set(strides)) != 1:
        raise ValueError(f"{names} must share their head stride, got {strides}")
    return 0 if strides[0] == n_tokens else strides[0]


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return LF_BF16
    if t.dtype == torch.float32:
        return LF_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _i32_array(xs: Sequence[int]):
    arr = (ctypes.c_int32 * max(1, len(xs)))(*[int(x) for x in xs])
    return arr


def lf_abi_version() -> int:
    return int(_load().lf_abi_version())


def lf_cag_schedule(n_chunks: int, T: int, s_base: float, s_target: float,
                    chunk_flops: Sequence[float], alpha: Optional[Sequence[float]] = None):
    """Host call: returns (s[0..n-1], beta)."""
    lib = _load()
    F = (ctypes.c_double * n_chunks)(*[float(x) for x in chunk_flops])
    A = None if alpha is None else (ctypes.c_double * n_chunks)(*[float(x) for x in alpha])
    s = (ctypes.c_double * n_chunks)()
    beta = ctypes.c_double()
    _check(lib.lf_cag_schedule(n_chunks, T, s_base, s_target, F, A, s, ctypes.byref(beta)))
    return list(s), beta.value


def lf_block_budget(s: float, n_kblocks: int, W_f: int, n_bpf_: int) -> int:
    out = ctypes.c_int32()
    _check(_load().lf_block_budget(s, n_kblocks, W_f, n_bpf_, ctypes.byref(out)))
    return out.value


def lf_pool(x: torch.Tensor, g: Geom, n_frames: int, blk_out: Optional[torch.Tensor] = None,
            frm_out: Optional[torch.Tensor] = None, with_frames: bool = True):
    """Block means [B,H,n_frames*n_bpf,d] fp32 and (optionally) frame means [B,H,n_frames,d]."""
    lib = _load()
    nb = n_bpf(g)
    if blk_out is None:
        blk_out = torch.empty((g.B, g.H, n_frames * nb, g.d), dtype=torch.float32, device=x.device)
    if frm_out is None and with_frames:
        frm_out = torch.empty((g.B, g.H, n_frames, g.d), dtype=torch.float32, device=x.device)
    gx = g.with_stride(_tokens(x, "x", g, n_frames * g.tokens_per_frame))
    fs = [_pooled(blk_out, "blk_out", g, n_frames, nb)]
    if frm_out is not None:
        fs.append(_pooled(frm_out, "frm_out", g, n_frames, 1))
    gx = _frame_geom(gx, n_frames, fs)
    _check(lib.lf_pool(x.data_ptr(), _dtype_code(x), gx, n_frames, blk_out.data_ptr(),
                       None if frm_out is None else frm_out.data_ptr(), _stream(x)))
    return blk_out, frm_out


def lf_pool_qk(q: torch.Tensor, k: torch.Tensor, g: Geom, n_qframes: int, n_kframes: int,
               q_blk: Optional[torch.Tensor] = None, k_blk: Optional[torch.Tensor] = None,
               k_frm: Optional[torch.Tensor] = None):
    """Query block means and key block + frame means in one launch: (q_blk, k_blk, k_frm).
    q_blk is packed; k_blk and k_frm may be the first n_kframes frames of bigger caches."""
    lib = _load()
    nb = n_bpf(g)
    f32, dev = torch.float32, q.device
    if q_blk is None:
        q_blk = torch.empty((g.B, g.H, n_qframes * nb, g.d), dtype=f32, device=dev)
    if k_blk is None:
        k_blk = torch.empty((g.B, g.H, n_kframes * nb, g.d), dtype=f32, device=dev)
    if k_frm is None:
        k_frm = torch.empty((g.B, g.H, n_kframes, g.d), dtype=f32, device=dev)
    if q.dtype != k.dtype:
        raise TypeError("q and k must share a dtype")
    lq, lk = n_qframes * g.tokens_per_frame, n_kframes * g.tokens_per_frame
    gg = g.with_stride(_shared("q", [_tokens(q, "q", g, lq)], lq), _shared("k", [_tokens(k, "k", g, lk)], lk))
    gg = _frame_geom(gg, n_kframes, [_pooled(k_blk, "k_blk", g, n_kframes, nb), _pooled(k_frm, "k_frm", g, n_kframes, 1)])
    _check(lib.lf_pool_qk(q.data_ptr(), k.data_ptr(), _dtype_code(q), gg, n_qframes, n_kframes,
                          _exact(q_blk, "q_blk", torch.float32, (g.B, g.H, n_qframes * nb, g.d)),
                          k_blk.data_ptr(), k_frm.data_ptr(), _stream(q)))
    return q_blk, k_blk, k_frm


def lf_qk_prologue(x: torch.Tensor, gamma: torch.Tensor, g: Geom, n_frames: int, frame0: int, lat_w: int,
                   eps: float = 1e-6, theta: float = 10000.0, x_out: Optional[torch.Tensor] = None,
                   blk_out: Optional[torch.Tensor] = None, frm_out: Optional[torch.Tensor] = None,
                   with_frames: bool = True):
    """RMSNorm + rotary embedding of x into x_out (which may be a token-range view of a
    KV cache), fused with its block (and frame) means: returns (x_out, blk_out, frm_out or
    None)."""
    lib = _load()
    nb = n_bpf(g)
    if x_out is None:
        x_out = torch.empty_like(x)
    if blk_out is None:
        blk_out = torch.empty((g.B, g.H, n_frames * nb, g.d), dtype=torch.float32, device=x.device)
    if frm_out is None and with_frames:
        frm_out = torch.empty((g.B, g.H, n_frames, g.d), dtype=torch.float32, device=x.device)
    if x_out.dtype != x.dtype:
        raise TypeError("x_out must have x's dtype")
    if gamma.dtype != torch.float32 or tuple(gamma.shape) != (g.d,):
        raise ValueError(f"gamma must be float32 of shape ({g.d},)")
    L = n_frames * g.tokens_per_frame
    sx = _shared("x", [_tokens(x, "x", g, L)], L)
    sy = _shared("x_out", [_tokens(x_out, "x_out", g, L)], L)
    fs = [_pooled(blk_out, "blk_out", g, n_frames, nb)]
    if frm_out is not None:
        fs.append(_pooled(frm_out, "frm_out", g, n_frames, 1))
    gx = _frame_geom(g.with_stride(sx, sy), n_frames, fs)
    _check(lib.lf_qk_prologue(x.data_ptr(), x_out.data_ptr(), _dev(gamma, "gamma"), _dtype_code(x), gx, n_frames,
                              frame0, lat_w, float(eps), float(theta), blk_out.data_ptr(),
                              None if frm_out is None else frm_out.data_ptr(), _stream(x)))
    return x_out, blk_out, frm_out


def _cache(k_blk: torch.Tensor, k_frm: torch.Tensor, g: Geom) -> int:
    """Checks a pooled-key cache pair (block means [B, H, frames*n_bpf, d], frame means
    [B, H, frames, d], fp32, each (b, h) slice contiguous); returns its frame count."""
    nb = n_bpf(g)
    frames = k_frm.shape[2] if isinstance(k_frm, torch.Tensor) and k_frm.dim() == 4 else -1
    if frames < 1:
        raise ValueError("k_frm must be [B, H, frames, d]")
    if _pooled(k_blk, "k_blk", g, frames, nb) != frames or _pooled(k_frm, "k_frm", g, frames, 1) != frames:
        raise ValueError("the pooled-key cache tensors must be whole (not views of a bigger cache)")
    return frames


def lf_pool_step(q: Optional[torch.Tensor], k_new: Optional[torch.Tensor], g: Geom, n_qframes: int, n_new: int,
                 f_new: int, f_lag: int, n_lag: int, q_blk: Optional[torch.Tensor], k_blk: torch.Tensor,
                 k_frm: torch.Tensor):
    """One steady-state pooling launch: q_blk <- block means of q, k_blk[frames f_new..] <-
    block means of k_new, k_frm[frames f_lag..f_lag+n_lag) <- frame means from k_blk
    (k_blk, k_frm: a whole pooled-key cache). Returns q_blk."""
    lib = _load()
    nb = n_bpf(g)
    frames = _cache(k_blk, k_frm, g)
    dev = k_blk.device
    if n_qframes > 0 and q_blk is None:
        q_blk = torch.empty((g.B, g.H, n_qframes * nb, g.d), dtype=torch.float32, device=dev)
    lq, lk = n_qframes * g.tokens_per_frame, n_new * g.tokens_per_frame
    hs = _shared("q", [_tokens(q, "q", g, lq)], lq) if n_qframes > 0 else 0
    ks = _shared("k_new", [_tokens(k_new, "k_new", g, lk)], lk) if n_new > 0 else 0
    dtc = _dtype_code(q if n_qframes > 0 else (k_new if n_new > 0 else k_blk))
    if n_qframes > 0 and n_new > 0 and q.dtype != k_new.dtype:
        raise TypeError("q and k_new must share a dtype")
    qp = _exact(q_blk, "q_blk", torch.float32, (g.B, g.H, n_qframes * nb, g.d)) if n_qframes > 0 else None
    gg = g.with_stride(hs, ks).with_frame_stride(frames)
    _check(lib.lf_pool_step(q.data_ptr() if n_qframes > 0 else None, k_new.data_ptr() if n_new > 0 else None, dtc, gg,
                            n_qframes, n_new, f_new, f_lag, n_lag, qp, k_blk.data_ptr(), k_frm.data_ptr(),
                            _stream(k_blk)))
    return q_blk


def lf_qk_prologue_step(q: torch.Tensor, k_new: torch.Tensor, gamma_q: torch.Tensor, gamma_k: torch.Tensor, g: Geom,
                        n_frames: int, frame0: int, lat_w: int, f_new: int, f_lag: int, n_lag: int,
                        k_out: torch.Tensor, k_blk: torch.Tensor, k_frm: torch.Tensor, eps: float = 1e-6,
                        theta: float = 10000.0, q_out: Optional[torch.Tensor] = None,
                        q_blk: Optional[torch.Tensor] = None):
    """RMSNorm + rotary of a chunk's queries and new keys in one launch (keys written to
    k_out, e.g. a KV cache view), with the block means of both and the lagged frame means
    of lf_pool_step. Returns (q_out, q_blk)."""
    lib = _load()
    nb = n_bpf(g)
    frames = _cache(k_blk, k_frm, g)
    L = n_frames * g.tokens_per_frame
    if q_out is None:
        q_out = torch.empty_like(q)
    if q_blk is None:
        q_blk = torch.empty((g.B, g.H, n_frames * nb, g.d), dtype=torch.float32, device=q.device)
    if not (q.dtype == k_new.dtype == q_out.dtype == k_out.dtype):
        raise TypeError("q, k_new, q_out and k_out must share a dtype")
    for name, gm in (("gamma_q", gamma_q), ("gamma_k", gamma_k)):
        if gm.dtype != torch.float32 or tuple(gm.shape) != (g.d,):
            raise ValueError(f"{name} must be float32 of shape ({g.d},)")
    hs = _shared("q, k_new and q_out", [_tokens(q, "q", g, L), _tokens(k_new, "k_new", g, L),
                                        _tokens(q_out, "q_out", g, L)], L)
    ks = _shared("k_out", [_tokens(k_out, "k_out", g, L)], L)
    gg = g.with_stride(hs, ks).with_frame_stride(frames)
    _check(lib.lf_qk_prologue_step(q.data_ptr(), k_new.data_ptr(), q_out.data_ptr(), k_out.data_ptr(),
                                   _dev(gamma_q, "gamma_q"), _dev(gamma_k, "gamma_k"), _dtype_code(q), gg, n_frames,
                                   frame0, lat_w, float(eps), float(theta), f_new, f_lag, n_lag,
                                   _exact(q_blk, "q_blk", torch.float32, (g.B, g.H, n_frames * nb, g.d)),
                                   k_blk.data_ptr(), k_frm.data_ptr(), _stream(q)))
    return q_out, q_blk


def lf_select_frames(q_blk: torch.Tensor, k_frm: torch.Tensor, g: Geom, n_qb: int, n_kframes: int,
                     mem: Sequence[int], forced: Sequence[int], k_f: int,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """T_r per row: [B,H,n_qb,W_f] int32, W_f = len(forced) + min(k_f, len(mem))."""
    lib = _load()
    W_f = len(forced) + min(k_f, len(mem))
    if out is None:
        out = torch.empty((g.B, g.H, n_qb, max(W_f, 1)), dtype=torch.int32, device=q_blk.device)
    qp = _exact(q_blk, "q_blk", torch.float32, (g.B, g.H, n_qb, g.d))
    op = _exact(out, "out", torch.int32, (g.B, g.H, n_qb, max(W_f, 1)))
    g = _frame_geom(g, n_kframes, [_pooled(k_frm, "k_frm", g, n_kframes, 1)])
    _check(lib.lf_select_frames(qp, k_frm.data_ptr(), g, n_qb, n_kframes,
                                _i32_array(mem), len(mem), _i32_array(forced), len(forced), k_f,
                                op, _stream(q_blk)))
    return out


def lf_select_blocks(q_blk: torch.Tensor, k_blk: torch.Tensor, g: Geom, n_qb: int, n_kframes: int,
                     frames: torch.Tensor, k_b: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Mask B_r as ascending block-id lists: [B,H,n_qb,W_f*min(k_b,n_bpf)] int32."""
    lib = _load()
    W_f = frames.shape[-1]
    W_b = W_f * min(k_b, n_bpf(g))
    if out is None:
        out = torch.empty((g.B, g.H, n_qb, W_b), dtype=torch.int32, device=q_blk.device)
    qp = _exact(q_blk, "q_blk", torch.float32, (g.B, g.H, n_qb, g.d))
    fp = _exact(frames, "frames", torch.int32, (g.B, g.H, n_qb, W_f))
    op = _exact(out, "out", torch.int32, (g.B, g.H, n_qb, W_b))
    g = _frame_geom(g, n_kframes, [_pooled(k_blk, "k_blk", g, n_kframes, n_bpf(g))])
    _check(lib.lf_select_blocks(qp, k_blk.data_ptr(), g, n_qb, n_kframes, fp, W_f, k_b, op, _stream(q_blk)))
    return out


def lf_select(q_blk: torch.Tensor, k_frm: torch.Tensor, k_blk: torch.Tensor, g: Geom, n_qb: int,
              n_kframes: int, mem: Sequence[int], forced: Sequence[int], k_f: int, k_b: int,
              frames_out: Optional[torch.Tensor] = None, blocks_out: Optional[torch.Tensor] = None,
              with_frames: bool = True):
    """Both selection stages in one launch: (T_r [B,H,n_qb,W_f] or None, lists [B,H,n_qb,W_b])."""
    lib = _load()
    W_f = len(forced) + min(k_f, len(mem))
    W_b = max(W_f, 1) * min(k_b, n_bpf(g))
    dev = q_blk.device
    if frames_out is None and with_frames:
        frames_out = torch.empty((g.B, g.H, n_qb, max(W_f, 1)), dtype=torch.int32, device=dev)
    if blocks_out is None:
        blocks_out = torch.empty((g.B, g.H, n_qb, W_b), dtype=torch.int32, device=dev)
    qp = _exact(q_blk, "q_blk", torch.float32, (g.B, g.H, n_qb, g.d))
    fp = None if frames_out is None else _exact(frames_out, "frames_out", torch.int32, (g.B, g.H, n_qb, max(W_f, 1)))
    bp = _exact(blocks_out, "blocks_out", torch.int32, (g.B, g.H, n_qb, W_b))
    g = _frame_geom(g, n_kframes, [_pooled(k_frm, "k_frm", g, n_kframes, 1),
                                   _pooled(k_blk, "k_blk", g, n_kframes, n_bpf(g))])
    _check(lib.lf_select(qp, k_frm.data_ptr(), k_blk.data_ptr(), g, n_qb, n_kframes,
                         _i32_array(mem), len(mem), _i32_array(forced), len(forced), k_f, k_b,
                         fp, bp, _stream(q_blk)))
    return frames_out, blocks_out


def lf_select_blocks_1d(q_blk: torch.Tensor, k_blk: torch.Tensor, g: Geom, n_qb: int, n_kframes: int, K: int,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Single-level block top-K over the whole prefix: ascending lists [B,H,n_qb,K] int32."""
    lib = _load()
    if out is None:
        out = torch.empty((g.B, g.H, n_qb, K), dtype=torch.int32, device=q_blk.device)
    qp = _exact(q_blk, "q_blk", torch.float32, (g.B, g.H, n_qb, g.d))
    op = _exact(out, "out", torch.int32, (g.B, g.H, n_qb, K))
    g = _frame_geom(g, n_kframes, [_pooled(k_blk, "k_blk", g, n_kframes, n_bpf(g))])
    _check(lib.lf_select_blocks_1d(qp, k_blk.data_ptr(), g, n_qb, n_kframes, K, op, _stream(q_blk)))
    return out


def lf_sparse_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Geom, n_qframes: int,
                   n_kframes: int, blocks: torch.Tensor, scale: float,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block-sparse attention output [B,H,n_qframes*tpf,d] in q's dtype."""
    lib = _load()
    if out is None:
        out = torch.empty_like(q)
    if not (q.dtype == k.dtype == v.dtype == out.dtype):
        raise TypeError("q, k, v and out must share a dtype")
    lq, lk = n_qframes * g.tokens_per_frame, n_kframes * g.tokens_per_frame
    ga = g.with_stride(_shared("q and out", [_tokens(q, "q", g, lq), _tokens(out, "out", g, lq)], lq),
                       _shared("k and v", [_tokens(k, "k", g, lk), _tokens(v, "v", g, lk)], lk))
    if not isinstance(blocks, torch.Tensor) or blocks.dim() != 4:
        raise ValueError("blocks must be a 4-D int32 tensor [B, H, n_qb, W_b]")
    W_b = blocks.shape[-1]
    bp = _exact(blocks, "blocks", torch.int32, (g.B, g.H, n_qframes * n_bpf(g), W_b))
    _check(lib.lf_sparse_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              _dtype_code(q), ga, n_qframes, n_kframes, bp, W_b, float(scale), _stream(q)))
    return out


def lf_probe_mfma_bf16(n_wg: int, iters: int, sink: torch.Tensor, clocks: torch.Tensor) -> None:
    """Enqueues the dense bf16 MFMA loop (include/lf_probe.h) on the current stream:
    n_wg * 16 * iters * 32768 FLOPs; sink: float32 [n_wg * 256], clocks: int64 [2] (shader
    cycles and 100 MHz ticks of one wave's loop)."""
    if sink.dtype != torch.float32 or sink.numel() < n_wg * 256:
        raise ValueError("sink must be float32 with n_wg * 256 entries")
    if clocks.dtype != torch.int64 or clocks.numel() < 2:
        raise ValueError("clocks must be int64 with 2 entries")
    _check(_load().lf_probe_mfma_bf16(n_wg, iters, _dev(sink, "sink"), _dev(clocks, "clocks"), _stream(sink)))


def lf_probe_hbm_read(x: torch.Tensor, n_wg: int, sink: torch.Tensor) -> None:
    """Enqueues a plain streaming read of all of x's bytes (include/lf_probe.h) on the
    current stream; sink: float32 [n_wg * 256]."""
    if sink.dtype != torch.float32 or sink.numel() < n_wg * 256:
        raise ValueError("sink must be float32 with n_wg * 256 entries")
    _check(_load().lf_probe_hbm_read(_dev(x, "x"), x.numel() * x.element_size(), n_wg, _dev(sink, "sink"),
                                     _stream(x)))
