"""MI355X (gfx950) FlashAttention backward: Python binding of libfabwd.so.

The functions named like the C entry points (``attn_fwd_stats``,
``attn_bwd_preprocess``, ``attn_bwd``, ``attn_bwd_dq_convert``,
``attn_bwd_with_dq``) only marshal
arguments: they read shapes and device pointers from torch tensors, pass the
current HIP stream, and raise on a non-zero status.  Every step of the
computation runs in the library's kernels.  The library is loaded on first
use; a missing or unloadable ``libfabwd.so`` raises ``RuntimeError`` (there is
no fallback path).

``attention_forward`` / ``attention_backward`` allocate outputs and
workspaces with torch and chain the entry points on the current stream.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfabwd.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_MISALIGNED, ATTN_ERR_HIP = range(5)
ATTN_FP32, ATTN_BF16 = 0, 1

# Entry points declared in include/fabwd.h, with their argument types.
_P = ctypes.c_void_p
EXPORTS = {
    "attn_fwd_stats": [_P, _P, _P, _P, _P, _P, _P],
    "attn_bwd_preprocess": [_P, _P, _P, _P, _P, _P],
    "attn_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "attn_bwd_dq_convert": [_P, _P, _P, _P],
    "attn_bwd_with_dq": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "attn_bwd_with_dq_noalloc": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "attn_bwd_kernels": [_P, ctypes.c_int],
    "attn_status_str": [ctypes.c_int],
    "attn_version": [],
}


class attn_params(ctypes.Structure):
    """Mirror of ``struct attn_params`` in include/fabwd.h."""

    _fields_ = [
        ("B", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("H_kv", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("softcap", ctypes.c_float),
        ("deterministic", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("dropout_p", ctypes.c_float),
        ("rng_seed_lo", ctypes.c_uint32),
        ("rng_seed_hi", ctypes.c_uint32),
        ("rng_offset", ctypes.c_uint32),
    ]


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libfabwd.so once; raises RuntimeError when it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run `python -m flashattention_backward_pass_amd._build` "
            "(or __graft_entry__.build()) first; there is no fallback path")
    lib = ctypes.CDLL(path)
    for name, args in EXPORTS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name in ("attn_status_str", "attn_version", "attn_bwd_kernels") else ctypes.c_int
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().attn_status_str(int(status)).decode()


def make_params(B, H, H_kv, N, d, dtype, causal=False, scale=None, softcap=0.0, deterministic=0,
                window=None, dropout=None) -> attn_params:
    """window = (window_left, window_right) local mask, -1 = unbounded side; None = no window.
    dropout = (p, seed, offset): dropout probability, 64-bit generator seed, 32-bit counter offset."""
    if scale is None:
        scale = d ** -0.5
    wl, wr = (-1, -1) if window is None else window
    p_drop, seed, offset = (0.0, 0, 0) if dropout is None else dropout
    seed = int(seed)
    if not (0 <= seed < 1 << 64 and 0 <= int(offset) < 1 << 32):
        raise ValueError("dropout seed must fit 64 bits and offset 32 bits")
    return attn_params(int(B), int(H), int(H_kv), int(N), int(d), int(dtype), int(bool(causal)),
                       float(scale), float(softcap), int(deterministic), int(wl), int(wr), float(p_drop),
                       seed & 0xFFFFFFFF, seed >> 32, int(offset))


# ------------------------------------------------------------ torch marshalling
def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return ATTN_FP32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: use float32 or bfloat16")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous ([B, H, N, d] with d fastest)")
    if t.device.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _params_from(q, k, causal, scale, softcap, deterministic=False, window=None, dropout=None) -> attn_params:
    B, H, N, d = q.shape
    if k.dim() != 4 or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"K shape {tuple(k.shape)} does not match Q shape {tuple(q.shape)}")
    if k.dtype != q.dtype:
        raise TypeError("Q, K, V, O, dO must share one dtype")
    return make_params(B, H, k.shape[1], N, d, _dtype_code(q), causal, scale, softcap, int(bool(deterministic)),
                       window, dropout)


def _expect(t, shape, dtype, name):
    """Shape and dtype of a buffer the kernels read or write: the C interface
    receives bare pointers, so a wrong size must be caught here."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _check(status: int, where: str):
    if status != ATTN_OK:
        raise AttnError(status, where)


def attn_bwd_kernels(q, k, *, causal=False, scale=None, softcap=0.0, deterministic=False, window=None,
                     dropout=None, with_dq=True) -> str:
    """Kernel names (launch order, '+'-separated) that attn_bwd_with_dq (with_dq=True) or attn_bwd
    runs for these shapes on the current device."""
    p = _params_from(q, k, causal, scale, softcap, deterministic, window, dropout)
    r = load_library().attn_bwd_kernels(ctypes.byref(p), int(bool(with_dq)))
    if r is None:
        raise AttnError(ATTN_ERR_INVALID_ARG, "attn_bwd_kernels")
    return r.decode()


def attn_fwd_stats(q, k, v, o, lse, *, causal=False, scale=None, softcap=0.0, stream=None, window=None,
                   dropout=None):
    p = _params_from(q, k, causal, scale, softcap, window=window, dropout=dropout)
    f32 = _torch().float32
    _expect(v, k.shape, q.dtype, "V")
    _expect(o, q.shape, q.dtype, "O")
    _expect(lse, q.shape[:3], f32, "LSE")
    lib = load_library()
    _check(lib.attn_fwd_stats(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _stream(stream)),
           "attn_fwd_stats")


def attn_bwd_preprocess(o, do, D, dq_accum, *, H_kv=None, causal=False, scale=None, softcap=0.0, stream=None,
                        window=None):
    B, H, N, d = o.shape
    p = make_params(B, H, H_kv or H, N, d, _dtype_code(o), causal, scale, softcap, window=window)
    f32 = _torch().float32
    _expect(do, o.shape, o.dtype, "dO")
    _expect(D, (B, H, N), f32, "D")
    _expect(dq_accum, o.shape, f32, "dQaccum")
    lib = load_library()
    _check(lib.attn_bwd_preprocess(ctypes.byref(p), _ptr(o), _ptr(do), _ptr(D), _ptr(dq_accum), _stream(stream)),
           "attn_bwd_preprocess")


def _expect_bwd(q, k, v, do, lse, D, dq_accum, dk, dv):
    f32 = _torch().float32
    _expect(v, k.shape, q.dtype, "V")
    _expect(do, q.shape, q.dtype, "dO")
    _expect(lse, q.shape[:3], f32, "LSE")
    _expect(D, q.shape[:3], f32, "D")
    _expect(dq_accum, q.shape, f32, "dQaccum")
    _expect(dk, k.shape, q.dtype, "dK")
    _expect(dv, k.shape, q.dtype, "dV")


def attn_bwd(q, k, v, do, lse, D, dq_accum, dk, dv, *, causal=False, scale=None, softcap=0.0, stream=None,
             deterministic=False, window=None, dropout=None):
    p = _params_from(q, k, causal, scale, softcap, deterministic, window, dropout)
    _expect_bwd(q, k, v, do, lse, D, dq_accum, dk, dv)
    lib = load_library()
    _check(lib.attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(D),
                        _ptr(dq_accum), _ptr(dk), _ptr(dv), _stream(stream)), "attn_bwd")


def attn_bwd_with_dq(q, k, v, do, lse, D, dq_accum, dq, dk, dv, *, causal=False, scale=None, softcap=0.0,
                     stream=None, deterministic=False, window=None, dropout=None):
    p = _params_from(q, k, causal, scale, softcap, deterministic, window, dropout)
    _expect_bwd(q, k, v, do, lse, D, dq_accum, dk, dv)
    _expect(dq, q.shape, q.dtype, "dQ")
    lib = load_library()
    _check(lib.attn_bwd_with_dq(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(D),
                                _ptr(dq_accum), _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)), "attn_bwd_with_dq")


def attn_bwd_with_dq_noalloc(q, k, v, o, do, lse, dq, dk, dv, *, causal=False, scale=None, softcap=0.0,
                             stream=None, deterministic=False, window=None, dropout=None):
    """preprocess + attn_bwd_with_dq with the library's own static scratch (no allocation)."""
    p = _params_from(q, k, causal, scale, softcap, deterministic, window, dropout)
    f32 = _torch().float32
    _expect(v, k.shape, q.dtype, "V")
    _expect(o, q.shape, q.dtype, "O")
    _expect(do, q.shape, q.dtype, "dO")
    _expect(lse, q.shape[:3], f32, "LSE")
    _expect(dq, q.shape, q.dtype, "dQ")
    _expect(dk, k.shape, q.dtype, "dK")
    _expect(dv, k.shape, q.dtype, "dV")
    lib = load_library()
    _check(lib.attn_bwd_with_dq_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                                        _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)), "attn_bwd_with_dq_noalloc")


def attn_bwd_dq_convert(dq_accum, dq, *, scale=None, stream=None):
    B, H, N, d = dq.shape
    p = make_params(B, H, H, N, d, _dtype_code(dq), False, scale, 0.0)
    _expect(dq_accum, dq.shape, _torch().float32, "dQaccum")
    lib = load_library()
    _check(lib.attn_bwd_dq_convert(ctypes.byref(p), _ptr(dq_accum), _ptr(dq), _stream(stream)),
           "attn_bwd_dq_convert")


def attention_forward(q, k, v, *, causal=False, scale=None, softcap=0.0, stream=None, window=None, dropout=None):
    """Returns (O, LSE) from attn_fwd_stats; dropout = (p, seed, offset) or None."""
    torch = _torch()
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device=q.device, dtype=torch.float32)
    attn_fwd_stats(q, k, v, o, lse, causal=causal, scale=scale, softcap=softcap, stream=stream, window=window,
                   dropout=dropout)
    return o, lse


def attention_backward(q, k, v, o, do, lse, *, causal=False, scale=None, softcap=0.0, stream=None,
                       workspace=None, deterministic=False, window=None, dropout=None):
    """Returns (dQ, dK, dV): preprocess -> bwd_with_dq on one stream.

    ``dropout`` = (p, seed, offset) must be what the forward used.

    ``deterministic`` selects the atomic-free fp32 path (bf16 is atomic-free
    either way).
    ``workspace`` may pass preallocated ``(D, dQaccum)`` fp32 tensors of shapes
    [B, H, N] and [B, H, N, d].
    """
    torch = _torch()
    B, H, N, d = q.shape
    if workspace is None:
        D = torch.empty(B, H, N, device=q.device, dtype=torch.float32)
        acc = torch.empty(B, H, N, d, device=q.device, dtype=torch.float32)
    else:
        D, acc = workspace
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    attn_bwd_preprocess(o, do, D, acc, H_kv=k.shape[1], causal=causal, scale=scale, softcap=softcap, stream=stream,
                        window=window)
    attn_bwd_with_dq(q, k, v, do, lse, D, acc, dq, dk, dv, causal=causal, scale=scale, softcap=softcap,
                     stream=stream, deterministic=deterministic, window=window, dropout=dropout)
    return dq, dk, dv
