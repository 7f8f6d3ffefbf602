"""MI355X (gfx950) GQA attention backward: thin Python binding of the C ABI.

The functions here carry the names of the C entry points declared in
``include/attn_bwd.h`` and only marshal arguments: they check tensor
dtypes/shapes/devices, pass raw device pointers and the current HIP stream,
and raise :class:`AttnError` on a non-zero status.  All computation happens in
the HIP kernels of ``libattn_bwd.so``; there is no CPU fallback.  If the
library has not been built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "AttnError",
    "Shape",
    "lib",
    "attn_fwd",
    "attn_bwd_preprocess",
    "attn_bwd",
    "attn_bwd_postprocess",
    "attn_bwd_dkdv",
    "attn_bwd_dq",
    "attn_bwd_dsink",
    "attn_bwd_dq_delta",
    "attn_bwd_split",
    "attn_bwd_dkv_reduce",
    "attn_bwd_static",
    "attn_bwd_fused_cast",
    "fused_cast_counters",
    "MAX_SPLIT",
    "STATIC_SCRATCH_BYTES",
    "attn_abi_version",
    "LIB_PATH",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn_bwd.so")

ATTN_F16, ATTN_BF16 = 0, 1
ATTN_LAYOUT_THD, ATTN_LAYOUT_BHSD = 0, 1
MAX_SPLIT = 16  # ATTN_MAX_SPLIT
STATIC_SCRATCH_BYTES = 64 * 1024 * 1024  # ATTN_STATIC_SCRATCH_BYTES
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED", 3: "ATTN_ERR_HIP"}


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Shape(ctypes.Structure):
    """Mirror of ``attn_shape_t``."""

    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32),
        ("total_tokens", ctypes.c_int32),
        ("hq", ctypes.c_int32),
        ("hkv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("layout", ctypes.c_int32),
    ]

    @classmethod
    def make(cls, *, num_seqs, max_seqlen, total_tokens, hq, hkv, head_dim, causal, window,
             scale, dtype, layout="thd") -> "Shape":
        if not isinstance(dtype, int):
            dtype = _dtype_code(dtype)
        if not isinstance(layout, int):
            layout = {"thd": ATTN_LAYOUT_THD, "bhsd": ATTN_LAYOUT_BHSD}[layout]
        return cls(int(num_seqs), int(max_seqlen), int(total_tokens), int(hq), int(hkv),
                   int(head_dim), int(bool(causal)), int(window), float(scale), int(dtype),
                   int(layout))


_lib = None


def lib() -> ctypes.CDLL:
    """Load ``libattn_bwd.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m atomics_bwd_preprocess_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.c_void_p, ctypes.POINTER(Shape)
        sig = {
            "attn_fwd": [S, P, P, P, P, P, P, P, P],
            "attn_bwd_preprocess": [S, P, P, P, P, P, P, P, P, P],
            "attn_bwd": [S, P, P, P, P, P, P, P, P, P, P, P],
            "attn_bwd_postprocess": [S, P, P, P],
            "attn_bwd_dkdv": [S, P, P, P, P, P, P, P, P, P, P],
            "attn_bwd_dq": [S, P, P, P, P, P, P, P, P, P],
            "attn_bwd_dsink": [S, P, P, P, P, P],
            "attn_bwd_dq_delta": [S, P, P, P, P, P, P, P, P, P, P],
            "attn_bwd_split": [S, P, P, P, P, P, P, P, P, P, ctypes.c_int32, P],
            "attn_bwd_dkv_reduce": [S, P, ctypes.c_int32, P, P, P],
            "attn_bwd_static": [S, P, P, P, P, P, P, P, P, P, P, P],
            "attn_bwd_fused_cast": [S, P, P, P, P, P, P, P, P, P, P, P, P, P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.attn_status_string.argtypes = [ctypes.c_int]
        L.attn_status_string.restype = ctypes.c_char_p
        L.attn_last_error.argtypes = []
        L.attn_last_error.restype = ctypes.c_char_p
        L.attn_abi_version.argtypes = []
        L.attn_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def attn_abi_version() -> int:
    return lib().attn_abi_version()


def _check(status: int) -> None:
    if status != 0:
        raise AttnError(status, lib().attn_last_error().decode())


def _dtype_code(dt) -> int:
    import torch

    if dt in (torch.float16, "f16", "fp16"):
        return ATTN_F16
    if dt in (torch.bfloat16, "bf16"):
        return ATTN_BF16
    raise AttnError(2, f"unsupported dtype {dt}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(t, name, dtype, shape, allow_none=False):
    import torch

    if t is None:
        if allow_none:
            return
        raise AttnError(1, f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise AttnError(1, f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise AttnError(1, f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise AttnError(1, f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise AttnError(1, f"{name} must be contiguous")


def _dims(shape: Shape):
    import torch

    T, Hq, Hkv, D = shape.total_tokens, shape.hq, shape.hkv, shape.head_dim
    dt = torch.float16 if shape.dtype == ATTN_F16 else torch.bfloat16
    return T, Hq, Hkv, D, dt


def qshape(shape: Shape) -> tuple:
    """Shape of q, o, dout, dq and dq_accum for the shape's layout."""
    if shape.layout == ATTN_LAYOUT_BHSD:
        return (shape.num_seqs, shape.hq, shape.max_seqlen, shape.head_dim)
    return (shape.total_tokens, shape.hq, shape.head_dim)


def kvshape(shape: Shape) -> tuple:
    """Shape of k, v, dk and dv for the shape's layout."""
    if shape.layout == ATTN_LAYOUT_BHSD:
        return (shape.num_seqs, shape.hkv, shape.max_seqlen, shape.head_dim)
    return (shape.total_tokens, shape.hkv, shape.head_dim)


def _cu(shape: Shape, cu_seqlens):
    import torch

    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (shape.num_seqs + 1,))
    return _ptr(cu_seqlens)


def attn_fwd(shape: Shape, q, k, v, cu_seqlens, sink, o, lse, stream=None) -> None:
    """Forward: writes ``o`` [T,Hq,D] and ``lse`` [Hq,T] (fp32)."""
    import torch

    T, Hq, Hkv, D, dt = _dims(shape)
    _need(q, "q", dt, qshape(shape))
    _need(k, "k", dt, kvshape(shape))
    _need(v, "v", dt, kvshape(shape))
    _need(sink, "sink", torch.float32, (Hq,), allow_none=True)
    _need(o, "o", dt, qshape(shape))
    _need(lse, "lse", torch.float32, (Hq, T))
    _check(lib().attn_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _cu(shape, cu_seqlens),
                          _ptr(sink), _ptr(o), _ptr(lse), _stream(stream)))


def attn_bwd_preprocess(shape: Shape, o, dout, lse, cu_seqlens, sink, delta, dq_accum, dsink,
                        stream=None) -> None:
    """Delta = rowsum(O * dO) [Hq,T]; dq_accum := 0 unless it is None; dsink [Hq] if a sink
    is given."""
    import torch

    T, Hq, Hkv, D, dt = _dims(shape)
    _need(o, "o", dt, qshape(shape))
    _need(dout, "dout", dt, qshape(shape))
    _need(lse, "lse", torch.float32, (Hq, T), allow_none=sink is None)
    _need(sink, "sink", torch.float32, (Hq,), allow_none=True)
    _need(delta, "delta", torch.float32, (Hq, T))
    _need(dq_accum, "dq_accum", torch.float32, qshape(shape), allow_none=True)
    _need(dsink, "dsink", torch.float32, (Hq,), allow_none=True)
    _check(lib().attn_bwd_preprocess(ctypes.byref(shape), _ptr(o), _ptr(dout), _ptr(lse),
                                     _cu(shape, cu_seqlens), _ptr(sink), _ptr(delta),
                                     _ptr(dq_accum), _ptr(dsink), _stream(stream)))


def attn_bwd(shape: Shape, q, k, v, dout, lse, delta, cu_seqlens, dq_accum, dk, dv,
             stream=None) -> None:
    """Main backward: accumulates dQ / scale into dq_accum (atomics), writes dk, dv."""
    import torch

    T, Hq, Hkv, D, dt = _dims(shape)
    _need(q, "q", dt, qshape(shape))
    _need(k, "k", dt, kvshape(shape))
    _need(v, "v", dt, kvshape(shape))
    _need(dout, "dout", dt, qshape(shape))
    _need(lse, "lse", torch.float32, (Hq, T))
    _need(delta, "delta", torch.float32, (Hq, T))
    _need(dq_accum, "dq_accum", torch.float32, qshape(shape))
    _need(dk, "dk", dt, kvshape(shape))
    _need(dv, "dv", dt, kvshape(shape))
    _check(lib().attn_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                          _ptr(delta), _cu(shape, cu_seqlens), _ptr(dq_accum), _ptr(dk), _ptr(dv),
                          _stream(stream)))


def attn_bwd_postprocess(shape: Shape, dq_accum, dq, stream=None) -> None:
    """dq = RNE cast of scale * dq_accum (fp32 multiply; dq_accum holds dQ / scale)."""
    import torch

    T, Hq, Hkv, D, dt = _dims(shape)
    _need(dq_accum, "dq_accum", torch.float32, qshape(shape))
    _need(dq, "dq", dt, qshape(shape))
    _check(lib().attn_bwd_postprocess(ctypes.byref(shape), _ptr(dq_accum), _ptr(dq),
                                      _stream(stream)))


def attn_bwd_dkdv(shape: Shape, q, k, v, dout, lse, delta, cu_seqlens, dk, dv,
                  stream=None) -> None:
    """Main backward without its dQ product: writes dk, dv (no atomics)."""
    import torch

    T, Hq, Hkv, D, dt = _dims(shape)
    _need(q, "q", dt, qshape(shape))
    _need(k, "k", dt, kvshape(shape))
    _need(v, "v", dt, kvshape(shape))
    _need(dout, "dout", dt, qshape(shape))
    _need(lse, "lse", torch.float32, (Hq, T))
    _need(delta, "delta", torch.float32, (Hq, T))
    _need(dk, "dk", dt, kvshape(shape))
    _need(dv, "dv", dt, kvshape(shape))
    _check(lib().attn_bwd_dkdv(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                               _ptr(lse), _ptr(delta), _cu(shape, cu_seqlens), _ptr(dk), _ptr(dv),
                               _stream(stream)))


def attn_bwd_dq(shape: Shape, q, k, v, dout, lse, delta, cu_seqlens, dq, stream=None) -> None:
    """Query-stationary dQ: writes dq once in the storage dtype (no atomics)."""
    import torch

    T, Hq, Hkv, D, dt = _dims(shape)
    _need(q, "q", dt, qshape(shape))
    _need(k, "k", dt, kvshape(shape))
    _need(v, "v", dt, kvshape(shape))
    _need(dout, "dout", dt, qshape(shape))
    _need(lse, "lse", torch.float32, (Hq, T))
    _need(delta, "delta", torch.float32, (Hq, T))
    _need(dq, "dq", dt, qshape(shape))
    _check(lib().attn_bwd_dq(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                             _ptr(lse), _ptr(delta), _cu(shape, cu_seqlens), _ptr(dq),
                             _stream(stream)))


def attn_bwd_dq_delta(shape: Shape, q, k, v, o, dout, lse, cu_seqlens, delta, dq,
                      stream=None) -> None:
    """Query-stationary dQ that also forms Delta from O and dO (written to delta),
    bitwise as attn_bwd_preprocess does; no preprocess needed before it."""
    import torch

    T, Hq, Hkv, D, dt = _dims(shape)
    _need(q, "q", dt, qshape(shape))
    _need(k, "k", dt, kvshape(shape))
    _need(v, "v", dt, kvshape(shape))
    _need(o, "o", dt, qshape(shape))
    _need(dout, "dout", dt, qshape(shape))
    _need(lse, "lse", torch.float32, (Hq, T))
    _need(delta, "delta", torch.float32, (Hq, T))
    _need(dq, "dq", dt, qshape(shape))
    _check(lib().attn_bwd_dq_delta(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                   _ptr(dout), _ptr(lse), _cu(shape, cu_seqlens), _ptr(delta),
                                   _ptr(dq), _stream(stream)))


def attn_bwd_dsink(shape: Shape, lse, delta, sink, dsink, stream=None) -> None:
    """dsink = -sum_t exp(sink - lse) * delta per query head (delta already written)."""
    import torch

    T, Hq, Hkv, D, dt = _dims(shape)
    _need(lse, "lse", torch.float32, (Hq, T))
    _need(delta, "delta", torch.float32, (Hq, T))
    _need(sink, "sink", torch.float32, (Hq,))
    _need(dsink, "dsink", torch.float32, (Hq,))
    _check(lib().attn_bwd_dsink(ctypes.byref(shape), _ptr(lse), _ptr(delta), _ptr(sink),
                                _ptr(dsink), _stream(stream)))


def dkv_partial_shape(shape: Shape, nsplit: int) -> tuple:
    """Shape of the fp32 dK / dV partial workspace of attn_bwd_split."""
    return (int(nsplit), 2) + kvshape(shape)


def attn_bwd_split(shape: Shape, q, k, v, dout, lse, delta, cu_seqlens, dq_accum, dkv_partial,
                   nsplit: int, stream=None) -> None:
    """Main backward with every key block's pairs split over nsplit workgroups: dQ / scale
    into dq_accum (atomics; None: no dQ product), fp32 dK / dV partials into dkv_partial."""
    import torch

    T, Hq, Hkv, D, dt = _dims(shape)
    _need(q, "q", dt, qshape(shape))
    _need(k, "k", dt, kvshape(shape))
    _need(v, "v", dt, kvshape(shape))
    _need(dout, "dout", dt, qshape(shape))
    _need(lse, "lse", torch.float32, (Hq, T))
    _need(delta, "delta", torch.float32, (Hq, T))
    _need(dq_accum, "dq_accum", torch.float32, qshape(shape), allow_none=True)
    _need(dkv_partial, "dkv_partial", torch.float32, dkv_partial_shape(shape, nsplit))
    _check(lib().attn_bwd_split(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                _ptr(lse), _ptr(delta), _cu(shape, cu_seqlens), _ptr(dq_accum),
                                _ptr(dkv_partial), int(nsplit), _stream(stream)))


def attn_bwd_dkv_reduce(shape: Shape, dkv_partial, nsplit: int, dk, dv, stream=None) -> None:
    """dk, dv = RNE casts of the fixed-order sums of the nsplit partial slots."""
    import torch

    T, Hq, Hkv, D, dt = _dims(shape)
    _need(dkv_partial, "dkv_partial", torch.float32, dkv_partial_shape(shape, nsplit))
    _need(dk, "dk", dt, kvshape(shape))
    _need(dv, "dv", dt, kvshape(shape))
    _check(lib().attn_bwd_dkv_reduce(ctypes.byref(shape), _ptr(dkv_partial), int(nsplit),
                                     _ptr(dk), _ptr(dv), _stream(stream)))


def attn_bwd_static(shape: Shape, q, k, v, dout, lse, delta, cu_seqlens, dq, dk, dv,
                    stream=None) -> None:
    """attn_bwd + attn_bwd_postprocess with the fp32 dQ accumulator in the library's own
    scratch array (no workspace, nothing allocated); writes dq, dk, dv.  Calls that overlap
    on one GPU race (the array is shared); T * Hq * D * 4 must fit STATIC_SCRATCH_BYTES."""
    import torch

    T, Hq, Hkv, D, dt = _dims(shape)
    _need(q, "q", dt, qshape(shape))
    _need(k, "k", dt, kvshape(shape))
    _need(v, "v", dt, kvshape(shape))
    _need(dout, "dout", dt, qshape(shape))
    _need(lse, "lse", torch.float32, (Hq, T))
    _need(delta, "delta", torch.float32, (Hq, T))
    _need(dq, "dq", dt, qshape(shape))
    _need(dk, "dk", dt, kvshape(shape))
    _need(dv, "dv", dt, kvshape(shape))
    _check(lib().attn_bwd_static(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                 _ptr(lse), _ptr(delta), _cu(shape, cu_seqlens), _ptr(dq),
                                 _ptr(dk), _ptr(dv), _stream(stream)))


def fused_cast_counters(shape: Shape) -> int:
    """ATTN_FUSED_CAST_COUNTERS: int32 arrival counters attn_bwd_fused_cast needs."""
    n = shape.num_seqs * shape.hq * ((shape.max_seqlen + 31) // 32)
    return (n + 3) // 4 * 4


def attn_bwd_fused_cast(shape: Shape, q, k, v, dout, lse, delta, cu_seqlens, dq_accum, counters,
                        dq, dk, dv, stream=None) -> None:
    """attn_bwd + attn_bwd_postprocess in one pass for causal problems: the last workgroup
    contributing to a query block casts it (arrival counters, zeroed by the call); writes
    dq, dk, dv.  dq_accum must have been zeroed by attn_bwd_preprocess."""
    import torch

    T, Hq, Hkv, D, dt = _dims(shape)
    _need(q, "q", dt, qshape(shape))
    _need(k, "k", dt, kvshape(shape))
    _need(v, "v", dt, kvshape(shape))
    _need(dout, "dout", dt, qshape(shape))
    _need(lse, "lse", torch.float32, (Hq, T))
    _need(delta, "delta", torch.float32, (Hq, T))
    _need(dq_accum, "dq_accum", torch.float32, qshape(shape))
    _need(counters, "counters", torch.int32, (fused_cast_counters(shape),))
    _need(dq, "dq", dt, qshape(shape))
    _need(dk, "dk", dt, kvshape(shape))
    _need(dv, "dv", dt, kvshape(shape))
    _check(lib().attn_bwd_fused_cast(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                     _ptr(lse), _ptr(delta), _cu(shape, cu_seqlens),
                                     _ptr(dq_accum), _ptr(counters), _ptr(dq), _ptr(dk),
                                     _ptr(dv), _stream(stream)))
