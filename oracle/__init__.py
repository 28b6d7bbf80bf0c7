"""CPU oracle for the RoPE apply path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  It wraps ``rope_oracle.c`` (a plain scalar C definition of both
operations, built with ``-O2 -ffp-contract=off``) through ctypes.  Tensors are plain PyTorch
CPU tensors, used as host memory only; all arithmetic happens in the C file.

Pages cited:
  [IPRM] "CANN ops-transformer 的 aclnnInplacePartialRotaryMul 算子：Inplace 部分旋转位置编码接口详解与实现剖析"
  [RSCC] "CANN ops-transformer 旋转位置编码算子 RopeWithSinCosCache 深度解析：cache 化 RoPE 的计算原理与 aclnn 两段式调用实战"
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from .build import LIB_PATH

OK = 0
ERR_PARAM_NULLPTR = 161001  # [IPRM §返回值与错误码]
ERR_PARAM_INVALID = 161002  # [IPRM §返回值与错误码]
ERR_OUTSIDE_CONTRACT = -1   # oracle only: a position outside the cache

_DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.int64: 3}


class OroTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"oracle library missing: {LIB_PATH} (run oracle.build.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.oro_rope_partial_inplace.argtypes = [
        P(OroTensor), P(OroTensor), P(OroTensor), ctypes.c_int64,
        P(ctypes.c_int64), ctypes.c_int64, P(ctypes.c_double)]
    lib.oro_rope_partial_inplace.restype = ctypes.c_int
    lib.oro_rope_partial_inplace_backward.argtypes = lib.oro_rope_partial_inplace.argtypes
    lib.oro_rope_partial_inplace_backward.restype = ctypes.c_int
    lib.oro_rope_with_cos_sin_cache.argtypes = [
        P(OroTensor), P(OroTensor), P(OroTensor), P(OroTensor),
        P(ctypes.c_int64), ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
        P(OroTensor), P(OroTensor), P(ctypes.c_double), P(ctypes.c_double)]
    lib.oro_rope_with_cos_sin_cache.restype = ctypes.c_int
    lib.oro_rope_with_cos_sin_cache_v2.argtypes = [
        P(OroTensor), P(OroTensor), P(OroTensor), P(OroTensor),
        P(ctypes.c_int64), ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
        P(OroTensor), P(OroTensor), P(ctypes.c_double), P(ctypes.c_double)]
    lib.oro_rope_with_cos_sin_cache_v2.restype = ctypes.c_int
    lib.oro_last_error.restype = ctypes.c_char_p
    for name in ("oro_round_bf16_array", "oro_round_f16_array"):
        getattr(lib, name).argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    lib.oro_f16_to_f32_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    lib.oro_round_bf16.argtypes = [ctypes.c_float]
    lib.oro_round_bf16.restype = ctypes.c_uint16
    lib.oro_round_f16.argtypes = [ctypes.c_float]
    lib.oro_round_f16.restype = ctypes.c_uint16
    lib.oro_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oro_bf16_to_f32.restype = ctypes.c_float
    lib.oro_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oro_f16_to_f32.restype = ctypes.c_float
    return lib


class _Lazy:
    """Loads the shared library on first use, so that ``oracle.build`` runs without it."""

    _lib = None

    def __getattr__(self, name):
        if _Lazy._lib is None:
            _Lazy._lib = _load()
        return getattr(_Lazy._lib, name)


_lib = _Lazy()


def _desc(t):
    """Descriptor of a CPU tensor (None -> NULL).  The tensor must stay alive for the call."""
    if t is None:
        return None
    if t.device.type != "cpu":
        raise ValueError("the oracle takes host tensors only")
    d = OroTensor()
    d.data = t.data_ptr() if t.numel() > 0 else 0
    d.dtype = _DTYPE_CODE.get(t.dtype, 99)
    d.ndim = t.dim()
    for i in range(min(t.dim(), 4)):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return ctypes.byref(d)


def _ints(seq):
    if seq is None:
        return None, 0
    arr = (ctypes.c_int64 * max(len(seq), 1))(*[int(v) for v in seq])
    return arr, len(seq)


def last_error() -> str:
    return _lib.oro_last_error().decode()


def rope_partial_inplace(x, cos, sin, rotary_mode=1, partial_slice=None, *, twin=False,
                         raw_desc=None):
    """Operation A on host tensors, in place on ``x`` ([IPRM §计算原理与公式]).

    Returns ``(status, x64)``: ``x64`` is the float64 twin (same shape as ``x``) when
    ``twin`` is set, else None.  ``raw_desc`` lets validation tests hand over hand-made
    descriptors (a dict name -> ctypes pointer or None) instead of tensors.
    """
    x64 = None
    x64p = None
    if twin:
        x64 = np.zeros(tuple(x.shape), dtype=np.float64)
        x64p = x64.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    sl, sl_len = _ints(partial_slice)
    if raw_desc is not None:
        dx, dc, ds = raw_desc["x"], raw_desc["cos"], raw_desc["sin"]
    else:
        dx, dc, ds = _desc(x), _desc(cos), _desc(sin)
    st = _lib.oro_rope_partial_inplace(dx, dc, ds, int(rotary_mode), sl, sl_len, x64p)
    return st, x64


def rope_partial_inplace_backward(g, cos, sin, rotary_mode=1, partial_slice=None, *,
                                  twin=False, raw_desc=None):
    """Gradient of operation A, in place on the incoming gradient ``g``: on each slice pair
    dx = (c0*g0 + s1*g1, c1*g1 - s0*g0), the transpose of the forward pair map
    ([IPRM §Python 接口与自动微分]).  Returns ``(status, g64)``."""
    g64 = None
    g64p = None
    if twin:
        g64 = np.zeros(tuple(g.shape), dtype=np.float64)
        g64p = g64.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    sl, sl_len = _ints(partial_slice)
    if raw_desc is not None:
        dg, dc, ds = raw_desc["x"], raw_desc["cos"], raw_desc["sin"]
    else:
        dg, dc, ds = _desc(g), _desc(cos), _desc(sin)
    st = _lib.oro_rope_partial_inplace_backward(dg, dc, ds, int(rotary_mode), sl, sl_len, g64p)
    return st, g64


def rope_with_cos_sin_cache(positions, query_in, key_in, cos_sin_cache, mrope_section,
                            head_size, is_neox_style, query_out, key_out, *, twin=False,
                            raw_desc=None, cache_mode=None):
    """Operation B on host tensors, writing ``query_out``/``key_out`` ([RSCC §设计动机]).
    ``cache_mode`` (not None) calls the V2 form ([RSCC §V2 接口：cacheMode 扩展]).

    Returns ``(status, q64, k64)`` where the float64 twins have the output shapes.
    """
    q64 = k64 = None
    q64p = k64p = None
    if twin:
        q64 = np.zeros(tuple(query_out.shape), dtype=np.float64)
        k64 = np.zeros(tuple(key_out.shape), dtype=np.float64)
        q64p = q64.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
        k64p = k64.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    ms, ms_len = _ints(mrope_section)
    if raw_desc is not None:
        descs = [raw_desc[k] for k in ("positions", "query_in", "key_in", "cache",
                                       "query_out", "key_out")]
    else:
        descs = [_desc(t) for t in (positions, query_in, key_in, cos_sin_cache,
                                    query_out, key_out)]
    if cache_mode is None:
        st = _lib.oro_rope_with_cos_sin_cache(descs[0], descs[1], descs[2], descs[3], ms, ms_len,
                                              int(head_size), int(bool(is_neox_style)),
                                              descs[4], descs[5], q64p, k64p)
    else:
        st = _lib.oro_rope_with_cos_sin_cache_v2(descs[0], descs[1], descs[2], descs[3], ms,
                                                 ms_len, int(head_size),
                                                 int(bool(is_neox_style)), int(cache_mode),
                                                 descs[4], descs[5], q64p, k64p)
    return st, q64, k64


# ---- rounding routines (exposed for their own exhaustive tests) -------------------------

def round_bf16_bits(f32: np.ndarray) -> np.ndarray:
    f32 = np.ascontiguousarray(f32, dtype=np.float32)
    out = np.empty(f32.shape, dtype=np.uint16)
    _lib.oro_round_bf16_array(f32.ctypes.data, out.ctypes.data, f32.size)
    return out


def round_f16_bits(f32: np.ndarray) -> np.ndarray:
    f32 = np.ascontiguousarray(f32, dtype=np.float32)
    out = np.empty(f32.shape, dtype=np.uint16)
    _lib.oro_round_f16_array(f32.ctypes.data, out.ctypes.data, f32.size)
    return out


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    _lib.oro_f16_to_f32_array(bits.ctypes.data, out.ctypes.data, bits.size)
    return out


def bf16_bits_to_f32(bits: int) -> float:
    return _lib.oro_bf16_to_f32(int(bits))
