"""Python binding of librope_amd.so, the MI355X (gfx950) RoPE apply library.

Argument marshalling only: tensors are described (pointer, dtype, shape, strides) and handed
to the C ABI declared in ``include/rope.h`` together with the current HIP stream; every step
of both operations runs in the library's HIP kernels.  PyTorch provides device memory and
streams.  There is no fallback: if the library is not built this import fails.

  rope_partial_inplace(x, cos, sin, rotary_mode=1, partial_slice=None, stream=None)
  rope_partial_inplace_backward(g, cos, sin, rotary_mode=1, partial_slice=None, stream=None)
  InplacePartialRotaryMul.apply(x, cos, sin, partial_slice, rotary_mode)
                                                  (autograd; x must not be a leaf)
  inplace_partial_rotary_mul(x, r1, r2, *, rotary_mode="interleave", partial_slice=None)
  inplace_partial_rotary_mul_backward(grad, r1, r2, *, rotary_mode="interleave",
                                      partial_slice=None)
                                                  (the pages' Python interface: same calls,
                                                  autograd when x requires grad)
  rope_with_cos_sin_cache(positions, query_in, key_in, cos_sin_cache, mrope_section,
                          head_size, is_neox_style, query_out=None, key_out=None, stream=None)
  rope_with_cos_sin_cache_v2(..., is_neox_style, cache_mode, query_out=None, ...)

Pages defining the operations:
  [IPRM] "CANN ops-transformer 的 aclnnInplacePartialRotaryMul 算子：Inplace 部分旋转位置编码接口详解与实现剖析"
  [RSCC] "CANN ops-transformer 旋转位置编码算子 RopeWithSinCosCache 深度解析：cache 化 RoPE 的计算原理与 aclnn 两段式调用实战"
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

ROPE_OK = 0
ROPE_ERR_PARAM_NULLPTR = 161001
ROPE_ERR_PARAM_INVALID = 161002
ROPE_ERR_RUNTIME = 361001

ROPE_F32, ROPE_F16, ROPE_BF16, ROPE_I64 = 0, 1, 2, 3


class RopeTensor(ctypes.Structure):
    """Mirror of ``rope_tensor`` in include/rope.h."""

    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


class RopeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"rope error {code}: {message}")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python __graft_entry__.py` at the repository root")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.rope_partial_inplace.argtypes = [P(RopeTensor), P(RopeTensor), P(RopeTensor),
                                         ctypes.c_int64, P(ctypes.c_int64), ctypes.c_int64,
                                         ctypes.c_void_p]
    lib.rope_partial_inplace.restype = ctypes.c_int
    lib.rope_partial_inplace_backward.argtypes = lib.rope_partial_inplace.argtypes
    lib.rope_partial_inplace_backward.restype = ctypes.c_int
    lib.rope_with_cos_sin_cache.argtypes = [P(RopeTensor), P(RopeTensor), P(RopeTensor),
                                            P(RopeTensor), P(ctypes.c_int64), ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_int, P(RopeTensor),
                                            P(RopeTensor), ctypes.c_void_p]
    lib.rope_with_cos_sin_cache.restype = ctypes.c_int
    lib.rope_with_cos_sin_cache_v2.argtypes = [P(RopeTensor), P(RopeTensor), P(RopeTensor),
                                               P(RopeTensor), P(ctypes.c_int64), ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                               P(RopeTensor), P(RopeTensor), ctypes.c_void_p]
    lib.rope_with_cos_sin_cache_v2.restype = ctypes.c_int
    lib.rope_last_error.argtypes = []
    lib.rope_last_error.restype = ctypes.c_char_p
    return lib


LIB = _load()


def last_error() -> str:
    return LIB.rope_last_error().decode()


def _dtype_code(t) -> int:
    import torch
    return {torch.float32: ROPE_F32, torch.float16: ROPE_F16, torch.bfloat16: ROPE_BF16,
            torch.int64: ROPE_I64}.get(t.dtype, 99)


def describe(t) -> RopeTensor:
    """A ``rope_tensor`` describing a torch tensor (which must outlive the call)."""
    if t.dim() > 4:
        raise RopeError(ROPE_ERR_PARAM_INVALID, "tensors of more than 4 dims are not supported")
    d = RopeTensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = _dtype_code(t)
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _int_array(values):
    if values is None:
        return None, 0
    vals = [int(v) for v in values]
    return (ctypes.c_int64 * max(len(vals), 1))(*vals), len(vals)


def _device_of(tensors):
    dev = None
    for t in tensors:
        if t is None or t.numel() == 0:
            continue
        if not t.is_cuda:
            raise RopeError(ROPE_ERR_PARAM_INVALID,
                            "tensors must live in GPU memory (torch device 'cuda')")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise RopeError(ROPE_ERR_PARAM_INVALID, "tensors are on different devices")
    return dev


def _stream_handle(stream, dev):
    import torch
    if stream is None:
        if dev is None:
            return None
        stream = torch.cuda.current_stream(dev)
    return getattr(stream, "cuda_stream", stream)


def _check(code: int):
    if code != ROPE_OK:
        raise RopeError(code, last_error())


def _on_device(dev, fn, args) -> int:
    """fn(*args) with the tensors' GPU as the current HIP device: the library launches on the
    current device, which must own the stream and the tensors."""
    import torch
    if dev is None or dev.index is None or dev.index == torch.cuda.current_device():
        return fn(*args)
    with torch.cuda.device(dev):
        return fn(*args)


def rope_partial_inplace(x, cos, sin, rotary_mode: int = 1, partial_slice=None, stream=None):
    """In-place partial RoPE on x[..., start:end) ([IPRM §计算原理与公式]): rotary_mode 1
    interleave, 0 half mode (x1, x2 the two halves of the slice)."""
    dev = _device_of([x, cos, sin])
    dx, dc, ds = describe(x), describe(cos), describe(sin)
    sl, sl_len = _int_array(partial_slice)
    _check(_on_device(dev, LIB.rope_partial_inplace,
                      (ctypes.byref(dx), ctypes.byref(dc), ctypes.byref(ds), int(rotary_mode),
                       sl, sl_len, _stream_handle(stream, dev))))


def rope_partial_inplace_backward(g, cos, sin, rotary_mode: int = 1, partial_slice=None,
                                  stream=None):
    """Gradient of rope_partial_inplace with respect to x, in place on the incoming gradient
    ``g`` ([IPRM §Python 接口与自动微分]; the transpose of the forward pair map)."""
    dev = _device_of([g, cos, sin])
    dg, dc, ds = describe(g), describe(cos), describe(sin)
    sl, sl_len = _int_array(partial_slice)
    _check(_on_device(dev, LIB.rope_partial_inplace_backward,
                      (ctypes.byref(dg), ctypes.byref(dc), ctypes.byref(ds), int(rotary_mode),
                       sl, sl_len, _stream_handle(stream, dev))))


def _autograd_function():
    import torch

    class InplacePartialRotaryMul(torch.autograd.Function):
        """Autograd wrapper ([IPRM §Python 接口与自动微分]): forward rotates x in place and marks
        it dirty; backward runs the backward kernel on a contiguous copy of the incoming
        gradient; cos and sin get no gradient."""

        @staticmethod
        def forward(ctx, x, cos, sin, partial_slice=None, rotary_mode=1):
            rope_partial_inplace(x, cos, sin, rotary_mode, partial_slice)
            ctx.mark_dirty(x)
            ctx.save_for_backward(cos, sin)
            ctx.partial_slice = partial_slice
            ctx.rotary_mode = rotary_mode
            return x

        @staticmethod
        def backward(ctx, grad):
            cos, sin = ctx.saved_tensors
            g = grad.contiguous().clone()
            rope_partial_inplace_backward(g, cos, sin, ctx.rotary_mode, ctx.partial_slice)
            return g, None, None, None, None

    return InplacePartialRotaryMul


def __getattr__(name):
    if name == "InplacePartialRotaryMul":
        fn = _autograd_function()
        globals()[name] = fn
        return fn
    raise AttributeError(name)


_ROTARY_MODES = {"interleave": 1, "half": 0}


def _rotary_mode_code(rotary_mode) -> int:
    if isinstance(rotary_mode, str):
        if rotary_mode not in _ROTARY_MODES:
            raise RopeError(ROPE_ERR_PARAM_INVALID,
                            f"rotary_mode {rotary_mode!r}: 'interleave' or 'half' (or 1 / 0)")
        return _ROTARY_MODES[rotary_mode]
    return int(rotary_mode)


def inplace_partial_rotary_mul(x, r1, r2, *, rotary_mode="interleave", partial_slice=None):
    """The Python interface of [IPRM §Python 接口与自动微分]: rotates x in place (r1 = cos,
    r2 = sin) and returns None.  rotary_mode is "interleave" (1) or "half" (0, reading R21).
    When autograd records x (x requires grad and grad mode is on), the call goes through
    InplacePartialRotaryMul, so the gradient of x comes from the backward kernel and r1, r2 get
    none; x must then not be a leaf (rotate a copy such as ``y = x * 1.0``)."""
    import torch
    mode = _rotary_mode_code(rotary_mode)
    if x.requires_grad and torch.is_grad_enabled():
        __getattr__("InplacePartialRotaryMul").apply(x, r1, r2, partial_slice, mode)
    else:
        rope_partial_inplace(x, r1, r2, mode, partial_slice)


def inplace_partial_rotary_mul_backward(grad, r1, r2, *, rotary_mode="interleave",
                                        partial_slice=None):
    """The gradient op named by [IPRM §Python 接口与自动微分], in place on ``grad`` (the
    transpose of each slice pair's rotation; outside the slice the gradient passes through).
    Returns None."""
    rope_partial_inplace_backward(grad, r1, r2, _rotary_mode_code(rotary_mode), partial_slice)


def _cache_args(positions, query_in, key_in, cos_sin_cache, mrope_section, head_size,
                is_neox_style, cache_mode, query_out, key_out, stream):
    """(C function, its arguments, objects to keep alive) of one cos/sin-cache call: the V1
    entry point when cache_mode is None, else the V2 one."""
    tensors = (positions, query_in, key_in, cos_sin_cache, query_out, key_out)
    dev = _device_of(list(tensors))
    descs = [describe(t) for t in tensors]
    ms, ms_len = _int_array(mrope_section)
    head = (ctypes.byref(descs[0]), ctypes.byref(descs[1]), ctypes.byref(descs[2]),
            ctypes.byref(descs[3]), ms, ms_len, int(head_size), int(bool(is_neox_style)))
    tail = (ctypes.byref(descs[4]), ctypes.byref(descs[5]), _stream_handle(stream, dev))
    if cache_mode is None:
        return LIB.rope_with_cos_sin_cache, head + tail, (tensors, descs, ms), dev
    return (LIB.rope_with_cos_sin_cache_v2, head + (int(cache_mode),) + tail,
            (tensors, descs, ms), dev)


def _with_cos_sin_cache(positions, query_in, key_in, cos_sin_cache, mrope_section, head_size,
                        is_neox_style, cache_mode, query_out, key_out, stream):
    import torch
    if head_size is None:
        head_size = cos_sin_cache.shape[-1]
    if query_out is None:
        query_out = torch.empty(query_in.shape, dtype=query_in.dtype, device=query_in.device)
    if key_out is None:
        key_out = torch.empty(key_in.shape, dtype=key_in.dtype, device=key_in.device)
    fn, args, _keep, dev = _cache_args(positions, query_in, key_in, cos_sin_cache,
                                       mrope_section, head_size, is_neox_style, cache_mode,
                                       query_out, key_out, stream)
    _check(_on_device(dev, fn, args))
    return query_out, key_out


def rope_with_cos_sin_cache(positions, query_in, key_in, cos_sin_cache, mrope_section=None,
                            head_size: int | None = None, is_neox_style: bool = True,
                            query_out=None, key_out=None, stream=None):
    """RoPE with a cos/sin cache ([RSCC §设计动机]); returns (query_out, key_out).

    Outputs are allocated (contiguous) when not given; ``head_size`` defaults to the cache's
    rotaryDim."""
    return _with_cos_sin_cache(positions, query_in, key_in, cos_sin_cache, mrope_section,
                               head_size, is_neox_style, None, query_out, key_out, stream)


def rope_with_cos_sin_cache_v2(positions, query_in, key_in, cos_sin_cache, mrope_section=None,
                               head_size: int | None = None, is_neox_style: bool = True,
                               cache_mode: int = 0, query_out=None, key_out=None, stream=None):
    """The V2 form with ``cache_mode`` ([RSCC §V2 接口：cacheMode 扩展]): 0 sectioned,
    1 interleaved mrope stitching.  Other arguments as rope_with_cos_sin_cache."""
    return _with_cos_sin_cache(positions, query_in, key_in, cos_sin_cache, mrope_section,
                               head_size, is_neox_style, int(cache_mode), query_out, key_out,
                               stream)


class PreparedCall:
    """A call whose arguments are marshalled once (for tight launch loops): invoking it
    issues exactly one C-ABI call with the prebuilt descriptors.  The tensors must stay
    alive and keep their storage while the object is used."""

    def __init__(self, fn, args, keep, dev=None):
        self._fn, self._args, self._keep, self._dev = fn, args, keep, dev

    def __call__(self) -> None:
        _check(_on_device(self._dev, self._fn, self._args))


def prepare_partial_inplace(x, cos, sin, rotary_mode: int = 1, partial_slice=None,
                            stream=None, backward: bool = False) -> PreparedCall:
    dev = _device_of([x, cos, sin])
    dx, dc, ds = describe(x), describe(cos), describe(sin)
    sl, sl_len = _int_array(partial_slice)
    args = (ctypes.byref(dx), ctypes.byref(dc), ctypes.byref(ds), int(rotary_mode), sl, sl_len,
            _stream_handle(stream, dev))
    fn = LIB.rope_partial_inplace_backward if backward else LIB.rope_partial_inplace
    return PreparedCall(fn, args, (x, cos, sin, dx, dc, ds, sl), dev)


def prepare_with_cos_sin_cache(positions, query_in, key_in, cos_sin_cache, mrope_section,
                               head_size, is_neox_style, query_out, key_out, stream=None,
                               cache_mode: int | None = None) -> PreparedCall:
    """cache_mode None: the V1 entry point; else the V2 one with that cacheMode."""
    fn, args, keep, dev = _cache_args(positions, query_in, key_in, cos_sin_cache, mrope_section,
                                      head_size, is_neox_style, cache_mode, query_out, key_out,
                                      stream)
    return PreparedCall(fn, args, keep, dev)
