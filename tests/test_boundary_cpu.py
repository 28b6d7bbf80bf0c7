"""CPU tests of the C-ABI boundary (no kernel runs here).

* the library loads on a machine without a GPU and exports every function include/rope.h
  declares;
* argument validation: every error row of [IPRM §返回值与错误码] and the checks of
  [RSCC §入参校验逻辑] are forced from the host; the library and the oracle (two separate
  implementations of the documented rules) must return the same status, which is also the
  one the pages prescribe;
* calls that validate but do no work (empty slice, empty x) return success without a launch;
* without a GPU, a call that reaches the launch reports ROPE_ERR_RUNTIME with a message.

Pages:
  [IPRM] "CANN ops-transformer 的 aclnnInplacePartialRotaryMul 算子：Inplace 部分旋转位置编码接口详解与实现剖析"
  [RSCC] "CANN ops-transformer 旋转位置编码算子 RopeWithSinCosCache 深度解析：cache 化 RoPE 的计算原理与 aclnn 两段式调用实战"
"""
import ctypes
import os
import re

import pytest
import torch

import oracle
import rope_partial_inplace_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NULLPTR, INVALID = 161001, 161002


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(rope_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"rope_partial_inplace", "rope_with_cos_sin_cache", "rope_last_error"} <= set(names)
    lib = ctypes.CDLL(ra.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


# ------------------------------------------------------------------------------------------
# Host descriptors for both implementations, built from the same CPU tensors.  Validation
# failures return before any HIP call, so CPU pointers are never dereferenced by a kernel.
# ------------------------------------------------------------------------------------------

def lib_desc(spec):
    if spec is None:
        return None
    d = ra.RopeTensor()
    d.data, d.dtype, d.ndim = spec["data"], spec["dtype"], spec["ndim"]
    for i in range(min(spec["ndim"], 4, len(spec["shape"]))):
        d.shape[i], d.stride[i] = spec["shape"][i], spec["stride"][i]
    return ctypes.byref(d)


def oro_desc(spec):
    if spec is None:
        return None
    d = oracle.OroTensor()
    d.data, d.dtype, d.ndim = spec["data"], spec["dtype"], spec["ndim"]
    for i in range(min(spec["ndim"], 4, len(spec["shape"]))):
        d.shape[i], d.stride[i] = spec["shape"][i], spec["stride"][i]
    return ctypes.byref(d)


_KEEP = []


def spec_of(t, **override):
    _KEEP.append(t)
    s = {"data": t.data_ptr() if t.numel() else None,
         "dtype": {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2,
                   torch.int64: 3}.get(t.dtype, 7),
         "ndim": t.dim(), "shape": list(t.shape), "stride": list(t.stride())}
    s.update(override)
    return s


def ints(v):
    if v is None:
        return None, 0
    return (ctypes.c_int64 * max(len(v), 1))(*v), len(v)


def call_inplace(x, c, s, mode, sl, sl_len=None, backward=False):
    arr, n = ints(sl)
    if sl_len is not None:
        n = sl_len
    lib_fn = ra.LIB.rope_partial_inplace_backward if backward else ra.LIB.rope_partial_inplace
    ora_fn = (oracle._lib.oro_rope_partial_inplace_backward if backward
              else oracle._lib.oro_rope_partial_inplace)
    lib_st = lib_fn(lib_desc(x), lib_desc(c), lib_desc(s), mode, arr, n, None)
    ora_st = ora_fn(oro_desc(x), oro_desc(c), oro_desc(s), mode, arr, n, None)
    return lib_st, ora_st


def inplace_base(B=2, S=3, N=2, D=16, L=8, xdt=torch.bfloat16, cdt=torch.float32):
    x = torch.zeros(B, S, N, D, dtype=xdt)
    c = torch.zeros(B, S, 1, L, dtype=cdt)
    return spec_of(x), spec_of(c), spec_of(c.clone())


INPLACE_CASES = [
    # (name, builder -> (x, cos, sin, mode, slice, slice_len override), expected status)
    ("x null", lambda b: (None, b[1], b[2], 1, [0, 8]), NULLPTR),
    ("cos null", lambda b: (b[0], None, b[2], 1, [0, 8]), NULLPTR),
    ("sin null", lambda b: (b[0], b[1], None, 1, [0, 8]), NULLPTR),
    ("x data null", lambda b: (dict(b[0], data=None), b[1], b[2], 1, [0, 8]), NULLPTR),
    ("slice pointer null", lambda b: (b[0], b[1], b[2], 1, None, 2), NULLPTR),
    ("x int64", lambda b: (dict(b[0], dtype=3), b[1], b[2], 1, [0, 8]), INVALID),
    ("x unknown dtype", lambda b: (dict(b[0], dtype=9), b[1], b[2], 1, [0, 8]), INVALID),
    ("cos f16 with bf16 x", lambda b: (b[0], dict(b[1], dtype=1), dict(b[2], dtype=1), 1,
                                       [0, 8]), INVALID),
    ("cos/sin dtypes differ", lambda b: (b[0], b[1], dict(b[2], dtype=2), 1, [0, 8]), INVALID),
    ("mode 2", lambda b: (b[0], b[1], b[2], 2, [0, 8]), INVALID),
    ("mode -1", lambda b: (b[0], b[1], b[2], -1, [0, 8]), INVALID),
    ("mode 3", lambda b: (b[0], b[1], b[2], 3, [0, 8]), INVALID),
    ("x 3-D", lambda b: (dict(b[0], ndim=3), b[1], b[2], 1, [0, 8]), INVALID),
    ("cos 3-D", lambda b: (b[0], dict(b[1], ndim=3), dict(b[2], ndim=3), 1, [0, 8]), INVALID),
    ("rank 5", lambda b: (dict(b[0], ndim=5), b[1], b[2], 1, [0, 8]), INVALID),
    ("cos/sin shapes differ", lambda b: (b[0], b[1], dict(b[2], shape=[2, 1, 1, 8]), 1, [0, 8]),
     INVALID),
    ("D > 1024", lambda b: (dict(b[0], shape=[2, 3, 2, 1026],
                                 stride=[6 * 1026, 2 * 1026, 1026, 1]), b[1], b[2], 1, [0, 8]),
     INVALID),
    ("D odd", lambda b: (dict(b[0], shape=[2, 3, 2, 15], stride=[90, 30, 15, 1]), b[1], b[2], 1,
                         [0, 8]), INVALID),
    ("slice of 1 value", lambda b: (b[0], b[1], b[2], 1, [0]), INVALID),
    ("slice of 3 values", lambda b: (b[0], b[1], b[2], 1, [0, 8, 9]), INVALID),
    ("slice start < 0", lambda b: (b[0], b[1], b[2], 1, [-2, 6]), INVALID),
    ("slice end < start", lambda b: (b[0], b[1], b[2], 1, [8, 0]), INVALID),
    ("slice end > D", lambda b: (b[0], b[1], b[2], 1, [10, 18]), INVALID),
    ("slice odd length", lambda b: (b[0], b[1], b[2], 1, [0, 7]), INVALID),
    ("x non-contiguous", lambda b: (dict(b[0], stride=[96, 32, 16, 2]), b[1], b[2], 1, [0, 8]),
     INVALID),
    ("cos non-contiguous", lambda b: (b[0], dict(b[1], stride=[48, 16, 8, 2]), b[2], 1, [0, 8]),
     INVALID),
    ("cos last dim != slice", lambda b: (b[0], b[1], b[2], 1, [0, 10]), INVALID),
    ("cos B neither 1 nor B", lambda b: (b[0], dict(b[1], shape=[3, 3, 1, 8]),
                                         dict(b[2], shape=[3, 3, 1, 8]), 1, [0, 8]), INVALID),
    ("negative dim", lambda b: (dict(b[0], shape=[-2, 3, 2, 16]), b[1], b[2], 1, [0, 8]),
     INVALID),
    ("negative slice length", lambda b: (b[0], b[1], b[2], 1, [0, 8], -1), INVALID),
    # x is written in place: it may share no memory with cos or sin (reading R22)
    ("cos inside x", lambda b: (b[0], dict(b[1], data=b[0]["data"]), b[2], 1, [0, 8]),
     INVALID),
    ("sin overlaps the end of x", lambda b: (b[0], b[1], dict(b[2], data=b[0]["data"] + 320), 1,
                                             [0, 8]), INVALID),
    # descriptors no buffer can have: refused before any size arithmetic could overflow
    ("x beyond 2^53 elements", lambda b: (dict(b[0], shape=[1 << 20, 1 << 20, 1 << 14, 16],
                                               stride=[1 << 38, 1 << 18, 16, 1]), b[1], b[2], 1,
                                          [0, 8]), INVALID),
    ("x element count overflows int64", lambda b: (
        dict(b[0], shape=[1 << 21, 1 << 21, 1 << 21, 16], stride=[1 << 46, 1 << 25, 16, 1]),
        b[1], b[2], 1, [0, 8]), INVALID),
    ("cos reaches 2^60 elements", lambda b: (b[0], dict(b[1], stride=[1 << 60, 8, 8, 1]), b[2],
                                             1, [0, 8]), INVALID),
    ("x data null, overflowing shape", lambda b: (
        dict(b[0], data=None, shape=[1 << 40, 1 << 40, 1, 16]), b[1], b[2], 1, [0, 8]), NULLPTR),
    # accepted, nothing launched
    ("empty slice", lambda b: (b[0], b[1], b[2], 1, [4, 4]), 0),
    ("empty slice ignores cos last dim", lambda b: (b[0], b[1], b[2], 1, [6, 6]), 0),
    ("empty x", lambda b: (dict(b[0], shape=[0, 3, 2, 16]), dict(b[1], shape=[1, 3, 1, 8]),
                           dict(b[2], shape=[1, 3, 1, 8]), 1, [0, 8]), 0),
    # an empty view keeps the strides torch gives it ([2,0,2,16]: 0 rows in the middle)
    ("empty x, zero middle dim", lambda b: (dict(b[0], shape=[2, 0, 2, 16], stride=[32, 32, 16, 1]),
                                            dict(b[1], shape=[1, 1, 1, 8]),
                                            dict(b[2], shape=[1, 1, 1, 8]), 1, [0, 8]), 0),
]


@pytest.mark.parametrize("mode", [1, 0], ids=["interleave", "half"])
@pytest.mark.parametrize("backward", [False, True], ids=["forward", "backward"])
@pytest.mark.parametrize("name,build,expected", INPLACE_CASES, ids=[c[0] for c in INPLACE_CASES])
def test_inplace_validation(name, build, expected, backward, mode):
    """Every case in interleave mode and again in half mode (cases written with mode 1 take
    the parametrized mode; the others keep their own)."""
    args = list(build(inplace_base()))
    if args[3] == 1:
        args[3] = mode
    lib_st, ora_st = call_inplace(*args, backward=backward)
    assert lib_st == expected, ra.last_error()
    assert ora_st == expected, oracle.last_error()


def cache_base(T=4, nq=2, nk=1, H=64, rd=32, dt=torch.bfloat16, m=0):
    q = torch.zeros(T, nq * H, dtype=dt)
    k = torch.zeros(T, nk * H, dtype=dt)
    cache = torch.zeros(10, rd, dtype=dt)
    pos = torch.zeros((m, T) if m else (T,), dtype=torch.int64)
    return {"pos": spec_of(pos), "q": spec_of(q), "k": spec_of(k), "cache": spec_of(cache),
            "qo": spec_of(torch.zeros_like(q)), "ko": spec_of(torch.zeros_like(k)),
            "msec": None, "H": H, "neox": 1}


def call_cache(a, msec_len=None, cache_mode=None):
    """Statuses of the library and of the oracle on the same arguments: the V1 entry points,
    or the V2 ones when cache_mode is given."""
    arr, n = ints(a["msec"])
    if msec_len is not None:
        n = msec_len
    order = ["pos", "q", "k", "cache"]
    lib_in = [lib_desc(a[k]) for k in order] + [arr, n, a["H"], a["neox"]]
    lib_out = [lib_desc(a["qo"]), lib_desc(a["ko"]), None]
    ora_in = [oro_desc(a[k]) for k in order] + [arr, n, a["H"], a["neox"]]
    ora_out = [oro_desc(a["qo"]), oro_desc(a["ko"]), None, None]
    if cache_mode is None:
        lib_st = ra.LIB.rope_with_cos_sin_cache(*lib_in, *lib_out)
        ora_st = oracle._lib.oro_rope_with_cos_sin_cache(*ora_in, *ora_out)
    else:
        lib_st = ra.LIB.rope_with_cos_sin_cache_v2(*lib_in, cache_mode, *lib_out)
        ora_st = oracle._lib.oro_rope_with_cos_sin_cache_v2(*ora_in, cache_mode, *ora_out)
    return lib_st, ora_st


def upd(a, **kw):
    b = dict(a)
    b.update(kw)
    return b


CACHE_CASES = [
    ("positions null", lambda a: upd(a, pos=None), NULLPTR),
    ("queryIn null", lambda a: upd(a, q=None), NULLPTR),
    ("keyIn null", lambda a: upd(a, k=None), NULLPTR),
    ("cache null", lambda a: upd(a, cache=None), NULLPTR),
    ("queryOut null", lambda a: upd(a, qo=None), NULLPTR),
    ("keyOut null", lambda a: upd(a, ko=None), NULLPTR),
    ("query data null", lambda a: upd(a, q=dict(a["q"], data=None)), NULLPTR),
    ("positions not int64", lambda a: upd(a, pos=dict(a["pos"], dtype=0)), INVALID),
    ("query int64", lambda a: upd(a, q=dict(a["q"], dtype=3)), INVALID),
    ("key dtype differs", lambda a: upd(a, k=dict(a["k"], dtype=1)), INVALID),
    ("cache dtype differs", lambda a: upd(a, cache=dict(a["cache"], dtype=0)), INVALID),
    ("output dtype differs", lambda a: upd(a, qo=dict(a["qo"], dtype=1)), INVALID),
    ("query 3-D", lambda a: upd(a, q=dict(a["q"], ndim=3, shape=[4, 2, 64],
                                          stride=[128, 64, 1])), INVALID),
    ("cache 1-D", lambda a: upd(a, cache=dict(a["cache"], ndim=1, shape=[320], stride=[1])),
     INVALID),
    ("query empty", lambda a: upd(a, q=dict(a["q"], shape=[0, 128]), qo=dict(a["qo"], shape=[0, 128]),
                                  k=dict(a["k"], shape=[0, 64]), ko=dict(a["ko"], shape=[0, 64]),
                                  pos=dict(a["pos"], shape=[0])), INVALID),
    ("cache empty", lambda a: upd(a, cache=dict(a["cache"], shape=[0, 32])), INVALID),
    ("token counts differ", lambda a: upd(a, k=dict(a["k"], shape=[3, 64]),
                                          ko=dict(a["ko"], shape=[3, 64])), INVALID),
    ("output shape differs", lambda a: upd(a, qo=dict(a["qo"], shape=[4, 64], stride=[64, 1])),
     INVALID),
    ("mrope 2 entries", lambda a: upd(a, msec=[8, 8]), INVALID),
    ("mrope 5 entries", lambda a: upd(a, msec=[4, 4, 4, 2, 2]), INVALID),
    ("mrope negative", lambda a: upd(a, msec=[16, -8, 8]), INVALID),
    ("mrope 2*sum != rd", lambda a: upd(a, msec=[16, 24, 24]), INVALID),
    ("mrope not listed", lambda a: upd(a, msec=[8, 4, 4]), INVALID),
    ("mrope null with length", lambda a: (upd(a, msec=None), 3), NULLPTR),
    ("mrope negative length", lambda a: (a, -1), INVALID),
    ("mrope [0,..] is rope: 2-D positions refused", lambda a: upd(
        a, msec=[0, 8, 8], pos=spec_of(torch.zeros(3, 4, dtype=torch.int64))), INVALID),
    ("headSize 0", lambda a: upd(a, H=0), INVALID),
    ("headSize negative", lambda a: upd(a, H=-64), INVALID),
    ("headSize not 64B multiple", lambda a: upd(a, H=48), INVALID),
    ("query width not multiple of headSize", lambda a: upd(a, H=96), INVALID),
    ("rotaryDim > headSize", lambda a: upd(a, H=32, cache=spec_of(torch.zeros(10, 64,
                                                                        dtype=torch.bfloat16))),
     INVALID),
    ("rotaryDim not 64B multiple", lambda a: upd(a, cache=spec_of(torch.zeros(10, 48,
                                                                        dtype=torch.bfloat16))),
     INVALID),
    ("rope positions 2-D", lambda a: upd(a, pos=spec_of(torch.zeros(1, 4, dtype=torch.int64))),
     INVALID),
    ("rope positions wrong length", lambda a: upd(a, pos=spec_of(torch.zeros(5,
                                                                           dtype=torch.int64))),
     INVALID),
    ("query inner stride 2", lambda a: upd(a, q=dict(a["q"], stride=[256, 2])), INVALID),
    ("query negative row stride", lambda a: upd(a, q=dict(a["q"], stride=[-128, 1])), INVALID),
    ("negative positions stride", lambda a: upd(a, pos=dict(a["pos"], stride=[-1])), INVALID),
    ("queryOut non-contiguous", lambda a: upd(a, qo=dict(a["qo"], stride=[256, 1])), INVALID),
    ("queryOut overlaps keyOut", lambda a: upd(a, ko=dict(a["ko"], data=a["qo"]["data"])),
     INVALID),
    ("queryOut overlaps cache", lambda a: upd(a, qo=dict(a["qo"], data=a["cache"]["data"])),
     INVALID),
    ("keyOut overlaps queryIn", lambda a: upd(a, ko=dict(a["ko"], data=a["q"]["data"])),
     INVALID),
    # descriptors no buffer can have, and mrope entries that would overflow a sum
    ("query row stride 2^60", lambda a: upd(a, q=dict(a["q"], stride=[1 << 60, 1])), INVALID),
    ("key element count overflows int64", lambda a: upd(
        a, k=dict(a["k"], shape=[1 << 62, 1 << 62]), ko=dict(a["ko"], shape=[1 << 62, 1 << 62])),
     INVALID),
    ("positions beyond 2^53 elements", lambda a: upd(a, pos=dict(a["pos"], shape=[1 << 60])),
     INVALID),
    ("mrope entries of 2^62", lambda a: upd(a, msec=[1 << 62, 1 << 62, 1 << 62]), INVALID),
]


@pytest.mark.parametrize("cache_mode", [None, 0, 1], ids=["v1", "v2_mode0", "v2_mode1"])
@pytest.mark.parametrize("name,build,expected", CACHE_CASES, ids=[c[0] for c in CACHE_CASES])
def test_cache_validation(name, build, expected, cache_mode):
    built = build(cache_base())
    if isinstance(built, tuple):
        lib_st, ora_st = call_cache(built[0], msec_len=built[1], cache_mode=cache_mode)
    else:
        lib_st, ora_st = call_cache(built, cache_mode=cache_mode)
    assert lib_st == expected, ra.last_error()
    assert ora_st == expected, oracle.last_error()
    assert ra.last_error() != ""


def mrope_base(msec, rd):
    a = cache_base(H=rd, rd=rd, m=len(msec))
    return upd(a, msec=msec)


# cacheMode rules of [RSCC §V2 接口：cacheMode 扩展]: 0 or 1 only, and 0 only with the
# 4-section list; the check applies in rope mode too.
V2_REFUSED = [
    ("rope mode, cacheMode 2", lambda: cache_base(), 2),
    ("rope mode, cacheMode -1", lambda: cache_base(), -1),
    ("mrope [16,24,24], cacheMode 2", lambda: mrope_base([16, 24, 24], 128), 2),
    ("mrope [16,16,16,16], cacheMode 1", lambda: mrope_base([16, 16, 16, 16], 128), 1),
    ("mrope [11,11,10], cacheMode 3", lambda: mrope_base([11, 11, 10], 64), 3),
]


@pytest.mark.parametrize("name,build,mode", V2_REFUSED, ids=[c[0] for c in V2_REFUSED])
def test_cache_mode_refused(name, build, mode):
    assert call_cache(build(), cache_mode=mode) == (INVALID, INVALID), ra.last_error()
    assert ra.last_error() != ""


V2_ACCEPTED = [
    ("rope mode, cacheMode 1", lambda: cache_base(), 1),
    ("mrope [16,16,16,16], cacheMode 0", lambda: mrope_base([16, 16, 16, 16], 128), 0),
    ("mrope [16,24,24], cacheMode 1", lambda: mrope_base([16, 24, 24], 128), 1),
    ("mrope [8,12,12], cacheMode 1", lambda: mrope_base([8, 12, 12], 64), 1),
    ("mrope [24,20,20], cacheMode 1", lambda: mrope_base([24, 20, 20], 128), 1),
    ("mrope [11,11,10], cacheMode 1", lambda: mrope_base([11, 11, 10], 64), 1),
]


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU error path")
@pytest.mark.parametrize("name,build,mode", V2_ACCEPTED, ids=[c[0] for c in V2_ACCEPTED])
def test_cache_mode_accepted(name, build, mode):
    """Accepted by both: the oracle computes, the library gets past validation to the launch
    (which fails without a GPU, so no host pointer reaches a kernel)."""
    lib_st, ora_st = call_cache(build(), cache_mode=mode)
    assert ora_st == 0, oracle.last_error()
    assert lib_st == ra.ROPE_ERR_RUNTIME and "launch" in ra.last_error()


def test_mrope_bad_positions_shape():
    a = cache_base()
    a = upd(a, msec=[8, 4, 4], cache=spec_of(torch.zeros(10, 32, dtype=torch.bfloat16)))
    # [8,4,4] is not a listed section: refused before positions are looked at
    assert call_cache(a) == (INVALID, INVALID)
    b = cache_base(H=128, rd=128)
    b = upd(b, msec=[16, 24, 24], pos=spec_of(torch.zeros(2, 4, dtype=torch.int64)))
    assert call_cache(b) == (INVALID, INVALID)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU error path")
def test_runtime_error_without_gpu():
    """A valid call reaches the kernel launch; with no GPU the launch fails and the library
    reports ROPE_ERR_RUNTIME with a message (nothing was dereferenced on the host)."""
    x, c, s = inplace_base()
    st = ra.LIB.rope_partial_inplace(lib_desc(x), lib_desc(c), lib_desc(s), 1,
                                     *ints([0, 8]), None)
    assert st == ra.ROPE_ERR_RUNTIME
    assert "launch" in ra.last_error()


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU error path")
@pytest.mark.parametrize("backward", [False, True], ids=["forward", "backward"])
def test_half_mode_accepted(backward):
    """rotary_mode 0 passes validation in both implementations: the oracle computes, the
    library reaches the launch (which fails without a GPU)."""
    lib_st, ora_st = call_inplace(*inplace_base(), 0, [0, 8], backward=backward)
    assert ora_st == 0, oracle.last_error()
    assert lib_st == ra.ROPE_ERR_RUNTIME and "launch" in ra.last_error()


def test_binding_refuses_host_tensors():
    x = torch.zeros(1, 2, 1, 8)
    with pytest.raises(ra.RopeError):
        ra.rope_partial_inplace(x, torch.zeros(1, 2, 1, 8), torch.zeros(1, 2, 1, 8))


def test_library_carries_gfx950_code_only():
    from rope_partial_inplace_amd import build
    targets = build.bundled_targets(ra.LIB_PATH)
    assert [t for t in targets if not t.startswith("host-")] == ["hipv4-amdgcn-amd-amdhsa--gfx950"]


def test_pages_python_interface_rotary_mode_names():
    """inplace_partial_rotary_mul takes rotary_mode by name as on [IPRM §Python 接口与自动微分]
    ("interleave"; "half" for mode 0) or by number; other names are refused before any call,
    other numbers go to the library, which refuses them."""
    assert ra._rotary_mode_code("interleave") == 1
    assert ra._rotary_mode_code("half") == 0
    assert ra._rotary_mode_code(1) == 1 and ra._rotary_mode_code(0) == 0
    with pytest.raises(ra.RopeError) as e:
        ra._rotary_mode_code("quarter")
    assert e.value.code == ra.ROPE_ERR_PARAM_INVALID
    x = torch.zeros(1, 2, 1, 8)
    with pytest.raises(ra.RopeError) as e:   # host tensors are refused before the library
        ra.inplace_partial_rotary_mul(x, x[..., :8], x[..., :8], partial_slice=[0, 8])
    assert e.value.code == ra.ROPE_ERR_PARAM_INVALID


def test_error_messages_are_per_thread():
    """rope_last_error() reports the failure of the calling thread's own last call: threads
    validating different bad calls at once (ctypes releases the GIL, so they run in parallel)
    each read back exactly the status and message that call gives when made alone."""
    from concurrent.futures import ThreadPoolExecutor

    picks = [c for c in INPLACE_CASES if c[2] != 0][::3]
    calls = []
    for name, build, _ in picks:
        a = build(inplace_base())
        arr, n = ints(a[4])
        n = a[5] if len(a) > 5 else n
        args = (lib_desc(a[0]), lib_desc(a[1]), lib_desc(a[2]), a[3], arr, n, None)
        calls.append(args)
    expected = []
    for args in calls:
        st = ra.LIB.rope_partial_inplace(*args)
        expected.append((st, ra.last_error()))
    assert len({m for _, m in expected}) > 5  # distinct messages, so a mix-up would show

    def worker(i):
        for _ in range(300):
            st = ra.LIB.rope_partial_inplace(*calls[i])
            if (st, ra.last_error()) != expected[i]:
                return False
        return True

    with ThreadPoolExecutor(max_workers=len(calls)) as ex:
        assert all(ex.map(worker, range(len(calls))))
