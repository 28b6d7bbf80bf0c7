"""Differential fuzz of argument validation (CPU, no kernel runs): seeded random descriptors,
mostly near the valid region and often just outside it, go to the library and to the oracle,
two separate implementations of the documented rules ([IPRM §返回值与错误码], [IPRM §约束说明],
[RSCC §入参校验逻辑], [RSCC §约束说明] and the readings listed with the oracle).  Both must
return the same status.  Without a GPU a call the library accepts stops at the launch
(ROPE_ERR_RUNTIME), so "accepted" means the library reports that and the oracle returns 0.

Every tensor points into its own zeroed host buffer, large enough for any descriptor the rules
accept, so the oracle's computation of an accepted call stays inside memory it owns.

Pages:
  [IPRM] "CANN ops-transformer 的 aclnnInplacePartialRotaryMul 算子：Inplace 部分旋转位置编码接口详解与实现剖析"
  [RSCC] "CANN ops-transformer 旋转位置编码算子 RopeWithSinCosCache 深度解析：cache 化 RoPE 的计算原理与 aclnn 两段式调用实战"
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import rope_partial_inplace_amd as ra
from test_boundary_cpu import ints, lib_desc, oro_desc

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="accepted calls must stop at the launch (no GPU)")

RUNTIME = ra.ROPE_ERR_RUNTIME
BUF_BYTES = 1 << 22
_BUFFERS = [torch.zeros(BUF_BYTES, dtype=torch.uint8) for _ in range(8)]


def agree(lib_st, ora_st):
    return lib_st == ora_st or (lib_st == RUNTIME and ora_st == 0)


def contiguous_strides(shape):
    st, acc = [], 1
    for d in reversed(shape):
        st.append(acc)
        acc *= max(d, 1)
    return list(reversed(st))


def spec(rng, buf, dtype, shape, perturb=0.08, null=0.02):
    """A descriptor of `shape` in buffer `buf`: usually contiguous, sometimes with one stride
    changed, sometimes with NULL data."""
    shape = list(shape)
    strides = contiguous_strides(shape)
    if shape and rng.random() < perturb:
        d = int(rng.integers(len(shape)))
        strides[d] = strides[d] * 2 if rng.random() < 0.5 else strides[d] + 1
    data = None if rng.random() < null else _BUFFERS[buf].data_ptr()
    # descriptors hold 4 dims; a 5-D view keeps its first 4 and is refused for its rank
    return {"data": data, "dtype": dtype, "ndim": len(shape), "shape": (shape + [0] * 4)[:4],
            "stride": (strides + [0] * 4)[:4]}


def pick(rng, choices):
    return choices[int(rng.integers(len(choices)))]


def inplace_case(rng):
    xdt = pick(rng, [0, 1, 2, 0, 1, 2, 3, 9])
    cdt = pick(rng, [xdt, xdt, 0, 0, 1, 2])
    B, S, N = (pick(rng, [1, 2, 3, 1, 2, 3, 0]) for _ in range(3))
    D = pick(rng, [2, 4, 8, 16, 64, 96, 1024, 0, 7, 1026])
    if rng.random() < 0.25:
        sl, sl_len = None, 0
    else:
        start = int(rng.integers(-1, D + 2))
        end = int(rng.integers(start - 1, D + 3))
        sl, sl_len = [start, end], 2
    if rng.random() < 0.05:
        sl_len = pick(rng, [1, 3, -1])
    if rng.random() < 0.03:
        sl, sl_len = None, 2
    lo, hi = (0, D) if sl is None else (sl[0], sl[1])
    L = hi - lo if rng.random() > 0.08 else hi - lo + 2
    cb = [pick(rng, [1, dim, dim, 2]) for dim in (B, S, N)]
    xndim = pick(rng, [4] * 12 + [3, 5])
    cndim = pick(rng, [4] * 12 + [3])
    xshape = [B, S, N, D][:xndim] if xndim <= 4 else [B, S, N, D, 1]
    cshape = (cb + [max(L, 0)])[:cndim]
    x = spec(rng, 0, xdt, xshape)
    c = spec(rng, 1, cdt, cshape)
    s = spec(rng, 2, cdt, cshape)
    if rng.random() < 0.05:
        s = dict(c)                              # one tensor for cos and sin: allowed
    if rng.random() < 0.04 and x["data"] is not None:
        c = dict(c, data=x["data"])              # cos inside x: refused (R22)
    mode = pick(rng, [1, 0, 1, 0, 2, -1])
    return x, c, s, mode, sl, sl_len


def cache_case(rng):
    dt = pick(rng, [0, 1, 2, 0, 1, 2, 3])
    es = {0: 4, 1: 2, 2: 2}.get(dt, 8)
    align = 64 // es
    T = pick(rng, [1, 2, 5, 1, 2, 5, 0])
    nq, nk = pick(rng, [1, 2, 3]), pick(rng, [1, 2, 3])
    msec = pick(rng, [None, None, None, [16, 24, 24], [8, 12, 12], [24, 20, 20], [11, 11, 10],
                      [16, 16, 16, 16], [0, 8, 8], [8, 4, 4], [4, 4, 4, 2, 2], [16, -8, 8]])
    if msec is not None and msec[0] > 0 and rng.random() < 0.85:
        rd = 2 * sum(msec)
    elif rng.random() < 0.12:
        # long rotaryDim: either side of 16384, where the library stops staging a token's
        # cos|sin row in LDS and reads the cache row directly (the pages set no upper bound)
        rd = pick(rng, [8192, 16384 - align, 16384, 16384 + align, 20480, 24576])
    else:
        rd = align * int(rng.integers(1, 5)) if rng.random() > 0.1 else pick(rng, [0, 48, align + 2])
    H = rd + align * int(rng.integers(0, 3)) if rng.random() > 0.1 else pick(rng, [0, -64, 48, rd - align])
    Hs = max(H, 1)
    m = len(msec) if msec else 0
    pshape = [m, T] if (m and msec[0] > 0) else [T]
    if rng.random() < 0.06:
        pshape = pick(rng, [[T + 1], [2, T], [3, T + 1]])
    pos = spec(rng, 3, pick(rng, [3] * 10 + [0]), pshape)
    q = spec(rng, 4, dt, [T, nq * Hs])
    if rng.random() < 0.15:
        q["stride"][0] = nq * Hs + align          # padded rows: allowed
    k = spec(rng, 5, pick(rng, [dt] * 12 + [0, 1]), [T, nk * Hs])
    cache = spec(rng, 6, dt, [pick(rng, [16, 16, 16, 0]), max(rd, 0)])
    qo = spec(rng, 7, dt, [T, nq * Hs])
    ko_buf = 7 if rng.random() < 0.04 else 0      # keyOut in queryOut's buffer: overlap
    ko = spec(rng, ko_buf, dt, [T, nk * Hs])
    if ko_buf == 0 and ko["data"] is not None:
        ko["data"] += BUF_BYTES // 2               # clear of anything else in buffer 0
    if rng.random() < 0.04:
        qo = dict(q)                               # queryOut aliasing queryIn exactly: allowed
    r = rng.random()
    if r < 0.03:
        k["stride"][1] = 2                         # inner stride 2: refused
    elif r < 0.06:
        k["stride"][0] = -k["stride"][0]           # negative row stride: refused
    elif r < 0.09:
        pos["stride"][0] = -1                      # negative positions stride: refused
    elif r < 0.12:
        qo["stride"][0] = qo["stride"][0] + align  # padded output rows: refused
    elif r < 0.2:
        cache["stride"][0] = cache["stride"][0] + align  # padded cache rows: allowed
    cache_mode = pick(rng, [None, None, 0, 1, 2])
    return dict(pos=pos, q=q, k=k, cache=cache, qo=qo, ko=ko, msec=msec, H=H,
                neox=int(rng.integers(0, 2)), cache_mode=cache_mode)


@pytest.mark.parametrize("block", range(8))
def test_inplace_validation_agrees(block):
    rng = np.random.default_rng(5000 + block)
    counts = {}
    for i in range(400):
        x, c, s, mode, sl, sl_len = inplace_case(rng)
        arr, _ = ints(sl)
        for backward in (False, True):
            lib_fn = ra.LIB.rope_partial_inplace_backward if backward else ra.LIB.rope_partial_inplace
            ora_fn = (oracle._lib.oro_rope_partial_inplace_backward if backward
                      else oracle._lib.oro_rope_partial_inplace)
            lib_st = lib_fn(lib_desc(x), lib_desc(c), lib_desc(s), mode, arr, sl_len, None)
            ora_st = ora_fn(oro_desc(x), oro_desc(c), oro_desc(s), mode, arr, sl_len, None)
            assert agree(lib_st, ora_st), (
                f"case {block}/{i}: library {lib_st} ({ra.last_error()}), oracle {ora_st} "
                f"({oracle.last_error()}): x {x} cos {c} sin {s} mode {mode} slice {sl} "
                f"len {sl_len} backward {backward}")
            counts[lib_st] = counts.get(lib_st, 0) + 1
    # the generator reaches every outcome
    assert {0, RUNTIME, 161001, 161002} <= set(counts), counts


@pytest.mark.parametrize("block", range(8))
def test_cache_validation_agrees(block):
    rng = np.random.default_rng(6000 + block)
    counts = {}
    for i in range(600):
        a = cache_case(rng)
        arr, n = ints(a["msec"])
        if a["msec"] is not None and rng.random() < 0.03:
            arr, n = None, 3
        order = ["pos", "q", "k", "cache"]
        lib_in = [lib_desc(a[key]) for key in order] + [arr, n, a["H"], a["neox"]]
        ora_in = [oro_desc(a[key]) for key in order] + [arr, n, a["H"], a["neox"]]
        lib_out = [lib_desc(a["qo"]), lib_desc(a["ko"]), None]
        ora_out = [oro_desc(a["qo"]), oro_desc(a["ko"]), None, None]
        if a["cache_mode"] is None:
            lib_st = ra.LIB.rope_with_cos_sin_cache(*lib_in, *lib_out)
            ora_st = oracle._lib.oro_rope_with_cos_sin_cache(*ora_in, *ora_out)
        else:
            lib_st = ra.LIB.rope_with_cos_sin_cache_v2(*lib_in, a["cache_mode"], *lib_out)
            ora_st = oracle._lib.oro_rope_with_cos_sin_cache_v2(*ora_in, a["cache_mode"],
                                                                 *ora_out)
        assert agree(lib_st, ora_st), (
            f"case {block}/{i}: library {lib_st} ({ra.last_error()}), oracle {ora_st} "
            f"({oracle.last_error()}): {a}")
        counts[lib_st] = counts.get(lib_st, 0) + 1
    assert {RUNTIME, 161001, 161002} <= set(counts), counts
