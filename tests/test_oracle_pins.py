"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks the oracle against what the pages and the mathematics fix: hand-expanded
worked cases (tests/golden), closed forms (RoPE is a rotation: complex multiplication by
e^{i*theta}), invariants (norm per pair, relative-position property), special cases with
exact answers, library routines (PyTorch / NumPy dtype conversion, NumPy complex and matmul)
and an error bound against the oracle's float64 twin.  The mistakes these are meant to catch:
a dropped term, a flipped sign, a cos/sin swap, an index shifted within a pair, pairs counted
from 0 instead of the slice start, NeoX/GPT-J mixed up, an mrope section boundary off by one,
a wrong broadcast index, a rounding-mode or NaN slip.

Pages:
  [IPRM] "CANN ops-transformer 的 aclnnInplacePartialRotaryMul 算子：Inplace 部分旋转位置编码接口详解与实现剖析"
  [RSCC] "CANN ops-transformer 旋转位置编码算子 RopeWithSinCosCache 深度解析：cache 化 RoPE 的计算原理与 aclnn 两段式调用实战"
"""
import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import rope_workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f64(t):
    return t.to(torch.float64).numpy()


def raw_bits(t):
    if t.dtype == torch.float32:
        return t.contiguous().view(torch.int32).numpy().view(np.uint32)
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def run_inplace(x, cos, sin, sl, twin=False, mode=1):
    x = x.clone()
    st, x64 = oracle.rope_partial_inplace(x, cos, sin, mode, sl, twin=twin)
    assert st == oracle.OK, oracle.last_error()
    return x, x64


def run_cache(pos, q, k, cache, msec, H, neox, twin=False):
    qo = torch.empty_like(q, memory_format=torch.contiguous_format)
    ko = torch.empty_like(k, memory_format=torch.contiguous_format)
    st, q64, k64 = oracle.rope_with_cos_sin_cache(pos, q, k, cache, msec, H, neox, qo, ko,
                                                  twin=twin)
    assert st == oracle.OK, oracle.last_error()
    return qo, ko, q64, k64


# ------------------------------------------------------------------------------------------
# Rounding and decoding routines vs library conversions (PyTorch, NumPy)
# ------------------------------------------------------------------------------------------

def _chunk_check(lo, n, sign):
    u = (np.arange(lo, lo + n, dtype=np.uint64) | (np.uint64(0x80000000) if sign else 0))
    f = u.astype(np.uint32).view(np.float32)
    isnan = np.isnan(f)
    ft = torch.from_numpy(f)
    ob = oracle.round_bf16_bits(f)
    tb = ft.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    of = oracle.round_f16_bits(f)
    tf = ft.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    bad_b = (ob != tb) & ~isnan
    bad_f = (of != tf) & ~isnan
    # NaN in, NaN out (payloads may differ; bit patterns of the outputs are NaN encodings)
    nan_b = ((ob[isnan] & 0x7FFF) > 0x7F80).all()
    nan_f = ((of[isnan] & 0x7FFF) > 0x7C00).all()
    return int(bad_b.sum()), int(bad_f.sum()), bool(nan_b), bool(nan_f)


def test_rounding_exhaustive_positive_and_sampled_negative():
    """Every non-negative binary32 pattern (2^31 of them) is rounded to bfloat16 and binary16
    by the oracle and by PyTorch's CPU conversion (round-to-nearest-even); they must agree
    bit for bit (NaN compared as NaN).  Negative patterns are checked on one 16M chunk."""
    step = 1 << 24
    jobs = [(lo, step, False) for lo in range(0, 1 << 31, step)]
    jobs.append((0x3F000000, step, True))
    with ThreadPoolExecutor(max_workers=6) as ex:
        res = list(ex.map(lambda a: _chunk_check(*a), jobs))
    assert sum(r[0] for r in res) == 0, "bf16 rounding disagrees with torch"
    assert sum(r[1] for r in res) == 0, "f16 rounding disagrees with torch"
    assert all(r[2] and r[3] for r in res), "NaN not mapped to NaN"


def test_rounding_against_numpy_f16_sample():
    """A second library routine for binary16: NumPy's float32 -> float16 cast."""
    rng = np.random.default_rng(7)
    u = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    # add the ties of every exponent explicitly: mantissa ending in exactly half an ulp
    ties = (np.arange(256, dtype=np.uint32) << 23) | np.uint32(0x1000) | np.uint32(0x2000)
    f = np.concatenate([u, ties, ties ^ np.uint32(0x2000)]).view(np.float32)
    ok = ~np.isnan(f)
    with np.errstate(over="ignore"):
        np16 = f.astype(np.float16).view(np.uint16)
    assert (oracle.round_f16_bits(f)[ok] == np16[ok]).all()


def _ties(dropped_bits: int) -> np.ndarray:
    """binary32 patterns whose dropped low bits are exactly half a unit, with the kept part
    even and odd, for every exponent and both signs, plus their neighbours one ulp away."""
    e = np.arange(256, dtype=np.uint32) << 23
    half = np.uint32(1 << (dropped_bits - 1))
    kept_lsb = np.uint32(1 << dropped_bits)
    base = np.concatenate([e | half, e | half | kept_lsb, e | half | np.uint32(0x2AAAAA & ~((1 << dropped_bits) - 1))])
    base = np.concatenate([base, base + 1, base - 1])
    return np.concatenate([base, base | np.uint32(0x80000000)])


def test_rounding_ties_and_boundaries():
    """Round-half-to-even at every exponent: bfloat16 drops 16 bits; binary16 drops 13 bits
    for normal results and more in the subnormal range (every shift up to 24 is covered)."""
    with np.errstate(over="ignore"):
        f = _ties(16).view(np.float32)
        ok = ~np.isnan(f)
        tb = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert (oracle.round_bf16_bits(f)[ok] == tb[ok]).all()
        for k in range(13, 25):
            f = _ties(k).view(np.float32)
            ok = ~np.isnan(f)
            tf = torch.from_numpy(f).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
            assert (oracle.round_f16_bits(f)[ok] == tf[ok]).all(), k


def test_decoding_all_f16_and_bf16_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = oracle.f16_bits_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    same = (mine.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()
    # bfloat16: the decoded value must be exactly the upper half of a binary32
    for b in (0x0000, 0x0001, 0x3F80, 0x7F7F, 0x8000, 0xC0A0, 0x7F80, 0xFF80):
        v = np.float32(oracle.bf16_bits_to_f32(b))
        assert v.view(np.uint32) == np.uint32(b << 16)


# ------------------------------------------------------------------------------------------
# Hand-expanded worked cases (tests/golden)
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("fname", ["t1_interleave_pairs.json", "t2_slice_even_start.json",
                                   "t3_slice_odd_start.json"])
@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_golden_inplace(fname, dt):
    g = golden(fname)
    x = torch.tensor(g["x"], dtype=DT[dt]).reshape(g["x_shape"])
    L = len(g["cos"])
    cos = torch.tensor(g["cos"], dtype=DT[dt]).reshape(1, 1, 1, L)
    sin = torch.tensor(g["sin"], dtype=DT[dt]).reshape(1, 1, 1, L)
    y, _ = run_inplace(x, cos, sin, g["partial_slice"])
    assert f64(y).ravel().tolist() == g["expected"]
    if "expected_if_literal_concatenation" in g:
        assert f64(y).ravel().tolist() != g["expected_if_literal_concatenation"]


@pytest.mark.parametrize("neox", [True, False])
def test_golden_page_example(neox):
    """[RSCC §完整调用示例]: the page's own inputs, bf16, all ones, headSize 32."""
    g = golden("t4_page_example_bf16.json")
    pos = torch.tensor(g["positions"], dtype=torch.int64)
    q = torch.full(g["query_shape"], g["fill"], dtype=torch.bfloat16)
    k = torch.full(g["key_shape"], g["fill"], dtype=torch.bfloat16)
    cache = torch.full(g["cache_shape"], g["fill"], dtype=torch.bfloat16)
    qo, ko, _, _ = run_cache(pos, q, k, cache, None, g["head_size"], neox)
    head = g["expected_head_neox"] if neox else g["expected_head_gptj"]
    for out in (qo, ko):
        for row in f64(out).reshape(-1, g["head_size"]):
            assert row.tolist() == head


@pytest.mark.parametrize("neox", [True, False])
def test_golden_styles_small(neox):
    g = golden("t5_styles_small.json")
    H, rd = g["head_size"], g["rotary_dim"]
    head = torch.arange(H, dtype=torch.float32) + 10
    head[rd:] = 7
    key = "neox" if neox else "gptj"
    for p, v in zip(g[key + "_positions_in_head"], g[key + "_inputs"]):
        head[p] = v
    cos = torch.ones(rd // 2)
    sin = torch.zeros(rd // 2)
    cos[:2] = torch.tensor(g["cos_first"])
    sin[:2] = torch.tensor(g["sin_first"])
    cache = torch.cat([cos, sin]).reshape(1, rd).to(torch.bfloat16)
    q = head.reshape(1, H).to(torch.bfloat16)
    qo, ko, _, _ = run_cache(torch.zeros(1, dtype=torch.int64), q, q.clone(), cache, None, H,
                             neox)
    expect = head.clone()
    for p, v in zip(g[key + "_positions_in_head"], g[key + "_expected"]):
        expect[p] = v
    assert f64(qo).ravel().tolist() == expect.tolist()
    assert f64(ko).ravel().tolist() == expect.tolist()


def test_golden_mrope_stitch():
    g = golden("t6_mrope_stitch.json")
    rd, H = g["rotary_dim"], g["head_size"]
    cache = torch.zeros(4, rd)
    for p in range(4):
        cache[p, : rd // 2] = p
        cache[p, rd // 2:] = 10 * p
    cache = cache.to(torch.bfloat16)
    head = torch.zeros(H)
    head[: rd // 2] = 1.0
    q = head.reshape(1, H).to(torch.bfloat16)
    pos = torch.tensor(g["positions"], dtype=torch.int64)
    qo, _, _, _ = run_cache(pos, q, q.clone(), cache, g["mrope_section"], H, True)
    out = f64(qo).ravel()
    for rng_s, v in g["expected_cos"].items():
        a, b = map(int, rng_s.split(":"))
        assert (out[a:b] == v).all()
    for rng_s, v in g["expected_sin"].items():
        a, b = map(int, rng_s.split(":"))
        assert (out[rd // 2 + a: rd // 2 + b] == v).all()


# ------------------------------------------------------------------------------------------
# Closed forms: the rotation as complex multiplication / 2x2 matrices (NumPy, float64)
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("cos_layout", ["BSND", "BS1D", "B1ND", "B11D", "111D", "1S1D"])
def test_inplace_matches_2x2_matrices(cos_layout):
    """Per pair j = (2i, 2i+1) of the slice, [IPRM §计算原理与公式] is y = M x with
    M = [[cos[2i], -sin[2i]], [sin[2i+1], cos[2i+1]]] (reading R1, per-element cos/sin R5).
    NumPy's batched matmul in float64 with NumPy broadcasting of cos/sin is the pin."""
    B, S, N, D, sl = 2, 3, 4, 20, [6, 18]
    L = sl[1] - sl[0]
    shape = {"BSND": (B, S, N, L), "BS1D": (B, S, 1, L), "B1ND": (B, 1, N, L),
             "B11D": (B, 1, 1, L), "111D": (1, 1, 1, L), "1S1D": (1, S, 1, L)}[cos_layout]
    g = torch.Generator().manual_seed(11)
    x = torch.randn(B, S, N, D, generator=g)
    c = torch.randn(shape, generator=g)
    s = torch.randn(shape, generator=g)
    _, x64 = run_inplace(x, c, s, sl, twin=True)
    xs = f64(x)[..., sl[0]:sl[1]].reshape(B, S, N, L // 2, 2, 1)
    cb = np.broadcast_to(f64(c), (B, S, N, L)).reshape(B, S, N, L // 2, 2)
    sb = np.broadcast_to(f64(s), (B, S, N, L)).reshape(B, S, N, L // 2, 2)
    M = np.empty((B, S, N, L // 2, 2, 2))
    M[..., 0, 0] = cb[..., 0]
    M[..., 0, 1] = -sb[..., 0]
    M[..., 1, 0] = sb[..., 1]
    M[..., 1, 1] = cb[..., 1]
    y = (M @ xs).reshape(B, S, N, L)
    np.testing.assert_allclose(x64[..., sl[0]:sl[1]], y, rtol=1e-14, atol=1e-14)
    # untouched parts of the twin are the inputs
    assert (x64[..., : sl[0]] == f64(x)[..., : sl[0]]).all()
    assert (x64[..., sl[1]:] == f64(x)[..., sl[1]:]).all()


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("mrope", [None, [16, 24, 24], [8, 12, 12], [24, 20, 20], [11, 11, 10],
                                   [16, 16, 16, 16]])
def test_cache_matches_complex_multiplication(neox, mrope):
    """[RSCC §设计动机 / §rope 模式 / §mrope 模式 / style sections]: for each head, pair
    (x1[i], x2[i]) becomes (x1 + i*x2) * (cos_i + i*sin_i) with cos/sin gathered from the
    cache by NumPy fancy indexing and stitched with np.split per section.  NumPy complex128
    multiplication is the pin (float64 twin of the oracle)."""
    T, nq, nk, H = 37, 3, 2, 64
    rd = 2 * sum(mrope) if mrope else 32
    H = max(H, rd)
    g = torch.Generator().manual_seed(5)
    q = torch.randn(T, nq * H, generator=g)
    k = torch.randn(T, nk * H, generator=g)
    cache = torch.randn(50, rd, generator=g)
    m = len(mrope) if mrope else 0
    pos = (torch.randint(0, 50, (m, T), generator=g) if mrope else
           torch.randint(0, 50, (T,), generator=g))
    _, _, q64, k64 = run_cache(pos, q, k, cache, mrope, H, neox, twin=True)
    C = f64(cache)
    if mrope:
        rows = [C[p] for p in pos.numpy()]              # m x [T, rd]
        cs = [r[:, : rd // 2] for r in rows]
        sn = [r[:, rd // 2:] for r in rows]
        edges = np.cumsum(mrope)[:-1]
        cos = np.concatenate([np.split(c, edges, axis=1)[j] for j, c in enumerate(cs)], axis=1)
        sin = np.concatenate([np.split(s, edges, axis=1)[j] for j, s in enumerate(sn)], axis=1)
    else:
        cos, sin = C[pos.numpy(), : rd // 2], C[pos.numpy(), rd // 2:]
    w = cos + 1j * sin                                           # [T, rd/2]
    for inp, got in ((q, q64), (k, k64)):
        X = f64(inp).reshape(T, -1, H)
        rot = X[..., :rd]
        if neox:
            z = rot[..., : rd // 2] + 1j * rot[..., rd // 2:]
        else:
            z = rot[..., 0::2] + 1j * rot[..., 1::2]
        r = z * w[:, None, :]
        exp = X.copy()
        if neox:
            exp[..., : rd // 2], exp[..., rd // 2: rd] = r.real, r.imag
        else:
            exp[..., 0:rd:2], exp[..., 1:rd:2] = r.real, r.imag
        np.testing.assert_allclose(got.reshape(T, -1, H), exp, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("rd,extra", [(16384, 0), (16416, 32), (24576, 0)])
def test_cache_long_rotary_dim_matches_complex_multiplication(neox, rd, extra):
    """[RSCC §约束说明] bounds rotaryDim only by headSize and 64-byte alignment, so the oracle
    evaluates any length: rotaryDim of 16384 and beyond, checked as above against NumPy complex
    multiplication of every pair (float64 twin), the float32 outputs within the error bound
    of their twin, and the head's tail copied bit for bit."""
    T, nq, nk = 3, 2, 1
    H = rd + extra
    g = torch.Generator().manual_seed(rd + extra + int(neox))
    q = torch.randn(T, nq * H, generator=g)
    k = torch.randn(T, nk * H, generator=g)
    cache = torch.randn(7, rd, generator=g)
    pos = torch.tensor([6, 0, 3])
    qo, ko, q64, k64 = run_cache(pos, q, k, cache, None, H, neox, twin=True)
    C = f64(cache)
    w = C[pos.numpy(), : rd // 2] + 1j * C[pos.numpy(), rd // 2:]
    for inp, out, got in ((q, qo, q64), (k, ko, k64)):
        X = f64(inp).reshape(T, -1, H)
        rot = X[..., :rd]
        z = (rot[..., : rd // 2] + 1j * rot[..., rd // 2:]) if neox else \
            (rot[..., 0::2] + 1j * rot[..., 1::2])
        r = z * w[:, None, :]
        exp = X.copy()
        if neox:
            exp[..., : rd // 2], exp[..., rd // 2: rd] = r.real, r.imag
        else:
            exp[..., 0:rd:2], exp[..., 1:rd:2] = r.real, r.imag
        np.testing.assert_allclose(got.reshape(T, -1, H), exp, rtol=1e-13, atol=1e-13)
        o = f64(out).reshape(T, -1, H)
        # each output is two float32 products and one sum: within 2 ulp of the term sizes
        # (|x1*c| + |x2*s|, the same for both outputs of a pair)
        if neox:
            terms = np.abs(rot[..., : rd // 2]) * np.abs(w.real)[:, None] + \
                np.abs(rot[..., rd // 2:]) * np.abs(w.imag)[:, None]
            terms = np.concatenate([terms, np.abs(rot[..., : rd // 2]) * np.abs(w.imag)[:, None]
                                    + np.abs(rot[..., rd // 2:]) * np.abs(w.real)[:, None]], -1)
        else:
            a, b = np.abs(rot[..., 0::2]), np.abs(rot[..., 1::2])
            terms = np.empty_like(rot)
            terms[..., 0::2] = a * np.abs(w.real)[:, None] + b * np.abs(w.imag)[:, None]
            terms[..., 1::2] = b * np.abs(w.real)[:, None] + a * np.abs(w.imag)[:, None]
        assert np.all(np.abs(o[..., :rd] - exp[..., :rd]) <= 2.0 ** -22 * terms + 1e-45)
        assert np.array_equal(raw_bits(out).reshape(T, -1, H)[..., rd:],
                              raw_bits(inp).reshape(T, -1, H)[..., rd:])


def test_relative_position_property():
    """RoPE's defining property: <R(p) q, R(p') k> depends on p - p' only.  Tables hold
    exact-angle values rounded to float32, so equality holds to float32-table accuracy."""
    H = rd = 64
    cache = W.cos_sin_cache(300, rd, torch.float32)
    g = torch.Generator().manual_seed(3)
    q = torch.randn(1, H, generator=g)
    k = torch.randn(1, H, generator=g)
    dots = []
    for p, pk in [(5, 2), (105, 102), (255, 252)]:
        _, _, q64, _ = run_cache(torch.tensor([p]), q, k, cache, None, H, True, twin=True)
        _, _, k64, _ = run_cache(torch.tensor([pk]), k, q, cache, None, H, True, twin=True)
        dots.append(float(q64.ravel() @ k64.ravel()))
    nrm = float(q.norm() * k.norm())
    assert abs(dots[0] - dots[1]) < 1e-5 * nrm and abs(dots[0] - dots[2]) < 1e-5 * nrm
    # and a different offset gives a different product (the property is not vacuous)
    _, _, q64, _ = run_cache(torch.tensor([5]), q, k, cache, None, H, True, twin=True)
    _, _, k64, _ = run_cache(torch.tensor([9]), k, q, cache, None, H, True, twin=True)
    assert abs(float(q64.ravel() @ k64.ravel()) - dots[0]) > 1e-3 * nrm


# ------------------------------------------------------------------------------------------
# Exact special cases and invariants
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("cv,sv,kind", [(1.0, 0.0, "identity"), (0.0, 1.0, "quarter"),
                                        (-1.0, 0.0, "half")])
def test_exact_angles(dt, cv, sv, kind):
    g = torch.Generator().manual_seed(2)
    x = torch.randn(2, 3, 2, 16, generator=g).to(DT[dt])
    c = torch.full((2, 3, 1, 16), cv).to(DT[dt])
    s = torch.full((2, 3, 1, 16), sv).to(DT[dt])
    y, _ = run_inplace(x, c, s, None)
    a, b = f64(x)[..., 0::2], f64(x)[..., 1::2]
    ya, yb = f64(y)[..., 0::2], f64(y)[..., 1::2]
    if kind == "identity":
        ea, eb = a, b
    elif kind == "quarter":
        ea, eb = -b, a
    else:
        ea, eb = -a, -b
    assert (ya == ea).all() and (yb == eb).all()


def test_norm_preserved_per_pair():
    c2 = W.inplace_bf16_slice()
    x = c2.x[:1, :64]
    y, x64 = run_inplace(x, c2.cos[:1, :64], c2.sin[:1, :64], c2.partial_slice, twin=True)
    sl = slice(*c2.partial_slice)
    a0, b0 = f64(x)[..., sl][..., 0::2], f64(x)[..., sl][..., 1::2]
    a1, b1 = x64[..., sl][..., 0::2], x64[..., sl][..., 1::2]
    n0 = a0 ** 2 + b0 ** 2
    n1 = a1 ** 2 + b1 ** 2
    # tables are float32-rounded cos/sin, so c^2 + s^2 = 1 within ~1e-7
    assert np.max(np.abs(n1 - n0) / np.maximum(n0, 1e-30)) < 1e-6


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_untouched_and_noop_bit_identical(dt):
    """[IPRM §partial_slice 局部旋转机制]: [0,start) and [end,D) keep their values, and
    start == end does nothing -- bit for bit, signalling-NaN canaries included."""
    g = torch.Generator().manual_seed(4)
    x = torch.randn(2, 5, 3, 40, generator=g).to(DT[dt])
    bits = raw_bits(x).copy()
    snan = {"f32": 0x7F800001, "f16": 0x7C01, "bf16": 0x7F81}[dt]
    bits[..., :7] = snan
    bits[..., 31:] = np.array(0xFFFF if dt != "f32" else 0xFFFFFFFF, dtype=bits.dtype)
    if dt == "f32":
        x = torch.from_numpy(bits.view(np.float32).copy())
    else:
        x = torch.from_numpy(bits.view(np.int16).copy()).view(DT[dt])
    c = torch.randn(2, 5, 1, 24, generator=g).to(DT[dt])
    s = torch.randn(2, 5, 1, 24, generator=g).to(DT[dt])
    y, _ = run_inplace(x, c, s, [7, 31])
    yb = raw_bits(y)
    assert (yb[..., :7] == bits[..., :7]).all() and (yb[..., 31:] == bits[..., 31:]).all()
    assert (yb[..., 7:31] != bits[..., 7:31]).any()
    # no-op: start == end, even with cos/sin whose last dim does not match (reading R3)
    z, _ = run_inplace(x, c, s, [12, 12])
    assert (raw_bits(z) == bits).all()


def test_styles_equivalent_under_permutation():
    """NeoX(P x) = P GPTJ(x) bit for bit, P mapping interleaved to half order."""
    T, H, rd = 9, 128, 64
    g = torch.Generator().manual_seed(8)
    x = torch.randn(T, 2 * H, generator=g).to(torch.bfloat16)
    cache = torch.randn(20, rd, generator=g).to(torch.bfloat16)
    pos = torch.randint(0, 20, (T,), generator=g)
    perm = torch.cat([torch.arange(0, rd, 2), torch.arange(1, rd, 2), torch.arange(rd, H)])
    xp = x.reshape(T, 2, H)[:, :, perm].reshape(T, 2 * H).contiguous()
    q_j, _, _, _ = run_cache(pos, x, x.clone(), cache, None, H, False)
    q_n, _, _, _ = run_cache(pos, xp, xp.clone(), cache, None, H, True)
    permuted = q_j.reshape(T, 2, H)[:, :, perm].reshape(T, 2 * H).contiguous()
    assert (raw_bits(permuted) == raw_bits(q_n)).all()


def test_inplace_interleave_equals_cache_gptj():
    """Cross-op: the in-place interleave op with cos/sin repeated per pair is the cache op in
    GPT-J style on the same data (the two pages describe the same rotation), bit for bit."""
    T, H = 11, 64
    g = torch.Generator().manual_seed(9)
    x = torch.randn(T, H, generator=g).to(torch.float16)
    cache = torch.randn(T, H, generator=g).to(torch.float16)
    pos = torch.arange(T)
    out, _, _, _ = run_cache(pos, x, x.clone(), cache, None, H, False)
    c = cache[:, : H // 2].repeat_interleave(2, dim=1).reshape(1, T, 1, H).contiguous()
    s = cache[:, H // 2:].repeat_interleave(2, dim=1).reshape(1, T, 1, H).contiguous()
    y, _ = run_inplace(x.reshape(1, T, 1, H), c, s, None)
    assert (raw_bits(y.reshape(T, H)) == raw_bits(out)).all()


@pytest.mark.parametrize("sec", [[16, 24, 24], [11, 11, 10], [16, 16, 16, 16]])
def test_mrope_equal_rows_is_rope(sec):
    T, H = 13, 128
    rd = 2 * sum(sec)
    g = torch.Generator().manual_seed(10)
    q = torch.randn(T, 2 * H, generator=g).to(torch.bfloat16)
    k = torch.randn(T, H, generator=g).to(torch.bfloat16)
    cache = torch.randn(40, rd, generator=g).to(torch.bfloat16)
    p = torch.randint(0, 40, (T,), generator=g)
    a = run_cache(p, q, k, cache, None, H, True)
    b = run_cache(p.repeat(len(sec), 1).contiguous(), q, k, cache, sec, H, True)
    assert (raw_bits(a[0]) == raw_bits(b[0])).all() and (raw_bits(a[1]) == raw_bits(b[1])).all()


def test_pass_through_bits_cache_op():
    T, H, rd = 5, 128, 64
    g = torch.Generator().manual_seed(12)
    q = torch.randn(T, H, generator=g).to(torch.float16)
    bits = raw_bits(q).copy()
    bits[:, rd:] = 0x7C01  # signalling NaN canaries in the pass-through part
    q = torch.from_numpy(bits.view(np.int16).copy()).view(torch.float16)
    cache = torch.randn(8, rd, generator=g).to(torch.float16)
    qo, ko, _, _ = run_cache(torch.arange(T) % 8, q, q.clone(), cache, None, H, False)
    assert (raw_bits(qo)[:, rd:] == bits[:, rd:]).all()


# ------------------------------------------------------------------------------------------
# float32 arithmetic against the float64 twin (error bound of two products and one sum)
# ------------------------------------------------------------------------------------------

def test_fp32_within_bound_of_twin():
    """|fl(fl(ac) - fl(bs)) - (ac - bs)| <= u(|ac| + |bs|) + u|result| with u = 2^-24,
    so 2^-23 (|ac| + |bs|) bounds it; the contract's 2e-6 relative is far looser."""
    T, H = 64, 128
    g = torch.Generator().manual_seed(13)
    q = torch.randn(T, 4 * H, generator=g) * torch.exp(torch.randn(T, 4 * H, generator=g) * 3)
    cache = torch.randn(64, H, generator=g)
    pos = torch.randint(0, 64, (T,), generator=g)
    qo, _, q64, _ = run_cache(pos, q, q[:, :H].clone(), cache, None, H, True, twin=True)
    X = f64(q).reshape(T, 4, H)
    C = f64(cache)[pos.numpy()]
    c, s = C[:, None, : H // 2], C[:, None, H // 2:]
    a, b = X[..., : H // 2], X[..., H // 2:]
    scale = np.concatenate([np.abs(a * c) + np.abs(b * s), np.abs(b * c) + np.abs(a * s)], -1)
    err = np.abs(f64(qo).reshape(T, 4, H) - q64.reshape(T, 4, H))
    assert (err <= 2.0 ** -23 * scale * (1 + 1e-6)).all()


# ------------------------------------------------------------------------------------------
# Validation: the error table of [IPRM §返回值与错误码] and the checks of [RSCC §入参校验逻辑]
# ------------------------------------------------------------------------------------------

def test_oracle_refuses_out_of_range_positions_without_writing():
    q = torch.randn(3, 64).to(torch.bfloat16)
    cache = torch.randn(4, 32).to(torch.bfloat16)
    qo = torch.zeros_like(q)
    ko = torch.zeros_like(q)
    st, _, _ = oracle.rope_with_cos_sin_cache(torch.tensor([0, 4, 1]), q, q.clone(), cache,
                                              None, 32, True, qo, ko)
    assert st == oracle.ERR_OUTSIDE_CONTRACT
    assert (raw_bits(qo) == 0).all()


# ------------------------------------------------------------------------------------------
# Backward of the in-place op ([IPRM §Python 接口与自动微分]; the transpose of the pair map)
# ------------------------------------------------------------------------------------------

def run_backward(g, cos, sin, sl, twin=False, mode=1):
    g = g.clone()
    st, g64 = oracle.rope_partial_inplace_backward(g, cos, sin, mode, sl, twin=twin)
    assert st == oracle.OK, oracle.last_error()
    return g, g64


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_golden_backward(dt):
    gj = golden("t7_backward_pairs.json")
    g = torch.tensor(gj["grad"], dtype=DT[dt]).reshape(gj["x_shape"])
    c = torch.tensor(gj["cos"], dtype=DT[dt]).reshape(1, 1, 1, 4)
    s = torch.tensor(gj["sin"], dtype=DT[dt]).reshape(1, 1, 1, 4)
    dx, _ = run_backward(g, c, s, gj["partial_slice"])
    assert f64(dx).ravel().tolist() == gj["expected"]


@pytest.mark.parametrize("cos_layout", ["BSND", "BS1D", "B11D", "1S1D"])
def test_backward_is_adjoint_of_forward(cos_layout):
    """<F(x), v> = <x, B(v)> for random x, v and per-element cos/sin (float64 twins)."""
    B_, S, N, D, sl = 2, 5, 3, 24, [4, 20]
    L = sl[1] - sl[0]
    shape = {"BSND": (B_, S, N, L), "BS1D": (B_, S, 1, L), "B11D": (B_, 1, 1, L),
             "1S1D": (1, S, 1, L)}[cos_layout]
    gen = torch.Generator().manual_seed(21)
    x = torch.randn(B_, S, N, D, generator=gen)
    v = torch.randn(B_, S, N, D, generator=gen)
    c = torch.randn(shape, generator=gen)
    s = torch.randn(shape, generator=gen)
    _, fx = run_inplace(x, c, s, sl, twin=True)
    _, bv = run_backward(v, c, s, sl, twin=True)
    lhs = float((fx * f64(v)).sum())
    rhs = float((f64(x) * bv).sum())
    assert abs(lhs - rhs) <= 1e-12 * (abs(lhs) + abs(rhs) + 1)


def test_backward_matches_torch_autograd():
    """PyTorch autograd of the forward written with tensor ops in float64 (x2 = odd
    elements, x1 = even ones, the pairwise rotation assembled with torch.stack)."""
    B_, S, N, D, sl = 2, 4, 2, 16, [2, 14]
    gen = torch.Generator().manual_seed(22)
    x = torch.randn(B_, S, N, D, generator=gen, dtype=torch.float64, requires_grad=True)
    c = torch.randn(B_, S, 1, sl[1] - sl[0], generator=gen, dtype=torch.float64)
    s = torch.randn(B_, S, 1, sl[1] - sl[0], generator=gen, dtype=torch.float64)
    g = torch.randn(B_, S, N, D, generator=gen, dtype=torch.float64)
    part = x[..., sl[0]:sl[1]]
    x1, x2 = part[..., 0::2], part[..., 1::2]
    rot = torch.stack((-x2, x1), dim=-1).flatten(-2)
    y = torch.cat([x[..., :sl[0]], part * c + rot * s, x[..., sl[1]:]], dim=-1)
    (grad,) = torch.autograd.grad(y, x, g)
    _, g64 = run_backward(g.float(), c.float(), s.float(), sl, twin=True)
    # the oracle reads float32 copies of c, s and g: compare at float32 input precision
    np.testing.assert_allclose(g64, grad.numpy(), rtol=2e-6, atol=2e-6)


def test_backward_inverts_rotation():
    case = W.inplace_case("inv", 2, 64, 2, 96, torch.float32, torch.float32, [32, 96], seed=23)
    y, _ = run_inplace(case.x, case.cos, case.sin, case.partial_slice)
    back, _ = run_backward(y, case.cos, case.sin, case.partial_slice)
    np.testing.assert_allclose(f64(back), f64(case.x), rtol=0, atol=1e-5)


def test_backward_untouched_and_noop():
    g = torch.randn(2, 3, 2, 20, generator=torch.Generator().manual_seed(24)).to(torch.bfloat16)
    c = torch.randn(2, 3, 1, 8).to(torch.bfloat16)
    out, _ = run_backward(g, c, c.clone(), [6, 14])
    assert (raw_bits(out)[..., :6] == raw_bits(g)[..., :6]).all()
    assert (raw_bits(out)[..., 14:] == raw_bits(g)[..., 14:]).all()
    same, _ = run_backward(g, c, c.clone(), [6, 6])
    assert (raw_bits(same) == raw_bits(g)).all()


@pytest.mark.parametrize("direction", ["forward", "backward"])
def test_inplace_fp32_within_bound_of_twin(direction):
    """The float32 results equal the float64 twin within 2^-23 (|p| + |q|) per element, with
    per-element (not pair-repeated) cos/sin: ties the float32 path to the twin that the
    adjoint, matrix and autograd pins check."""
    gen = torch.Generator().manual_seed(25)
    x = torch.randn(3, 7, 2, 40, generator=gen) * torch.exp(torch.randn(3, 7, 2, 40, generator=gen))
    c = torch.randn(3, 7, 1, 32, generator=gen)
    s = torch.randn(3, 7, 1, 32, generator=gen)
    sl = [4, 36]
    run = run_inplace if direction == "forward" else run_backward
    y, y64 = run(x, c, s, sl, twin=True)
    a, b = f64(x)[..., 4:36:2], f64(x)[..., 5:36:2]
    cb = np.broadcast_to(f64(c), (3, 7, 2, 32))
    sb = np.broadcast_to(f64(s), (3, 7, 2, 32))
    c0, c1, s0, s1 = cb[..., 0::2], cb[..., 1::2], sb[..., 0::2], sb[..., 1::2]
    scale = np.empty((3, 7, 2, 32))
    if direction == "forward":
        scale[..., 0::2] = np.abs(a * c0) + np.abs(b * s0)
        scale[..., 1::2] = np.abs(b * c1) + np.abs(a * s1)
    else:
        scale[..., 0::2] = np.abs(a * c0) + np.abs(b * s1)
        scale[..., 1::2] = np.abs(b * c1) + np.abs(a * s0)
    err = np.abs(f64(y)[..., 4:36] - y64[..., 4:36])
    assert (err <= 2.0 ** -23 * scale * (1 + 1e-6)).all()


# ------------------------------------------------------------------------------------------
# V2 cacheMode = 1: interleaved mrope stitching ([RSCC §V2 接口：cacheMode 扩展])
# ------------------------------------------------------------------------------------------

def run_cache_v2(pos, q, k, cache, msec, H, neox, mode, twin=False):
    qo = torch.empty_like(q, memory_format=torch.contiguous_format)
    ko = torch.empty_like(k, memory_format=torch.contiguous_format)
    st, q64, k64 = oracle.rope_with_cos_sin_cache(pos, q, k, cache, msec, H, neox, qo, ko,
                                                  twin=twin, cache_mode=mode)
    return st, qo, ko, q64, k64


@pytest.mark.parametrize("case_i", [0, 1])
def test_golden_mrope_interleaved(case_i):
    g = golden("t8_mrope_interleaved.json")
    cs = g["cases"][case_i]
    rd = H = cs["rotary_dim"]
    cache = torch.zeros(4, rd)
    for p in range(4):
        cache[p, : rd // 2] = p
        cache[p, rd // 2:] = 10 * p
    cache = cache.to(torch.bfloat16)
    head = torch.zeros(H)
    head[: rd // 2] = 1.0
    q = head.reshape(1, H).to(torch.bfloat16)
    st, qo, _, _, _ = run_cache_v2(torch.tensor(g["positions"]), q, q.clone(), cache,
                                   cs["mrope_section"], H, True, 1)
    assert st == 0, oracle.last_error()
    out = f64(qo).ravel()
    for i in range(rd // 2):
        exp = cs["expected_cos_by_index_mod3"][i % 3]
        if cs["tail_from"] is not None and i >= cs["tail_from"]:
            exp = cs["expected_cos_by_index_mod3"][0]
        assert out[i] == exp and out[rd // 2 + i] == 10 * exp, i


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("sec", [[16, 24, 24], [8, 12, 12], [24, 20, 20], [11, 11, 10]])
def test_interleaved_matches_complex_multiplication(neox, sec):
    """NumPy: start from row 0's cos/sin, overwrite the slices 1::3 and 2::3 below
    3*mropeSection[1] from rows 1 and 2, then complex multiplication per pair."""
    T, H = 29, 128
    rd = 2 * sum(sec)
    gen = torch.Generator().manual_seed(26)
    q = torch.randn(T, 3 * H, generator=gen)
    k = torch.randn(T, H, generator=gen)
    cache = torch.randn(40, rd, generator=gen)
    pos = torch.randint(0, 40, (3, T), generator=gen)
    st, _, _, q64, k64 = run_cache_v2(pos, q, k, cache, sec, H, neox, 1, twin=True)
    assert st == 0, oracle.last_error()
    C = f64(cache)
    gathered = C[pos.numpy()]                      # [3, T, rd]
    cos = gathered[0, :, : rd // 2].copy()
    sin = gathered[0, :, rd // 2:].copy()
    for r in (1, 2):
        sl = slice(r, sec[1] * 3, 3)
        cos[:, sl] = gathered[r, :, : rd // 2][:, sl]
        sin[:, sl] = gathered[r, :, rd // 2:][:, sl]
    w = cos + 1j * sin
    for inp, got in ((q, q64), (k, k64)):
        X = f64(inp).reshape(T, -1, H)
        if neox:
            z = X[..., : rd // 2] + 1j * X[..., rd // 2: rd]
        else:
            z = X[..., 0:rd:2] + 1j * X[..., 1:rd:2]
        r_ = z * w[:, None, :]
        exp = X.copy()
        if neox:
            exp[..., : rd // 2], exp[..., rd // 2: rd] = r_.real, r_.imag
        else:
            exp[..., 0:rd:2], exp[..., 1:rd:2] = r_.real, r_.imag
        np.testing.assert_allclose(got.reshape(T, -1, H), exp, rtol=1e-13, atol=1e-13)


def test_interleaved_equal_rows_and_rope_mode_and_validation():
    T, H = 11, 128
    gen = torch.Generator().manual_seed(27)
    q = torch.randn(T, 2 * H, generator=gen).to(torch.bfloat16)
    cache = torch.randn(30, 128, generator=gen).to(torch.bfloat16)
    p = torch.randint(0, 30, (T,), generator=gen)
    rope = run_cache(p, q, q[:, :H].clone(), cache, None, H, True)
    st, qo, ko, _, _ = run_cache_v2(p.repeat(3, 1).contiguous(), q, q[:, :H].clone(), cache,
                                    [16, 24, 24], H, True, 1)
    assert st == 0 and (raw_bits(qo) == raw_bits(rope[0])).all()
    # cacheMode has no effect in rope mode
    st, qo, _, _, _ = run_cache_v2(p, q, q[:, :H].clone(), cache, None, H, True, 1)
    assert st == 0 and (raw_bits(qo) == raw_bits(rope[0])).all()
    # cacheMode outside {0, 1}, and 1 with the 4-section list, are refused
    st, *_ = run_cache_v2(p, q, q[:, :H].clone(), cache, None, H, True, 2)
    assert st == oracle.ERR_PARAM_INVALID
    st, *_ = run_cache_v2(p.repeat(4, 1).contiguous(), q, q[:, :H].clone(), cache,
                          [16, 16, 16, 16], H, True, 1)
    assert st == oracle.ERR_PARAM_INVALID


# ------------------------------------------------------------------------------------------
# Half mode, rotary_mode = 0 ([IPRM §参数说明]; reading R21: x1, x2 are the slice's halves)
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("direction", ["forward", "backward"])
@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_golden_half_mode(dt, direction):
    gj = golden("t9_half_mode.json")
    x = torch.tensor(gj["x"], dtype=DT[dt]).reshape(gj["x_shape"])
    c = torch.tensor(gj["cos"], dtype=DT[dt]).reshape(1, 1, 1, 4)
    s = torch.tensor(gj["sin"], dtype=DT[dt]).reshape(1, 1, 1, 4)
    run = run_inplace if direction == "forward" else run_backward
    y, _ = run(x, c, s, gj["partial_slice"], mode=0)
    assert f64(y).ravel().tolist() == gj[f"expected_{direction}"]


def half_to_interleave(n):
    """Index map taking a slice in half layout (x1 then x2) to the interleaved layout:
    interleaved element 2i is half element i, 2i+1 is half element i + n/2."""
    h = n // 2
    idx = np.empty(n, dtype=np.int64)
    idx[0::2] = np.arange(h)
    idx[1::2] = np.arange(h) + h
    return idx


@pytest.mark.parametrize("direction", ["forward", "backward"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_half_mode_is_interleave_after_permutation(dt, direction):
    """Half mode on (x, cos, sin) equals interleave mode (pinned on its own) on the same slice
    with its elements, cos and sin permuted so that the pairs (i, i + L/2) become adjacent:
    bit for bit, since each output is the same two float32 products and one sum."""
    gen = torch.Generator().manual_seed(41)
    B_, S, N, D, sl = 2, 5, 3, 40, [6, 38]
    L = sl[1] - sl[0]
    x = torch.randn(B_, S, N, D, generator=gen).to(DT[dt])
    c = torch.randn(B_, S, 1, L, generator=gen).to(DT[dt])
    s = torch.randn(B_, S, 1, L, generator=gen).to(DT[dt])
    perm = torch.from_numpy(half_to_interleave(L))
    xp = x.clone()
    xp[..., sl[0]:sl[1]] = x[..., sl[0]:sl[1]][..., perm]
    run = run_inplace if direction == "forward" else run_backward
    y_half, _ = run(x, c, s, sl, mode=0)
    y_int, _ = run(xp, c[..., perm].contiguous(), s[..., perm].contiguous(), sl, mode=1)
    back = y_int.clone()
    back[..., sl[0] + perm] = y_int[..., sl[0]:sl[1]]
    assert (raw_bits(y_half) == raw_bits(back)).all()


@pytest.mark.parametrize("cos_layout", ["BSND", "BS1D", "B11D", "111D"])
def test_half_mode_matches_complex_multiplication(cos_layout):
    """With the rotate-half table layout (cos[i] = cos[i + L/2] = cos(theta_i), same for sin),
    half mode multiplies z_i = x[i] + j x[i + L/2] by e^{j theta_i} (NumPy complex128)."""
    B_, S, N, D, sl = 2, 6, 4, 48, [8, 40]
    L, h = sl[1] - sl[0], (sl[1] - sl[0]) // 2
    cshape = {"BSND": (B_, S, N, h), "BS1D": (B_, S, 1, h), "B11D": (B_, 1, 1, h),
              "111D": (1, 1, 1, h)}[cos_layout]
    gen = torch.Generator().manual_seed(42)
    x = torch.randn(B_, S, N, D, generator=gen, dtype=torch.float64)
    theta = torch.rand(cshape, generator=gen, dtype=torch.float64) * 6.283
    c = torch.cat([torch.cos(theta)] * 2, dim=-1).float()
    s = torch.cat([torch.sin(theta)] * 2, dim=-1).float()
    xf = x.float()
    _, y64 = run_inplace(xf, c, s, sl, twin=True, mode=0)
    xs = f64(xf)[..., sl[0]:sl[1]]
    z = xs[..., :h] + 1j * xs[..., h:]
    # the float32 tables' own (cos, sin) as the unit complex number e^{j theta}
    rot = np.broadcast_to(f64(c)[..., :h] + 1j * f64(s)[..., :h], z.shape)
    w = z * rot
    np.testing.assert_allclose(y64[..., sl[0]:sl[0] + h], w.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y64[..., sl[0] + h:sl[1]], w.imag, rtol=0, atol=1e-12)
    assert (y64[..., :sl[0]] == f64(xf)[..., :sl[0]]).all()
    assert (y64[..., sl[1]:] == f64(xf)[..., sl[1]:]).all()


def test_half_mode_backward_adjoint_and_autograd():
    """<F(x), v> = <x, B(v)> with per-element tables, and B equals PyTorch autograd of the
    half-mode forward written with torch.chunk / torch.cat in float64."""
    B_, S, N, D, sl = 2, 4, 3, 36, [4, 36]
    L = sl[1] - sl[0]
    gen = torch.Generator().manual_seed(43)
    x = torch.randn(B_, S, N, D, generator=gen, dtype=torch.float64)
    v = torch.randn(B_, S, N, D, generator=gen, dtype=torch.float64)
    c = torch.randn(B_, S, 1, L, generator=gen, dtype=torch.float64)
    s = torch.randn(B_, S, 1, L, generator=gen, dtype=torch.float64)
    _, fx = run_inplace(x.float(), c.float(), s.float(), sl, twin=True, mode=0)
    _, bv = run_backward(v.float(), c.float(), s.float(), sl, twin=True, mode=0)
    lhs = float((fx * f64(v.float())).sum())
    rhs = float((f64(x.float()) * bv).sum())
    assert abs(lhs - rhs) <= 1e-12 * (abs(lhs) + abs(rhs) + 1)

    xr = x.float().double().requires_grad_(True)
    cf, sf = c.float().double(), s.float().double()
    part = xr[..., sl[0]:sl[1]]
    x1, x2 = torch.chunk(part, 2, dim=-1)
    y = torch.cat([xr[..., :sl[0]], part * cf + torch.cat((-x2, x1), dim=-1) * sf,
                   xr[..., sl[1]:]], dim=-1)
    (grad,) = torch.autograd.grad(y, xr, v.float().double())
    np.testing.assert_allclose(bv, grad.numpy(), rtol=1e-12, atol=1e-12)


def test_half_mode_untouched_noop_and_inverse():
    gen = torch.Generator().manual_seed(44)
    x = torch.randn(2, 3, 2, 20, generator=gen).to(torch.bfloat16)
    c = torch.randn(2, 3, 1, 8, generator=gen).to(torch.bfloat16)
    out, _ = run_inplace(x, c, c.clone(), [6, 14], mode=0)
    assert (raw_bits(out)[..., :6] == raw_bits(x)[..., :6]).all()
    assert (raw_bits(out)[..., 14:] == raw_bits(x)[..., 14:]).all()
    same, _ = run_inplace(x, c, c.clone(), [6, 6], mode=0)
    assert (raw_bits(same) == raw_bits(x)).all()
    # rotate-half tables: the gradient op undoes the rotation (R^T R = I)
    theta = torch.rand(2, 3, 1, 16, generator=gen, dtype=torch.float64) * 6.283
    cc = torch.cat([torch.cos(theta)] * 2, -1).float()
    ss = torch.cat([torch.sin(theta)] * 2, -1).float()
    xf = torch.randn(2, 3, 2, 40, generator=gen)
    y, _ = run_inplace(xf, cc, ss, [4, 36], mode=0)
    back, _ = run_backward(y, cc, ss, [4, 36], mode=0)
    np.testing.assert_allclose(f64(back), f64(xf), rtol=0, atol=1e-5)


def test_rotary_modes_other_than_0_and_1_refused():
    x = torch.zeros(1, 2, 1, 8)
    c = torch.zeros(1, 2, 1, 8)
    for mode in (2, 3, -1):
        st, _ = oracle.rope_partial_inplace(x, c, c, mode, None)
        assert st == oracle.ERR_PARAM_INVALID
