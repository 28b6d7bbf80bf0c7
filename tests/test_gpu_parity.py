"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element.

Tolerances are in tests/parity.py: bf16/f16 within 1 ulp of the oracle's float32-then-rounded
value, f32 within 2e-6 of the exact value relative to the magnitude of the products, data
outside the rotated range bit-exact.  Inputs are seeded and synthetic (rope_workloads.py).

Pages:
  [IPRM] "CANN ops-transformer 的 aclnnInplacePartialRotaryMul 算子：Inplace 部分旋转位置编码接口详解与实现剖析"
  [RSCC] "CANN ops-transformer 旋转位置编码算子 RopeWithSinCosCache 深度解析：cache 化 RoPE 的计算原理与 aclnn 两段式调用实战"
"""
import numpy as np
import pytest
import torch

import oracle
import rope_partial_inplace_amd as ra
import rope_workloads as W
from parity import (as_f64, bits, cache_scale, check_bits_equal, check_f32, check_half,
                    gathered_tables, inplace_scale)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
HALF = (torch.float16, torch.bfloat16)


# ------------------------------------------------------------------------------------------
# in-place op
# ------------------------------------------------------------------------------------------

def check_inplace(x_before, x_after_gpu, cos, sin, sl, what, mode=1):
    """x_before: host copy of x before the call; the rest compared to the oracle."""
    x_cpu = x_before.clone()
    c_cpu, s_cpu = cos.cpu(), sin.cpu()
    st, x64 = oracle.rope_partial_inplace(x_cpu, c_cpu, s_cpu, mode, sl, twin=True)
    assert st == 0, oracle.last_error()
    D = x_before.shape[-1]
    start, end = (0, D) if sl is None else sl
    got = x_after_gpu.cpu()
    # untouched data: bit-exact
    check_bits_equal(got[..., :start], x_before[..., :start], what + " [0,start)")
    check_bits_equal(got[..., end:], x_before[..., end:], what + " [end,D)")
    if x_before.dtype in HALF:
        return check_half(got[..., start:end], x_cpu[..., start:end], what)
    scale = inplace_scale(x_before, c_cpu, s_cpu, start, end, mode)
    return check_f32(got[..., start:end], x64[..., start:end], scale, what)


def run_inplace(case, stream=None):
    x = case.x.to(DEV)
    before = x.cpu()
    ra.rope_partial_inplace(x, case.cos.to(DEV), case.sin.to(DEV), case.rotary_mode,
                            case.partial_slice, stream=stream)
    torch.cuda.synchronize()
    return before, x


@pytest.mark.parametrize("cfg", ["inplace_f32_1x16x2x64", "inplace_bf16_8x4096x1x576_s512",
                                 "inplace_half_bf16_8x4096x1x576_s512",
                                 "inplace_heads_bf16_4x2048x32x192_s128_bs1d"])
def test_inplace_configs_full(cfg):
    case = W.CONFIGS[cfg](DEV)
    before, x = run_inplace(case)
    check_inplace(before, x, case.cos, case.sin, case.partial_slice, case.name,
                  case.rotary_mode)


def test_inplace_f32_scaled_full_and_pair_norms():
    """The 768 MiB fp32 workload [1,524288,2,64], the launch the benchmark times: every
    element compared with the oracle (bit for bit, and within the fp32 bound of the oracle's
    float64 twin), and for every pair the norm kept: the tables hold cos and sin of one angle
    per pair, so |(y0, y1)|^2 = |(x0, x1)|^2 up to the fp32 roundings of the tables and the
    four products (about 11 units of 2^-24 in all)."""
    case = W.CONFIGS["inplace_f32_1x524288x2x64"](DEV)
    x = case.x
    before = x.clone()
    ra.rope_partial_inplace(x, case.cos, case.sin, 1, case.partial_slice)
    torch.cuda.synchronize()
    S = x.shape[1]
    ref = before.cpu()
    assert oracle.rope_partial_inplace(ref, case.cos.cpu(), case.sin.cpu(), 1,
                                       case.partial_slice)[0] == 0
    check_bits_equal(x.cpu(), ref, case.name + " all positions")
    check_inplace(before.cpu(), x, case.cos, case.sin, case.partial_slice,
                  case.name + " all positions")
    for h in range(0, S, 1 << 17):  # fp64 norms in slices of the sequence
        a = before[:, h:h + (1 << 17)].double().view(-1, 2)
        y = x[:, h:h + (1 << 17)].double().view(-1, 2)
        na, ny = (a * a).sum(1), (y * y).sum(1)
        worst = ((ny - na).abs() / na.clamp_min(1e-300)).max().item()
        assert worst <= 2e-6, f"pair norm changed by {worst:.3g} in positions [{h}, {h + (1 << 17)})"


LAYOUTS = {"BSND": lambda B, S, N: (B, S, N), "BS1D": lambda B, S, N: (B, S, 1),
           "B1ND": lambda B, S, N: (B, 1, N), "B11D": lambda B, S, N: (B, 1, 1),
           "111D": lambda B, S, N: (1, 1, 1), "1SND": lambda B, S, N: (1, S, N)}
DTYPE_PAIRS = [(torch.float32, torch.float32), (torch.float16, torch.float16),
               (torch.float16, torch.float32), (torch.bfloat16, torch.bfloat16),
               (torch.bfloat16, torch.float32)]


@pytest.mark.parametrize("xdt,cdt", DTYPE_PAIRS, ids=lambda d: str(d).split(".")[-1])
@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("shape,sl", [((3, 37, 5, 96), [16, 80]),    # ragged rows, inner slice
                                      ((2, 65, 3, 64), None),        # whole D
                                      ((1, 300, 2, 40), [1, 37]),    # odd start: element path
                                      ((4, 7, 1, 1024), [0, 1024]),  # D at its maximum
                                      ((2, 3, 2, 10), [4, 6]),       # one pair per row
                                      ((2, 33, 8, 64), None),        # 8 heads per lane
                                      ((3, 17, 12, 96), [32, 96]),   # 4 heads per lane
                                      ((2, 9, 6, 48), [16, 48])])    # 2 heads per lane
def test_inplace_sweep(xdt, cdt, layout, shape, sl):
    B, S, N, D = shape
    start, end = (0, D) if sl is None else sl
    L = end - start
    cshape = LAYOUTS[layout](B, S, N) + (L,)
    case = W.inplace_case("sweep", B, S, N, D, xdt, cdt, sl, cos_shape=cshape, seed=B * 7 + S,
                          table="randn", device=DEV)
    before, x = run_inplace(case)
    check_inplace(before, x, case.cos, case.sin, sl, f"{layout} {shape} {sl} {xdt}/{cdt}")


def test_inplace_cos_and_sin_may_share_memory():
    """cos and sin are only read, so one tensor may serve as both (reading R22 forbids only
    overlap with x)."""
    case = W.inplace_case("shared", 2, 33, 4, 64, torch.bfloat16, torch.float32, [0, 64],
                          seed=9, table="randn", device=DEV)
    before, x = case.x.cpu(), case.x
    ra.rope_partial_inplace(x, case.cos, case.cos, 1, [0, 64])
    torch.cuda.synchronize()
    check_inplace(before, x, case.cos, case.cos, [0, 64], "cos and sin one tensor")


def test_inplace_misaligned_base_uses_element_path():
    """x starts 2 bytes past a 16-byte boundary: the library must take its element-wise path
    and still match."""
    B, S, N, D = 2, 33, 3, 64
    buf = torch.randn(B * S * N * D + 8, device=DEV).to(torch.bfloat16)
    x = buf[1:1 + B * S * N * D].view(B, S, N, D)
    c = torch.randn(B, S, 1, 32, device=DEV)
    s = torch.randn(B, S, 1, 32, device=DEV)
    before = x.cpu()
    ra.rope_partial_inplace(x, c, s, 1, [16, 48])
    torch.cuda.synchronize()
    check_inplace(before, x, c, s, [16, 48], "misaligned bf16")


def test_inplace_noop_and_empty_leave_x_untouched():
    x = torch.randn(2, 8, 2, 32, device=DEV).to(torch.float16)
    ref = x.clone()
    c = torch.randn(2, 8, 1, 5, device=DEV).to(torch.float16)  # last dim irrelevant for a no-op
    ra.rope_partial_inplace(x, c, c, 1, [10, 10])
    e = torch.empty(0, 8, 2, 32, device=DEV, dtype=torch.float16)
    ra.rope_partial_inplace(e, torch.randn(1, 8, 1, 32, device=DEV).half(),
                            torch.randn(1, 8, 1, 32, device=DEV).half(), 1, None)
    torch.cuda.synchronize()
    check_bits_equal(x, ref, "no-op")


@pytest.mark.parametrize("dt", [torch.float32, torch.float16, torch.bfloat16])
def test_inplace_canaries_and_specials(dt):
    """Signalling-NaN canaries outside the slice stay bit-identical; NaN/Inf inside the slice
    propagate as the oracle says."""
    B, S, N, D = 2, 50, 2, 48
    g = W.generator(3, DEV)
    x = W.randn((B, S, N, D), dt, g)
    raw = x.view(torch.int32 if dt == torch.float32 else torch.int16)
    snan = 0x7F800001 if dt == torch.float32 else (0x7C01 if dt == torch.float16 else 0x7F81)
    raw[..., :8] = snan
    raw[..., 40:] = -1
    flat = x.view(-1)
    flat[8 * 3 + 11] = float("nan")
    flat[D * 5 + 9] = float("inf")
    flat[D * 9 + 20] = float("-inf")
    c = W.randn((B, S, 1, 32), dt, g)
    s = W.randn((B, S, 1, 32), dt, g)
    c.view(-1)[17] = float("inf")
    before = x.cpu()
    ra.rope_partial_inplace(x, c, s, 1, [8, 40])
    torch.cuda.synchronize()
    check_inplace(before, x, c, s, [8, 40], f"specials {dt}")


# Scales that put N(0,1) values into each dtype's subnormal range (below 2^-126 for f32 and
# bf16, below 2^-14 for f16), so inputs and products are subnormal.  There the f32 rounding
# error is absolute, so the relative f32 bound does not apply; instead the GPU result must
# equal the oracle's float32 result bit for bit (same operations in the same order, IEEE
# subnormals on both sides): a kernel that flushed subnormals to zero would differ.
SUBNORMAL_SCALE = {torch.float32: 2.0 ** -130, torch.bfloat16: 2.0 ** -130,
                   torch.float16: 2.0 ** -17}


@pytest.mark.parametrize("xdt,cdt", DTYPE_PAIRS, ids=lambda d: str(d).split(".")[-1])
def test_inplace_subnormal_inputs(xdt, cdt):
    B, S, N, D = 2, 40, 3, 64
    g = W.generator(21, DEV)
    x = (W.randn((B, S, N, D), torch.float32, g) * SUBNORMAL_SCALE[xdt]).to(xdt)
    c = W.randn((B, S, 1, 48), cdt, g)
    s = W.randn((B, S, 1, 48), cdt, g)
    assert (x.float().abs() < 2.0 ** -14).all() and (x != 0).any()
    ref = x.cpu()
    assert oracle.rope_partial_inplace(ref, c.cpu(), s.cpu(), 1, [16, 64])[0] == 0
    ra.rope_partial_inplace(x, c, s, 1, [16, 64])
    torch.cuda.synchronize()
    check_bits_equal(x.cpu(), ref, f"subnormal x {xdt}/{cdt}")


@pytest.mark.parametrize("dt", [torch.float32, torch.float16, torch.bfloat16],
                         ids=lambda d: str(d).split(".")[-1])
def test_cache_subnormal_inputs(dt):
    T, nq, nk, H = 33, 3, 2, 128
    g = W.generator(22, DEV)
    q = (W.randn((T, nq * H), torch.float32, g) * SUBNORMAL_SCALE[dt]).to(dt)
    k = (W.randn((T, nk * H), torch.float32, g) * SUBNORMAL_SCALE[dt]).to(dt)
    cache = W.randn((64, 128), dt, g)
    pos = torch.randint(0, 64, (T,), generator=g, device=DEV)
    for neox in (True, False):
        qo, ko = ra.rope_with_cos_sin_cache(pos, q, k, cache, None, H, neox)
        torch.cuda.synchronize()
        rq, rk, _, _ = oracle_cache(pos.cpu(), q.cpu(), k.cpu(), cache.cpu(), None, H, neox)
        check_bits_equal(qo.cpu(), rq, f"subnormal q {dt} neox={neox}")
        check_bits_equal(ko.cpu(), rk, f"subnormal k {dt} neox={neox}")


@pytest.mark.parametrize("cfg", ["inplace_bf16_8x4096x1x576_s512", "inplace_f32_1x16x2x64",
                                 "inplace_half_bf16_8x4096x1x576_s512",
                                 "inplace_heads_bf16_4x2048x32x192_s128_bs1d",
                                 "cache_rope_neox_bf16_t8192", "cache_rope_gptj_f16_t32768_rd64",
                                 "cache_mrope_neox_bf16_t16384",
                                 "cache_mrope_interleaved_neox_bf16_t16384"])
def test_configs_bit_identical_to_oracle(cfg):
    """Beyond the tolerances: the kernels perform the oracle's float32 operations in the
    oracle's order, with one rounding to the storage type, so every output element equals
    the oracle's bit for bit (NaN-free inputs)."""
    case = W.CONFIGS[cfg](DEV)
    if hasattr(case, "x"):
        ref = case.x.cpu()
        assert oracle.rope_partial_inplace(ref, case.cos.cpu(), case.sin.cpu(), case.rotary_mode,
                                           case.partial_slice)[0] == 0
        ra.rope_partial_inplace(case.x, case.cos, case.sin, case.rotary_mode,
                                case.partial_slice)
        torch.cuda.synchronize()
        check_bits_equal(case.x.cpu(), ref, cfg)
    else:
        qo, ko = run_cache_case(case)
        rq, rk, _, _ = oracle_cache(case.positions.cpu(), case.query.cpu(), case.key.cpu(),
                                    case.cache.cpu(), case.mrope_section, case.head_size,
                                    case.is_neox, case.cache_mode)
        check_bits_equal(qo.cpu(), rq, cfg + " q")
        check_bits_equal(ko.cpu(), rk, cfg + " k")


def test_inplace_deterministic_and_stream():
    case = W.inplace_bf16_slice(DEV)
    x1 = case.x.clone()
    x2 = case.x.clone()
    side = torch.cuda.Stream()
    ra.rope_partial_inplace(x1, case.cos, case.sin, 1, case.partial_slice)
    torch.cuda.current_stream().synchronize()
    with torch.cuda.stream(side):
        ra.rope_partial_inplace(x2, case.cos, case.sin, 1, case.partial_slice, stream=side)
    side.synchronize()
    check_bits_equal(x1, x2, "two runs / two streams")


# ------------------------------------------------------------------------------------------
# cache op
# ------------------------------------------------------------------------------------------

def oracle_cache(pos, q, k, cache, msec, H, neox, cache_mode=None):
    qo = torch.empty(q.shape, dtype=q.dtype)
    ko = torch.empty(k.shape, dtype=k.dtype)
    st, q64, k64 = oracle.rope_with_cos_sin_cache(pos, q, k, cache, msec, H, neox, qo, ko,
                                                  twin=True, cache_mode=cache_mode)
    assert st == 0, oracle.last_error()
    return qo, ko, q64, k64


def compare_cache(pos, q_in, k_in, cache, msec, H, neox, q_gpu, k_gpu, what, cache_mode=None):
    """All arguments on the host; q_gpu/k_gpu are host copies of the GPU outputs."""
    rd = cache.shape[1]
    qo, ko, q64, k64 = oracle_cache(pos, q_in, k_in, cache, msec, H, neox, cache_mode)
    cos_t, sin_t = gathered_tables(cache, pos, msec, cache_mode or 0)
    exact = 0
    for name, inp, got, ref, ref64 in (("q", q_in, q_gpu, qo, q64), ("k", k_in, k_gpu, ko, k64)):
        T = inp.shape[0]
        g3, r3, i3 = (got.reshape(T, -1, H), ref.reshape(T, -1, H),
                      inp.contiguous().reshape(T, -1, H))
        check_bits_equal(g3[..., rd:], i3[..., rd:], f"{what} {name} pass-through")
        if got.dtype in HALF:
            exact += check_half(g3[..., :rd], r3[..., :rd], f"{what} {name}")
        else:
            sc = cache_scale(inp.contiguous(), cos_t, sin_t, H, rd, neox).reshape(T, -1, H)
            exact += check_f32(g3[..., :rd], ref64.reshape(T, -1, H)[..., :rd], sc[..., :rd],
                               f"{what} {name}")
    return exact


def run_cache_case(case, **kw):
    if case.cache_mode is None:
        qo, ko = ra.rope_with_cos_sin_cache(case.positions, case.query, case.key, case.cache,
                                            case.mrope_section, case.head_size, case.is_neox,
                                            **kw)
    else:
        qo, ko = ra.rope_with_cos_sin_cache_v2(case.positions, case.query, case.key, case.cache,
                                               case.mrope_section, case.head_size, case.is_neox,
                                               case.cache_mode, **kw)
    torch.cuda.synchronize()
    return qo, ko


def compare_cache_case(case, qo, ko, what=None):
    compare_cache(case.positions.cpu(), case.query.cpu(), case.key.cpu(), case.cache.cpu(),
                  case.mrope_section, case.head_size, case.is_neox, qo.cpu(), ko.cpu(),
                  what or case.name, case.cache_mode)


@pytest.mark.parametrize("cfg", ["cache_rope_neox_bf16_t8192", "cache_rope_gptj_f16_t32768_rd64",
                                 "cache_mrope_neox_bf16_t16384",
                                 "cache_mrope_interleaved_neox_bf16_t16384"])
def test_cache_configs_full(cfg):
    case = W.CONFIGS[cfg](DEV)
    qo, ko = run_cache_case(case)
    compare_cache_case(case, qo, ko)


@pytest.mark.parametrize("mrope", [False, True], ids=["rope", "mrope"])
@pytest.mark.parametrize("neox", [True, False], ids=["neox", "gptj"])
@pytest.mark.parametrize("dt", [torch.float32, torch.float16, torch.bfloat16],
                         ids=lambda d: str(d).split(".")[-1])
def test_cache_long_launch_many_tiles(dt, neox, mrope):
    """Launches of several rounds of workgroups (4000 to 12288 tiles, tapered end included):
    12288 tokens, 8 + 8 heads of 128, q rows padded by 64 elements, rope or mrope [16,24,24]
    positions, every dtype and both styles."""
    T, nq, nk, H = 12288, 8, 8, 128
    rd = 128 if (neox or mrope) else 64
    sec = [16, 24, 24] if mrope else None
    g = W.generator(4100 + int(neox) + 2 * int(mrope), DEV)
    qbig = W.randn((T, nq * H + 64), dt, g)
    q = qbig[:, :nq * H]
    k = W.randn((T, nk * H), dt, g)
    cache = W.randn((4096, rd), dt, g)
    pos = torch.randint(0, 4096, (3, T) if mrope else (T,), generator=g, device=DEV)
    qo, ko = ra.rope_with_cos_sin_cache(pos, q, k, cache, sec, H, neox)
    torch.cuda.synchronize()
    compare_cache(pos.cpu(), q.cpu(), k.cpu(), cache.cpu(), sec, H, neox, qo.cpu(), ko.cpu(),
                  f"long launch {dt} neox={neox} mrope={mrope}")


@pytest.mark.parametrize("neox", [True, False], ids=["neox", "gptj"])
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=lambda d: str(d).split(".")[-1])
@pytest.mark.parametrize("rd,extra", [(16384, 0), (16384, 64), ("past", 0), (24576, 32)],
                         ids=["lds_limit", "lds_limit_tail", "direct", "direct_tail"])
def test_cache_rotary_dim_at_and_past_the_lds_tile(rd, extra, dt, neox):
    """[RSCC §约束说明] bounds rotaryDim only by headSize and 64-byte alignment.  16384 is the
    longest cos|sin row the tile kernel stages in LDS (64 KiB for float32); one 64-byte step
    past it, and at 24576, each item reads its cos/sin straight from the cache row.  Heads with
    and without a pass-through tail, every token against the oracle."""
    align = 64 // torch.tensor([], dtype=dt).element_size()
    rd = 16384 + align if rd == "past" else rd
    H = rd + extra
    case = W.cache_case("longrd", 9, 2, 1, H, rd, dt, neox, 40, seed=rd + extra, device=DEV)
    qo, ko = run_cache_case(case)
    compare_cache_case(case, qo, ko, f"rd {rd} H {H} {dt} neox={neox}")


def test_cache_long_rotary_dim_unaligned_rows():
    """The direct cos/sin reads on rows that are not 16-byte aligned (cache and query one
    element off): element-wise loads of the cache row and of q."""
    rd, H, T = 16416, 16448, 5
    g = W.generator(31, DEV)
    cbuf = W.cos_sin_cache(12, rd, torch.bfloat16).to(DEV).reshape(-1)
    cache = torch.cat([cbuf[:1], cbuf]).narrow(0, 1, cbuf.numel()).view(12, rd)
    qbuf = W.randn((T * 2 * H + 1,), torch.bfloat16, g)
    q = qbuf.narrow(0, 1, T * 2 * H).view(T, 2 * H)
    k = W.randn((T, H), torch.bfloat16, g)
    pos = torch.tensor([11, 0, 5, 5, 3], device=DEV)
    assert cache.data_ptr() % 16 and q.data_ptr() % 16
    for neox in (True, False):
        qo, ko = ra.rope_with_cos_sin_cache(pos, q, k, cache, None, H, neox)
        torch.cuda.synchronize()
        compare_cache(pos.cpu(), q.cpu(), k.cpu(), cache.cpu(), None, H, neox, qo.cpu(),
                      ko.cpu(), f"unaligned rd {rd} neox={neox}")


HEADS = [(torch.bfloat16, 32, 32), (torch.bfloat16, 64, 32), (torch.bfloat16, 96, 96),
         (torch.bfloat16, 128, 64), (torch.bfloat16, 128, 96), (torch.float16, 64, 64),
         (torch.float16, 96, 32), (torch.float16, 128, 128), (torch.float32, 16, 16),
         (torch.float32, 48, 32), (torch.float32, 128, 64), (torch.float32, 96, 96)]


@pytest.mark.parametrize("neox", [True, False], ids=["neox", "gptj"])
@pytest.mark.parametrize("dt,H,rd", HEADS, ids=lambda v: str(v).split(".")[-1])
@pytest.mark.parametrize("T,nq,nk", [(1, 1, 1), (3, 2, 1), (127, 5, 3), (4097, 4, 2)])
def test_cache_sweep(dt, H, rd, neox, T, nq, nk):
    case = W.cache_case("sweep", T, nq, nk, H, rd, dt, neox, 500, seed=T + H + rd, device=DEV)
    qo, ko = run_cache_case(case)
    compare_cache(case.positions.cpu(), case.query.cpu(), case.key.cpu(), case.cache.cpu(),
                  None, H, neox, qo.cpu(), ko.cpu(), f"T{T} {dt} H{H} rd{rd} neox={neox}")


@pytest.mark.parametrize("neox", [True, False], ids=["neox", "gptj"])
@pytest.mark.parametrize("sec", [[16, 24, 24], [8, 12, 12], [24, 20, 20], [11, 11, 10],
                                 [16, 16, 16, 16]])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16, torch.float32])
def test_cache_mrope(sec, neox, dt):
    rd = 2 * sum(sec)
    H = 128 if rd <= 128 else 256
    if dt == torch.float32 and rd % 16:
        pytest.skip("rotaryDim must be a 64-byte multiple")
    pos = W.mrope_positions(300, 2, 16, 16, m=len(sec))
    T = pos.shape[1]
    case = W.cache_case("mrope", T, 6, 2, H, rd, dt, neox, 400, seed=rd, mrope_section=sec,
                        positions=pos, device=DEV)
    qo, ko = run_cache_case(case)
    compare_cache(case.positions.cpu(), case.query.cpu(), case.key.cpu(), case.cache.cpu(),
                  sec, H, neox, qo.cpu(), ko.cpu(), f"mrope {sec} {dt} neox={neox}")


@pytest.mark.parametrize("neox", [True, False], ids=["neox", "gptj"])
@pytest.mark.parametrize("sec", [[16, 24, 24], [8, 12, 12], [24, 20, 20], [11, 11, 10]])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("cache_mode", [0, 1], ids=["sectioned", "interleaved"])
def test_cache_mrope_v2(sec, neox, dt, cache_mode):
    """The V2 entry point: both stitchings of every 3-section list, on text + image
    positions whose three rows differ (so each element's source row shows in the result)."""
    rd = 2 * sum(sec)
    H = 128 if rd <= 128 else 256
    if dt == torch.float32 and rd % 16:
        pytest.skip("rotaryDim must be a 64-byte multiple")
    pos = W.mrope_positions(200, 3, 12, 10, m=3)
    T = pos.shape[1]
    case = W.cache_case("mrope_v2", T, 5, 3, H, rd, dt, neox, 400, seed=rd + 7,
                        mrope_section=sec, positions=pos, device=DEV, cache_mode=cache_mode)
    qo, ko = run_cache_case(case)
    compare_cache_case(case, qo, ko, f"mrope v2 {sec} mode {cache_mode} {dt} neox={neox}")


@pytest.mark.parametrize("sec,rd", [([16, 16, 16, 16], 128), (None, 64)])
def test_cache_v2_mode0_equals_v1(sec, rd):
    """cacheMode 0 is the V1 call: bit-identical outputs (4-section mrope, rope mode)."""
    m = len(sec) if sec else 0
    pos = W.mrope_positions(100, 2, 8, 8, m=m) if m else None
    case = W.cache_case("v2_vs_v1", 228, 4, 2, 128, rd, torch.bfloat16, True, 300, seed=21,
                        mrope_section=sec, positions=pos, device=DEV)
    q1, k1 = run_cache_case(case)
    q2, k2 = ra.rope_with_cos_sin_cache_v2(case.positions, case.query, case.key, case.cache, sec,
                                           128, True, 0)
    torch.cuda.synchronize()
    check_bits_equal(q1.cpu(), q2.cpu(), "q v1 vs v2 mode 0")
    check_bits_equal(k1.cpu(), k2.cpu(), "k v1 vs v2 mode 0")
    if not m:  # rope mode: cacheMode 1 changes nothing
        q3, k3 = ra.rope_with_cos_sin_cache_v2(case.positions, case.query, case.key, case.cache,
                                               None, 128, True, 1)
        torch.cuda.synchronize()
        check_bits_equal(q1.cpu(), q3.cpu(), "q rope mode, cacheMode 1")
        check_bits_equal(k1.cpu(), k3.cpu(), "k rope mode, cacheMode 1")


def test_cache_v2_interleaved_misaligned_cache_rows():
    """Interleaved stitching from a cache whose rows are not 16-byte aligned (element
    staging path)."""
    sec, rd, H = [8, 12, 12], 64, 128
    g = W.generator(31, DEV)
    full = torch.zeros(300, rd + 3, dtype=torch.bfloat16, device=DEV)
    full[:, 1:1 + rd] = W.cos_sin_cache(300, rd, torch.bfloat16).to(DEV)
    cache = full[:, 1:1 + rd]                # row stride rd + 3 elements, 2-byte offset
    pos = W.mrope_positions(60, 2, 6, 5, m=3).to(DEV)
    T = pos.shape[1]
    q = W.randn((T, 3 * H), torch.bfloat16, g)
    k = W.randn((T, H), torch.bfloat16, g)
    for neox in (True, False):
        qo, ko = ra.rope_with_cos_sin_cache_v2(pos, q, k, cache, sec, H, neox, 1)
        torch.cuda.synchronize()
        compare_cache(pos.cpu(), q.cpu(), k.cpu(), cache.cpu(), sec, H, neox, qo.cpu(), ko.cpu(),
                      f"interleaved misaligned cache neox={neox}", 1)


def test_cache_strided_inputs_and_positions():
    """Row strides larger than the row (qStride/kStride), a row-strided cache, strided
    positions; outputs contiguous."""
    T, H, rd = 257, 128, 64
    g = W.generator(5, DEV)
    qbig = W.randn((T, 3 * H + 64), torch.bfloat16, g)
    kbig = W.randn((T, 2 * H + 32), torch.bfloat16, g)
    q = qbig[:, 32:32 + 3 * H]
    k = kbig[:, :H]
    cbig = W.cos_sin_cache(100, 128, torch.bfloat16).to(DEV)
    cache = cbig[:, :rd]
    pos_big = torch.randint(0, 100, (2 * T,), generator=g, device=DEV)
    pos = pos_big[::2]
    for neox in (True, False):
        qo, ko = ra.rope_with_cos_sin_cache(pos, q, k, cache, None, H, neox)
        torch.cuda.synchronize()
        compare_cache(pos.cpu(), q.cpu(), k.cpu(), cache.cpu(), None, H, neox, qo.cpu(), ko.cpu(),
                      f"strided neox={neox}")


def test_cache_misaligned_rows_use_element_path():
    T, H = 33, 64
    g = W.generator(6, DEV)
    buf = W.randn((T * (2 * H + 1) + 8,), torch.float16, g)
    q = buf[1:1 + T * (2 * H + 1)].view(T, 2 * H + 1)[:, :2 * H]   # row stride 129 elements
    k = W.randn((T, H), torch.float16, g)
    cache = W.cos_sin_cache(64, 64, torch.float16).to(DEV)
    pos = torch.randint(0, 64, (T,), generator=g, device=DEV)
    for neox in (True, False):
        qo, ko = ra.rope_with_cos_sin_cache(pos, q, k, cache, None, H, neox)
        torch.cuda.synchronize()
        compare_cache(pos.cpu(), q.cpu(), k.cpu(), cache.cpu(), None, H, neox, qo.cpu(),
                      ko.cpu(), f"misaligned neox={neox}")


def test_cache_exact_alias_in_place():
    case = W.cache_case("alias", 1000, 8, 2, 128, 64, torch.bfloat16, True, 2048, seed=8,
                        device=DEV)
    q_in, k_in = case.query.cpu(), case.key.cpu()
    q, k = case.query, case.key
    ra.rope_with_cos_sin_cache(case.positions, q, k, case.cache, None, 128, True,
                               query_out=q, key_out=k)
    torch.cuda.synchronize()
    compare_cache(case.positions.cpu(), q_in, k_in, case.cache.cpu(), None, 128, True, q.cpu(),
                  k.cpu(), "aliased")


@pytest.mark.parametrize("dt", [torch.float32, torch.float16, torch.bfloat16])
def test_cache_specials(dt):
    case = W.cache_case("specials", 64, 3, 1, 64, 32, dt, True, 128, seed=9, device=DEV)
    q = case.query.view(-1)
    q[5] = float("nan")
    q[64 * 3 + 40] = float("inf")      # a pass-through element
    q[64 * 7 + 17] = float("-inf")
    case.key.view(-1)[3] = float("nan")
    case.cache[case.positions[2], 4] = float("inf")
    qo, ko = run_cache_case(case)
    compare_cache(case.positions.cpu(), case.query.cpu(), case.key.cpu(), case.cache.cpu(),
                  None, 64, True, qo.cpu(), ko.cpu(), f"specials {dt}")


def test_cache_positions_out_of_range_are_clamped():
    """Outside the contract ([RSCC §约束说明]: positions < maxSeqLen).  The library documents a
    clamp into [0, maxSeqLen); the call must complete and match the clamped positions."""
    case = W.cache_case("oob", 50, 2, 1, 64, 64, torch.bfloat16, True, 32, seed=10, device=DEV)
    pos = case.positions.clone()
    pos[3] = 1 << 40
    pos[7] = -5
    qo, ko = ra.rope_with_cos_sin_cache(pos, case.query, case.key, case.cache, None, 64, True)
    torch.cuda.synchronize()
    clamped = pos.clamp(0, 31).cpu()
    compare_cache(clamped, case.query.cpu(), case.key.cpu(), case.cache.cpu(), None, 64, True,
                  qo.cpu(), ko.cpu(), "clamped")


@pytest.mark.parametrize(
    "dt,H,T,nq,nk",
    [(torch.float16, 128, 4096, 5, 3),    # rotaryDim 64 of 128: a pass-through half
     (torch.bfloat16, 64, 3000, 7, 5),    # full rotary
     (torch.float32, 96, 2500, 3, 2),     # rotaryDim 32 of 96 floats, two wavefronts a token
     (torch.float16, 192, 2100, 1, 1)],   # 2 heads of 24 lanes: idle lanes in every wavefront
    ids=["f16_rd64_of_128", "bf16_full", "f32_rd32_of_96", "f16_idle_lanes"])
def test_cache_gptj_scalar_cos_sin_row(dt, H, T, nq, nk):
    """GPT-J rope mode with a 128-byte cos|sin row in launches of at least eight wavefronts per
    compute unit: each wavefront reads its token's row with scalar loads and every lane selects
    its own chunk ([RSCC §rotate_interleaved（GPT-J style）旋转模式]).  Outputs start as all-ones
    bit patterns and must all be overwritten; positions include out-of-range values (clamped,
    so compared with the oracle at the clamped positions); every token is compared."""
    rd = 128 // torch.empty(0, dtype=dt).element_size()
    case = W.cache_case("srow", T, nq, nk, H, rd, dt, False, 900, seed=7000 + H, device=DEV)
    pos = case.positions.clone()
    pos[5] = 1 << 40
    pos[T - 1] = -3
    qo, ko = torch.empty_like(case.query), torch.empty_like(case.key)
    ibits = torch.int32 if dt == torch.float32 else torch.int16
    for t in (qo, ko):
        t.view(ibits).fill_(-1)
    ra.rope_with_cos_sin_cache(pos, case.query, case.key, case.cache, None, H, False,
                               query_out=qo, key_out=ko)
    torch.cuda.synchronize()
    for name, t in (("q", qo), ("k", ko)):
        left = int((t.view(ibits) == -1).sum())
        assert left == 0, f"{left} {name} output elements never written"
    compare_cache(pos.clamp(0, 899).cpu(), case.query.cpu(), case.key.cpu(), case.cache.cpu(),
                  None, H, False, qo.cpu(), ko.cpu(), f"scalar row {dt} H{H}")


@pytest.mark.parametrize("dt,H,rd,T,nq,nk,sec", [
    (torch.bfloat16, 128, 96, 700, 5, 3, None), (torch.float16, 192, 192, 300, 3, 2, None),
    (torch.float32, 96, 96, 500, 4, 4, None), (torch.bfloat16, 64, 64, 2500, 6, 2, None),
    (torch.float16, 160, 32, 400, 3, 1, None), (torch.bfloat16, 64, 64, 600, 3, 2, [11, 11, 10]),
    (torch.bfloat16, 128, 64, 700, 5, 3, None), (torch.float32, 128, 32, 500, 3, 3, None),
    (torch.bfloat16, 128, 64, 600, 3, 2, [11, 11, 10])],
    ids=["bf16_H128_rd96", "f16_H192_rd192", "f32_H96_rd96", "bf16_H64_rd64_T2500",
         "f16_H160_rd32", "bf16_mrope_11_11_10", "xch_bf16_H128_rd64", "xch_f32_H128_rd32",
         "xch_bf16_mrope_11_11_10"])
def test_cache_neox_one_vector_units_shared_gather(dt, H, rd, T, nq, nk, sec):
    """NeoX shapes whose rotated half is not a whole number of 128-byte lines: one-vector units
    (the pair partner two or more lanes away) and, with rotaryDim at most half the head, the
    exchange layout; in both the pair's cos and sin halves are gathered one by each lane and
    swapped
    ([RSCC §rotate_half（GPT-NeoX style）旋转模式]).  Outputs start as all-ones bit patterns and
    must all be overwritten; positions include out-of-range values (clamped, so compared with
    the oracle at the clamped positions)."""
    m = len(sec) if sec else 0
    g = W.generator(7100 + H + rd, DEV)
    pos = torch.randint(0, 800, (m, T) if m else (T,), generator=g, device=DEV)
    case = W.cache_case("lin", T, nq, nk, H, rd, dt, True, 800, seed=7200 + H, device=DEV,
                        mrope_section=sec, positions=pos)
    pos = case.positions.clone()
    pos.view(-1)[3] = 1 << 40
    pos.view(-1)[-1] = -5
    qo, ko = torch.empty_like(case.query), torch.empty_like(case.key)
    ibits = torch.int32 if dt == torch.float32 else torch.int16
    for t in (qo, ko):
        t.view(ibits).fill_(-1)
    ra.rope_with_cos_sin_cache(pos, case.query, case.key, case.cache, sec, H, True,
                               query_out=qo, key_out=ko)
    torch.cuda.synchronize()
    for name, t in (("q", qo), ("k", ko)):
        left = int((t.view(ibits) == -1).sum())
        assert left == 0, f"{left} {name} output elements never written"
    compare_cache(pos.clamp(0, 799).cpu(), case.query.cpu(), case.key.cpu(), case.cache.cpu(),
                  sec, H, True, qo.cpu(), ko.cpu(), f"one-vector NeoX {dt} H{H} rd{rd} {sec}")


def test_cache_max_tokens_and_large_rotary_dim():
    case = W.cache_case("maxT", 131073, 1, 1, 32, 32, torch.bfloat16, False, 1000, seed=11,
                        device=DEV)
    qo, ko = run_cache_case(case)
    compare_cache(case.positions.cpu(), case.query.cpu(), case.key.cpu(), case.cache.cpu(),
                  None, 32, False, qo.cpu(), ko.cpu(), "T=131073")
    big = W.cache_case("bigrd", 40, 2, 1, 4096, 2048, torch.float16, True, 64, seed=12,
                       device=DEV)
    qo, ko = run_cache_case(big)
    compare_cache(big.positions.cpu(), big.query.cpu(), big.key.cpu(), big.cache.cpu(), None,
                  4096, True, qo.cpu(), ko.cpu(), "rd=2048")


@pytest.mark.parametrize("H,neox", [(1024, True), (1056, True), (512, False), (544, False)],
                         ids=["neox64units", "neox66units", "gptj64units", "gptj68units"])
def test_cache_units_per_head_either_side_of_64(H, neox):
    """bf16 heads of exactly 64 units (one row of lanes per head on the wavefront path) and
    just above (the tile path): 5 + 3 heads, half of each head rotated, 300 tokens."""
    rd = H // 2 if (H // 2) % 32 == 0 else H - 32
    case = W.cache_case("units", 300, 5, 3, H, rd, torch.bfloat16, neox, 700, seed=H,
                        device=DEV)
    qo, ko = run_cache_case(case)
    compare_cache_case(case, qo, ko, f"H{H} rd{rd} neox={neox}")


@pytest.mark.parametrize(
    "dt,H,rd,neox,sec,cache_mode",
    [(torch.float16, 128, 64, False, None, None),       # GPT-J one-vector units
     (torch.bfloat16, 128, 128, True, None, None),      # NeoX pair units
     (torch.bfloat16, 128, 64, True, None, None),       # NeoX exchange layout (rd <= H/2)
     (torch.bfloat16, 128, 96, True, None, None),       # NeoX one-vector units
     (torch.float32, 64, 64, True, None, None),
     (torch.bfloat16, 128, 128, True, [16, 24, 24], 0),
     (torch.bfloat16, 128, 128, True, [16, 16, 16, 16], 0),
     (torch.bfloat16, 128, 128, True, [24, 20, 20], 1),  # interleaved stitching
     (torch.bfloat16, 1056, 1024, True, None, None)],   # 66 units a head: the tile form
    ids=["gptj_f16", "neox_pairs", "neox_exchange", "neox_one_vector", "neox_f32", "mrope3",
         "mrope4", "mrope_interleaved", "tile_form"])
def test_cache_every_output_element_written(dt, H, rd, neox, sec, cache_mode):
    """The outputs start as all-ones bit patterns (a NaN in every dtype, which finite inputs
    never produce), so a store that never lands cannot pass as a correct value left over in
    reused memory: every element must be overwritten, and all of them must match the oracle.
    [RSCC §设计动机]: every element of query_out/key_out is either rotated or passed through."""
    T, nq, nk = 333, 5, 3
    pos = None
    if sec is not None:
        pos = W.mrope_positions(T - 2 * 8 * 8, 2, 8, 8, len(sec))
    case = W.cache_case("written", T, nq, nk, H, rd, dt, neox, 700, seed=4242 + H + rd,
                        mrope_section=sec, positions=pos, device=DEV, cache_mode=cache_mode)
    qo, ko = torch.empty_like(case.query), torch.empty_like(case.key)
    ibits = torch.int32 if dt == torch.float32 else torch.int16
    for t in (qo, ko):
        t.view(ibits).fill_(-1)
    run_cache_case(case, query_out=qo, key_out=ko)
    for name, t in (("q", qo), ("k", ko)):
        left = int((t.view(ibits) == -1).sum())
        assert left == 0, f"{left} {name} output elements never written"
    compare_cache_case(case, qo, ko, f"every element H{H} rd{rd} neox={neox} sec={sec}")


@pytest.mark.parametrize("neox", [True, False], ids=["neox", "gptj"])
@pytest.mark.parametrize("sec,cache_mode", [(None, None), ([16, 24, 24], 0), ([24, 20, 20], 1),
                                            ([11, 11, 10], 0)],
                         ids=["rope", "mrope", "interleaved", "split_sections"])
def test_cache_idle_lanes_with_pass_through(sec, cache_mode, neox):
    """Heads whose units do not divide a row of 64 lanes (bf16 H = 192: 12 NeoX units, 5 heads
    per row and 4 idle lanes; 24 GPT-J units, 2 heads per row and 16 idle lanes), with a
    pass-through part (rd 128 of 192; 64 for [11,11,10]), 7 + 3 heads, in rope mode and every
    stitching form."""
    H, rd = 192, 2 * sum(sec) if sec else 128
    m = len(sec) if sec else 0
    pos = W.mrope_positions(150, 2, 9, 7, m=m) if m else None
    case = W.cache_case("idle", 276 if not m else pos.shape[1], 7, 3, H, rd, torch.bfloat16,
                        neox, 400, seed=77, mrope_section=sec, positions=pos, device=DEV,
                        cache_mode=cache_mode)
    qo, ko = run_cache_case(case)
    compare_cache_case(case, qo, ko, f"idle lanes {sec} mode {cache_mode} neox={neox}")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16, torch.float32],
                         ids=lambda d: str(d).split(".")[-1])
@pytest.mark.parametrize("H,rd,sec,cache_mode", [(128, 32, None, None), (128, 64, None, None),
                                                  (256, 128, None, None),
                                                  (128, 64, [11, 11, 10], 1),
                                                  (256, 128, [16, 24, 24], 0)],
                         ids=["rd_quarter", "rd_half", "rd_half_H256", "mrope_interleaved",
                              "mrope_sections"])
def test_cache_neox_partial_lane_exchange(H, rd, sec, cache_mode, dt):
    """NeoX with rotaryDim <= headSize/2 (the wavefront kernel's lane-exchange layout: a
    rotated vector's pair partner is read from another lane of the same head): 28 + 4 heads,
    777 tokens or the mrope text + image positions, every dtype."""
    es = torch.empty(0, dtype=dt).element_size()
    if rd * es % 64:
        pytest.skip("rotaryDim must be a 64-byte multiple")
    pos = W.mrope_positions(300, 2, 12, 10, m=3) if sec else None
    T = pos.shape[1] if sec else 777
    case = W.cache_case("xch", T, 28, 4, H, rd, dt, True, 900, seed=H + rd + es,
                        mrope_section=sec, positions=pos, device=DEV, cache_mode=cache_mode)
    qo, ko = run_cache_case(case)
    compare_cache_case(case, qo, ko, f"NeoX H{H} rd{rd} {sec} mode {cache_mode} {dt}")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16, torch.float32],
                         ids=lambda d: str(d).split(".")[-1])
@pytest.mark.parametrize("H,rd,sec,cache_mode", [(128, 96, None, None), (64, 64, None, None),
                                                  (96, 96, None, None), (64, 32, None, None),
                                                  (64, 64, [11, 11, 10], 1),
                                                  (64, 64, [8, 12, 12], 0)],
                         ids=["rd96_H128", "H64", "H96", "rd32_H64", "mrope_interleaved",
                              "mrope_split_sections"])
def test_cache_neox_one_vector_units(H, rd, sec, cache_mode, dt):
    """NeoX shapes whose pair units would leave each access part of every line (half of the
    rotated part not a whole number of 128-byte lines, and no whole-line exchange layout):
    the wavefront kernel then gives a unit one vector and completes each pair from another
    lane.  28 + 4 heads, 777 tokens or the mrope text + image positions, every dtype."""
    es = torch.empty(0, dtype=dt).element_size()
    if rd * es % 64 or H * es % 64:
        pytest.skip("headSize and rotaryDim must be 64-byte multiples")
    pos = W.mrope_positions(300, 2, 12, 10, m=3) if sec else None
    T = pos.shape[1] if sec else 777
    case = W.cache_case("lin", T, 28, 4, H, rd, dt, True, 900, seed=H + 3 * rd + es,
                        mrope_section=sec, positions=pos, device=DEV, cache_mode=cache_mode)
    qo, ko = run_cache_case(case)
    compare_cache_case(case, qo, ko, f"NeoX H{H} rd{rd} {sec} mode {cache_mode} {dt}")


def test_cache_more_waves_than_one_grid():
    """4.5M tokens of one q and one k head (bf16, H = rd = 32, GPT-J): one wavefront per
    token, more wavefronts than the largest grid holds, so the kernel's grid-stride loop runs.
    Every output's rotation is checked on the GPU against the oracle's at seeded sample tokens,
    the first 2048 and the last 2048 tokens (the last ones come from the loop's later
    trips)."""
    T, H = 4_500_000, 32
    case = W.cache_case("grid", T, 1, 1, H, H, torch.bfloat16, False, 5000, seed=4500,
                        device=DEV)
    qo, ko = run_cache_case(case)
    g = torch.Generator().manual_seed(45)
    idx = torch.cat([torch.arange(2048), torch.randperm(T, generator=g)[:4096],
                     torch.arange(T - 2048, T)]).unique().sort().values
    gi = idx.to(DEV)
    compare_cache(case.positions[gi].cpu(), case.query[gi].cpu(), case.key[gi].cpu(),
                  case.cache.cpu(), None, H, False, qo[gi].cpu(), ko[gi].cpu(), case.name)


def test_cache_positions_rewritten_between_calls():
    """The wavefront kernel reads positions through the scalar cache.  Positions rewritten in
    place on the GPU between two launches (by a torch kernel on the same stream) must be the
    ones the second launch uses: both launches are checked against the oracle, for rope and
    mrope positions."""
    for sec in (None, [16, 24, 24]):
        m = 3 if sec else 0
        pos = W.mrope_positions(64, 1, 8, 8, m=3) if sec else None
        case = W.cache_case("rewrite", 128 if not sec else pos.shape[1], 6, 2, 128, 128,
                            torch.bfloat16, True, 1000, seed=77, mrope_section=sec,
                            positions=pos, device=DEV)
        first = [t.cpu() for t in run_cache_case(case)]
        before = case.positions.cpu()
        case.positions.mul_(3).add_(1).remainder_(1000)   # in place, same stream
        second = [t.cpu() for t in run_cache_case(case)]
        after = case.positions.cpu()
        assert not torch.equal(before, after)
        compare_cache(before, case.query.cpu(), case.key.cpu(), case.cache.cpu(), sec, 128,
                      True, first[0], first[1], f"positions before rewrite, m={m}")
        compare_cache(after, case.query.cpu(), case.key.cpu(), case.cache.cpu(), sec, 128,
                      True, second[0], second[1], f"positions after rewrite, m={m}")


def test_cache_query_beyond_2e31_elements():
    """A query of more than 2^31 elements (2^21 + 7 tokens of 8 heads of 128, bf16, 4.3 GB):
    row offsets past 32 bits on the wavefront kernel.  The rotated outputs of the last 1024
    tokens and of 3072 seeded sample tokens are compared with the oracle."""
    T, nq, nk, H = (1 << 21) + 7, 8, 1, 128
    assert T * nq * H > (1 << 31)
    g = W.generator(2031, DEV)
    q = W.randn((T, nq * H), torch.bfloat16, g)
    k = W.randn((T, nk * H), torch.bfloat16, g)
    cache = W.cos_sin_cache(4096, H, torch.bfloat16).to(DEV)
    pos = torch.randint(0, 4096, (T,), generator=g, device=DEV)
    qo, ko = ra.rope_with_cos_sin_cache(pos, q, k, cache, None, H, True)
    torch.cuda.synchronize()
    idx = torch.cat([torch.randperm(T - 1024, generator=torch.Generator().manual_seed(31))[:3072],
                     torch.arange(T - 1024, T)]).sort().values
    gi = idx.to(DEV)
    compare_cache(pos[gi].cpu(), q[gi].cpu(), k[gi].cpu(), cache.cpu(), None, H, True,
                  qo[gi].cpu(), ko[gi].cpu(), "query beyond 2^31 elements")
    del q, k, qo, ko
    torch.cuda.empty_cache()


@pytest.mark.parametrize("heads", [(1 << 23) - 1, 1 << 23], ids=["row_below_2e31_bytes",
                                                              "row_of_2e31_bytes"])
def test_cache_output_row_at_the_buffer_range_limit(heads):
    """One token with a query row of 2^31 - 256 bytes (bf16 heads of 128: the wavefront kernel,
    whose stores address a token's output row as one buffer range of 32-bit offsets, up to the
    last head) and of exactly 2^31 bytes (the plan sends it to the tile form).  The output starts
    as all-ones bit patterns and must be overwritten everywhere; the first and the last 64 heads
    are compared with the oracle (heads are independent, so a slice of them is a valid call)."""
    T, H, nk = 1, 128, 3
    g = W.generator(2023, DEV)
    q = W.randn((T, heads * H), torch.bfloat16, g)
    k = W.randn((T, nk * H), torch.bfloat16, g)
    cache = W.cos_sin_cache(512, H, torch.bfloat16).to(DEV)
    pos = torch.tensor([333], dtype=torch.int64, device=DEV)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    for t in (qo, ko):
        t.view(torch.int16).fill_(-1)
    ra.rope_with_cos_sin_cache(pos, q, k, cache, None, H, True, query_out=qo, key_out=ko)
    torch.cuda.synchronize()
    for name, t in (("q", qo), ("k", ko)):
        left = int((t.view(torch.int16) == -1).sum())
        assert left == 0, f"{left} {name} output elements never written"
    for part in (slice(0, 64 * H), slice((heads - 64) * H, heads * H)):
        compare_cache(pos.cpu(), q[:, part].cpu(), k.cpu(), cache.cpu(), None, H, True,
                      qo[:, part].cpu(), ko.cpu(), f"{heads} heads, {part}")
    del q, qo
    torch.cuda.empty_cache()


def test_cache_deterministic():
    case = W.cache_mrope(DEV)
    a = run_cache_case(case)
    b = run_cache_case(case)
    check_bits_equal(a[0], b[0], "q twice")
    check_bits_equal(a[1], b[1], "k twice")


def test_binding_errors_touch_nothing():
    case = W.cache_case("err", 16, 2, 1, 64, 32, torch.bfloat16, True, 64, seed=13, device=DEV)
    qo = torch.zeros_like(case.query)
    ko = torch.zeros_like(case.key)
    with pytest.raises(ra.RopeError) as e:
        ra.rope_with_cos_sin_cache(case.positions, case.query, case.key, case.cache, [16, 24, 24],
                                   64, True, query_out=qo, key_out=ko)
    assert e.value.code == ra.ROPE_ERR_PARAM_INVALID
    torch.cuda.synchronize()
    assert not qo.any() and not ko.any()


# ------------------------------------------------------------------------------------------
# backward of the in-place op ([IPRM §Python 接口与自动微分]; transpose of the pair map)
# ------------------------------------------------------------------------------------------

def check_backward(g_before, g_after_gpu, cos, sin, sl, what, mode=1):
    ref = g_before.clone()
    st, g64 = oracle.rope_partial_inplace_backward(ref, cos.cpu(), sin.cpu(), mode, sl,
                                                   twin=True)
    assert st == 0, oracle.last_error()
    D = g_before.shape[-1]
    start, end = (0, D) if sl is None else sl
    got = g_after_gpu.cpu()
    check_bits_equal(got[..., :start], g_before[..., :start], what + " [0,start)")
    check_bits_equal(got[..., end:], g_before[..., end:], what + " [end,D)")
    if g_before.dtype in HALF:
        return check_half(got[..., start:end], ref[..., start:end], what)
    scale = inplace_scale(g_before, cos.cpu(), sin.cpu(), start, end, mode, backward=True)
    return check_f32(got[..., start:end], g64[..., start:end], scale, what)


@pytest.mark.parametrize("cfg", ["inplace_f32_1x16x2x64", "inplace_bf16_8x4096x1x576_s512"])
def test_backward_configs_full(cfg):
    case = W.CONFIGS[cfg](DEV)
    g = case.x  # the same seeded N(0,1) tensor serves as the incoming gradient
    before = g.cpu()
    ra.rope_partial_inplace_backward(g, case.cos, case.sin, 1, case.partial_slice)
    torch.cuda.synchronize()
    check_backward(before, g, case.cos, case.sin, case.partial_slice, "backward " + case.name)


@pytest.mark.parametrize("xdt,cdt", DTYPE_PAIRS, ids=lambda d: str(d).split(".")[-1])
@pytest.mark.parametrize("layout", ["BSND", "BS1D", "B11D", "111D"])
@pytest.mark.parametrize("shape,sl", [((3, 37, 5, 96), [16, 80]), ((1, 300, 2, 40), [1, 37]),
                                      ((2, 33, 8, 64), [0, 64]), ((3, 17, 12, 96), [32, 96])])
def test_backward_sweep(xdt, cdt, layout, shape, sl):
    B, S, N, D = shape
    L = sl[1] - sl[0]
    cshape = LAYOUTS[layout](B, S, N) + (L,)
    case = W.inplace_case("bwd", B, S, N, D, xdt, cdt, sl, cos_shape=cshape, seed=S + 5,
                          table="randn", device=DEV)
    before = case.x.cpu()
    ra.rope_partial_inplace_backward(case.x, case.cos, case.sin, 1, sl)
    torch.cuda.synchronize()
    check_backward(before, case.x, case.cos, case.sin, sl, f"backward {layout} {shape} {xdt}/{cdt}")


def test_autograd_wrapper_gradient():
    """InplacePartialRotaryMul (forward kernel, mark_dirty, backward kernel) gives the same
    gradient as the oracle's backward applied to the incoming gradient."""
    B, S, N, D, sl = 2, 32, 8, 128, [0, 64]
    g = W.generator(31, DEV)
    x = W.randn((B, S, N, D), torch.float32, g).requires_grad_(True)
    c = W.randn((B, S, 1, 64), torch.float32, g)
    s = W.randn((B, S, 1, 64), torch.float32, g)
    y = x * 1.0
    y = ra.InplacePartialRotaryMul.apply(y, c, s, sl)
    w = W.randn((B, S, N, D), torch.float32, g)
    (y * w).sum().backward()
    torch.cuda.synchronize()
    check_backward(w.cpu(), x.grad, c, s, sl, "autograd")


@pytest.mark.parametrize("mode", ["interleave", "half"])
def test_pages_python_interface(mode):
    """inplace_partial_rotary_mul / _backward, the Python interface of [IPRM §Python 接口与自动
    微分]: returns None and rotates x in place (as rope_partial_inplace does) without autograd;
    with x requiring grad it records the op, and the gradient of x equals the backward op
    applied to the incoming gradient; r1, r2 get no gradient."""
    code = {"interleave": 1, "half": 0}[mode]
    B, S, N, D, sl = 2, 32, 8, 128, [0, 64]
    g = W.generator(41 + code, DEV)
    x = W.randn((B, S, N, D), torch.bfloat16, g)
    r1 = W.randn((B, S, 1, 64), torch.bfloat16, g)
    r2 = W.randn((B, S, 1, 64), torch.bfloat16, g)
    a, b = x.clone(), x.clone()
    assert ra.inplace_partial_rotary_mul(a, r1, r2, rotary_mode=mode, partial_slice=sl) is None
    ra.rope_partial_inplace(b, r1, r2, code, sl)
    torch.cuda.synchronize()
    check_bits_equal(a, b, f"{mode}: pages' interface vs entry point")
    # autograd
    xg = x.float().requires_grad_(True)
    c32, s32 = r1.float().requires_grad_(True), r2.float().requires_grad_(True)
    y = xg * 1.0
    assert ra.inplace_partial_rotary_mul(y, c32, s32, rotary_mode=mode, partial_slice=sl) is None
    w = W.randn((B, S, N, D), torch.float32, g)
    (y * w).sum().backward()
    ref = w.clone()
    assert ra.inplace_partial_rotary_mul_backward(ref, c32.detach(), s32.detach(),
                                                  rotary_mode=mode, partial_slice=sl) is None
    torch.cuda.synchronize()
    check_bits_equal(xg.grad, ref, f"{mode}: autograd gradient vs the backward op")
    assert c32.grad is None and s32.grad is None
    check_backward(w.cpu(), xg.grad, c32.detach(), s32.detach(), sl, f"{mode} autograd",
                   mode=code)


# ------------------------------------------------------------------------------------------
# half mode, rotary_mode 0 (x1, x2 the two halves of the slice)
# ------------------------------------------------------------------------------------------

HALF_SHAPES = [((3, 37, 5, 96), [16, 80]),    # ragged rows, inner slice, lane pairs
               ((2, 65, 3, 64), None),        # whole D
               ((1, 300, 2, 40), [1, 37]),    # odd start: element path
               ((2, 9, 2, 48), [8, 20]),      # halves of 6: element path for 16-bit types
               ((4, 7, 1, 1024), [0, 1024]),  # D at its maximum
               ((2, 3, 2, 10), [4, 6]),       # one pair per row
               ((2, 33, 8, 64), None),        # 4 heads per lane (half mode's maximum)
               ((2, 9, 6, 48), [16, 48]),     # 2 heads per lane
               ((2, 9, 3, 128), [32, 128])]   # 12 or 6 chunks per half: two chunks per lane


@pytest.mark.parametrize("direction", ["forward", "backward"])
@pytest.mark.parametrize("xdt,cdt", DTYPE_PAIRS, ids=lambda d: str(d).split(".")[-1])
@pytest.mark.parametrize("layout", ["BSND", "BS1D", "B1ND", "111D"])
@pytest.mark.parametrize("shape,sl", HALF_SHAPES)
def test_half_mode_sweep(xdt, cdt, layout, shape, sl, direction):
    B, S, N, D = shape
    start, end = (0, D) if sl is None else sl
    cshape = LAYOUTS[layout](B, S, N) + (end - start,)
    case = W.inplace_case("half", B, S, N, D, xdt, cdt, sl, cos_shape=cshape, seed=B * 11 + S,
                          table="randn", device=DEV, rotary_mode=0)
    what = f"half {direction} {layout} {shape} {sl} {xdt}/{cdt}"
    if direction == "forward":
        before, x = run_inplace(case)
        check_inplace(before, x, case.cos, case.sin, sl, what, mode=0)
    else:
        g = case.x
        before = g.cpu()
        ra.rope_partial_inplace_backward(g, case.cos, case.sin, 0, sl)
        torch.cuda.synchronize()
        check_backward(before, g, case.cos, case.sin, sl, what, mode=0)


@pytest.mark.parametrize("mode,direction", [(1, "forward"), (0, "forward"), (1, "backward"),
                                            (0, "backward")])
@pytest.mark.parametrize("xdt,cdt", DTYPE_PAIRS, ids=lambda d: str(d).split(".")[-1])
@pytest.mark.parametrize("layout", ["BSND", "BS1D"])
def test_inplace_past_one_round_of_lanes(xdt, cdt, layout, mode, direction):
    """Launches longer than one round of resident lanes (256 CUs x 2048) run with 512-lane
    workgroups: [4,2048,10,128] has 0.65M to 2.6M items (two heads per lane in BS1D)."""
    B, S, N, D = 4, 2048, 10, 128
    cshape = LAYOUTS[layout](B, S, N) + (D,)
    case = W.inplace_case("rounds", B, S, N, D, xdt, cdt, None, cos_shape=cshape, seed=77,
                          table="randn", device=DEV, rotary_mode=mode)
    what = f"past one round {layout} mode {mode} {direction} {xdt}/{cdt}"
    if direction == "forward":
        before, x = run_inplace(case)
        check_inplace(before, x, case.cos, case.sin, None, what, mode=mode)
    else:
        g = case.x
        before = g.cpu()
        ra.rope_partial_inplace_backward(g, case.cos, case.sin, mode, None)
        torch.cuda.synchronize()
        check_backward(before, g, case.cos, case.sin, None, what, mode=mode)


@pytest.mark.parametrize("direction", ["forward", "backward"])
@pytest.mark.parametrize("xdt,cdt", DTYPE_PAIRS, ids=lambda d: str(d).split(".")[-1])
@pytest.mark.parametrize("layout", ["BSND", "BS1D"])
@pytest.mark.parametrize("cph", [3, 5, 6, 7, 10, 12])
def test_half_mode_padded_lane_pairs(cph, layout, xdt, cdt, direction):
    """Half mode whose halves split into a chunk count that is not a power of two: a row's
    lanes are padded to twice the next power of two and the padding lanes store nothing.
    The slice is 2 * cph chunks of the vector width, placed at an aligned inner offset of a
    wider D; 3 x 37 x 4 rows (ragged against the workgroups), cos/sin per head or shared by
    the heads (heads per lane)."""
    xs, cs = torch.empty(0, dtype=xdt).element_size(), torch.empty(0, dtype=cdt).element_size()
    V = 16 // max(xs, cs)
    L = 2 * cph * V
    start = V
    D = L + 2 * V
    B, S, N = 3, 37, 4
    sl = [start, start + L]
    cshape = LAYOUTS[layout](B, S, N) + (L,)
    case = W.inplace_case("half_pad", B, S, N, D, xdt, cdt, sl, cos_shape=cshape,
                          seed=cph * 7 + xs + cs, table="randn", device=DEV, rotary_mode=0)
    what = f"padded half {direction} cph={cph} {layout} {xdt}/{cdt}"
    if direction == "forward":
        before, x = run_inplace(case)
        check_inplace(before, x, case.cos, case.sin, sl, what, mode=0)
    else:
        g = case.x
        before = g.cpu()
        ra.rope_partial_inplace_backward(g, case.cos, case.sin, 0, sl)
        torch.cuda.synchronize()
        check_backward(before, g, case.cos, case.sin, sl, what, mode=0)


def test_half_mode_backward_full_and_autograd():
    case = W.inplace_half_bf16_slice(DEV)
    g = case.x
    before = g.cpu()
    ra.rope_partial_inplace_backward(g, case.cos, case.sin, 0, case.partial_slice)
    torch.cuda.synchronize()
    check_backward(before, g, case.cos, case.sin, case.partial_slice, "half backward full",
                   mode=0)
    # autograd wrapper in half mode: gradient of sum(w * y) is the backward op applied to w
    x0 = W.randn((2, 16, 3, 64), torch.float32, W.generator(45, DEV))
    c = W.randn((2, 16, 1, 32), torch.float32, W.generator(46, DEV))
    s = W.randn((2, 16, 1, 32), torch.float32, W.generator(47, DEV))
    w = W.randn((2, 16, 3, 64), torch.float32, W.generator(48, DEV))
    xl = x0.clone().requires_grad_(True)
    y = ra.InplacePartialRotaryMul.apply(xl * 1.0, c, s, [16, 48], 0)
    (y * w).sum().backward()
    expect = w.clone()
    ra.rope_partial_inplace_backward(expect, c, s, 0, [16, 48])
    torch.cuda.synchronize()
    check_bits_equal(xl.grad.cpu(), expect.cpu(), "autograd half mode")


# ------------------------------------------------------------------------------------------
# HIP graph capture: the library allocates nothing, never synchronizes and records no memset,
# so both operations can be captured and replayed; every replay is checked against eager runs
# (with eager work and synchronizations between the replays).
# ------------------------------------------------------------------------------------------

def test_graph_capture_replays_match_eager():
    # in-place op: each replay rotates x again, so k replays equal k eager calls
    case = W.inplace_case("graph", 2, 64, 4, 96, torch.bfloat16, torch.float32, [32, 96],
                          cos_shape=(2, 64, 1, 64), seed=61, device=DEV)
    x_static = case.x.clone()
    x_eager = case.x.clone()
    # cache op (interleaved mrope through the V2 entry point): outputs are rewritten per replay
    pos = W.mrope_positions(40, 2, 4, 5, m=3).to(DEV)
    ccase = W.cache_case("graph", pos.shape[1], 4, 2, 128, 128, torch.bfloat16, True, 100,
                         seed=62, mrope_section=[24, 20, 20], positions=pos, device=DEV,
                         cache_mode=1)
    q_static, k_static = ccase.query.clone(), ccase.key.clone()
    qo = torch.empty_like(q_static)
    ko = torch.empty_like(k_static)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as graph capture requires
        ra.rope_partial_inplace(x_static.clone(), case.cos, case.sin, 1, [32, 96])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ra.rope_partial_inplace(x_static, case.cos, case.sin, 1, [32, 96])
        ra.rope_with_cos_sin_cache_v2(ccase.positions, q_static, k_static, ccase.cache,
                                      [24, 20, 20], 128, True, 1, query_out=qo, key_out=ko)
    gen = W.generator(63, DEV)
    for replay in range(4):
        # new cache-op inputs in the captured buffers (eager work between replays)
        q_static.copy_(W.randn(q_static.shape, torch.bfloat16, gen))
        k_static.copy_(W.randn(k_static.shape, torch.bfloat16, gen))
        torch.cuda.synchronize()
        g.replay()
        ra.rope_partial_inplace(x_eager, case.cos, case.sin, 1, [32, 96])
        q_ref, k_ref = ra.rope_with_cos_sin_cache_v2(ccase.positions, q_static, k_static,
                                                     ccase.cache, [24, 20, 20], 128, True, 1)
        torch.cuda.synchronize()
        check_bits_equal(x_static.cpu(), x_eager.cpu(), f"in-place replay {replay}")
        check_bits_equal(qo.cpu(), q_ref.cpu(), f"cache q replay {replay}")
        check_bits_equal(ko.cpu(), k_ref.cpu(), f"cache k replay {replay}")
    # and the replayed cache op against the oracle on the last inputs
    compare_cache(ccase.positions.cpu(), q_static.cpu(), k_static.cpu(), ccase.cache.cpu(),
                  [24, 20, 20], 128, True, qo.cpu(), ko.cpu(), "graph replay vs oracle", 1)


def test_inplace_64bit_item_decode():
    """2^32 work items, past the 32-bit decode: x bf16 [1, 2^25, 1, 1024] (64 GiB), whole-D
    slice, bf16 cos/sin broadcast (111D).  x is filled from a seeded 65536-row block scaled per
    block (so every row's input can be rebuilt); sampled rows, including the first and last,
    are compared with the oracle.  The decode's bounds are checked on the host by
    tests/inplace_plan_check.cpp."""
    S, D, R = 1 << 25, 1024, 1 << 16
    gen = W.generator(71, DEV)
    base = W.randn((R, D), torch.bfloat16, gen)
    scales = [1.0 + 0.125 * k for k in range(7)]

    def block(blk):
        return base * scales[blk % 7]

    x = torch.empty((1, S, 1, D), dtype=torch.bfloat16, device=DEV)
    for blk in range(S // R):
        x[0, blk * R:(blk + 1) * R, 0] = block(blk)
    c = W.randn((1, 1, 1, D), torch.bfloat16, gen)
    s = W.randn((1, 1, 1, D), torch.bfloat16, gen)
    ra.rope_partial_inplace(x, c, s, 1, None)
    torch.cuda.synchronize()
    pick = torch.randint(0, S, (200,), generator=torch.Generator().manual_seed(72)).tolist()
    rows = sorted(set([0, 1, R - 1, R, S // 2, S - 2, S - 1] + pick))
    before = torch.stack([block(r // R)[r % R] for r in rows]).cpu().reshape(1, len(rows), 1, D)
    after = torch.stack([x[0, r, 0] for r in rows]).cpu().reshape(1, len(rows), 1, D)
    del x
    torch.cuda.empty_cache()
    check_inplace(before, after, c, s, None, "2^32 items, sampled rows")
