"""Seeded random configurations of both operations on the GPU, each checked element by element
against the oracle (same tolerances as test_gpu_parity).  Every case is drawn from a fixed seed,
so a failure names a reproducible configuration.

In-place op: dtype pair, D, slice (even or odd start, any even length), B/S/N, cos/sin layout,
rotary mode and direction.  Cache op: dtype, style, rope / mrope (every whitelisted list) and
cacheMode, headSize and rotaryDim (including heads of 8 to 34 64-byte blocks, either side of
64 units per head), head counts (up to 48 + 16), token count, cache length, positions and
row strides; GPT-J rope mode with a 128-byte cos|sin row over 2048+ tokens on its own.
"""
import numpy as np
import pytest
import torch

import rope_partial_inplace_amd as ra
import rope_workloads as W
from test_gpu_parity import (DEV, DTYPE_PAIRS, LAYOUTS, check_backward, check_inplace,
                             compare_cache)

pytestmark = pytest.mark.gpu

D_CHOICES = [2, 6, 10, 16, 24, 40, 64, 96, 128, 130, 192, 256, 576, 1024]
N_CHOICES = [1, 2, 3, 4, 6, 8, 12, 16, 32]
MROPE_LISTS = [[16, 24, 24], [8, 12, 12], [24, 20, 20], [11, 11, 10], [16, 16, 16, 16]]


def inplace_fuzz(seed):
    rng = np.random.default_rng(1000 + seed)
    xdt, cdt = DTYPE_PAIRS[int(rng.integers(len(DTYPE_PAIRS)))]
    D = int(rng.choice(D_CHOICES))
    L = 2 * int(rng.integers(1, D // 2 + 1))
    start = int(rng.integers(0, D - L + 1))
    if rng.random() < 0.6:
        start -= start % 2
    sl = None if (start == 0 and L == D and rng.random() < 0.5) else [start, start + L]
    N = int(rng.choice(N_CHOICES))
    B = int(rng.integers(1, 4))
    S = max(1, min(int(rng.integers(1, 300)), 300_000 // (B * N * D)))
    layout = list(LAYOUTS)[int(rng.integers(len(LAYOUTS)))]
    mode = int(rng.integers(0, 2))
    backward = bool(rng.integers(0, 2))
    return dict(xdt=xdt, cdt=cdt, shape=(B, S, N, D), sl=sl, layout=layout, mode=mode,
                backward=backward)


@pytest.mark.parametrize("seed", range(300))
def test_inplace_fuzz(seed):
    cfg = inplace_fuzz(seed)
    B, S, N, D = cfg["shape"]
    start, end = (0, D) if cfg["sl"] is None else cfg["sl"]
    cshape = LAYOUTS[cfg["layout"]](B, S, N) + (end - start,)
    case = W.inplace_case("fuzz", B, S, N, D, cfg["xdt"], cfg["cdt"], cfg["sl"], cos_shape=cshape,
                          seed=seed, table="randn", device=DEV, rotary_mode=cfg["mode"])
    what = f"fuzz {seed}: {cfg}"
    x = case.x
    before = x.cpu()
    if cfg["backward"]:
        ra.rope_partial_inplace_backward(x, case.cos, case.sin, cfg["mode"], cfg["sl"])
        torch.cuda.synchronize()
        check_backward(before, x, case.cos, case.sin, cfg["sl"], what, mode=cfg["mode"])
    else:
        ra.rope_partial_inplace(x, case.cos, case.sin, cfg["mode"], cfg["sl"])
        torch.cuda.synchronize()
        check_inplace(before, x, case.cos, case.sin, cfg["sl"], what, mode=cfg["mode"])


def cache_fuzz(seed):
    rng = np.random.default_rng(2000 + seed)
    dt = [torch.float32, torch.float16, torch.bfloat16][int(rng.integers(3))]
    align = 64 // torch.empty(0, dtype=dt).element_size()
    neox = bool(rng.integers(0, 2))
    kind = int(rng.integers(0, 3))  # 0: rope mode, 1 or 2: mrope
    sec = None
    if kind == 0:
        rd = align * int(rng.integers(1, 5))
    else:
        sec = MROPE_LISTS[int(rng.integers(len(MROPE_LISTS)))]
        rd = 2 * sum(sec)
    H = rd + align * int(rng.integers(0, 3))
    nq, nk = int(rng.integers(1, 9)), int(rng.integers(1, 9))
    T = int(rng.integers(1, 1500))
    wide = rng.random()
    if wide < 0.15:  # many heads: several wavefronts per token, a partly empty last row
        nq, nk = int(rng.integers(9, 49)), int(rng.integers(1, 17))
        T = int(rng.integers(1, 400))
    elif wide < 0.25 and kind == 0:  # wide heads either side of 64 units per head
        H = align * int(rng.choice([8, 16, 17, 32, 33, 34]))
        rd = align * int(rng.integers(1, H // align + 1))
        T = int(rng.integers(1, 200))
    max_seq = int(rng.integers(1, 3000))
    modes = [None, 0] + ([1] if sec is not None and len(sec) == 3 else [])
    cache_mode = modes[int(rng.integers(len(modes)))]
    pad_q = int(rng.integers(0, 3)) * align if rng.random() < 0.3 else 0
    return dict(dt=dt, neox=neox, sec=sec, rd=rd, H=H, nq=nq, nk=nk, T=T, max_seq=max_seq,
                cache_mode=cache_mode, pad_q=pad_q)


@pytest.mark.parametrize("seed", range(300))
def test_cache_fuzz(seed):
    cfg = cache_fuzz(seed)
    g = W.generator(3000 + seed, DEV)
    T, H, rd, dt = cfg["T"], cfg["H"], cfg["rd"], cfg["dt"]
    qbig = W.randn((T, cfg["nq"] * H + cfg["pad_q"]), dt, g)
    q = qbig[:, :cfg["nq"] * H]                 # row stride nq*H + pad (qStride)
    k = W.randn((T, cfg["nk"] * H), dt, g)
    cache = W.randn((cfg["max_seq"], rd), dt, g)
    m = len(cfg["sec"]) if cfg["sec"] else 0
    pshape = (m, T) if m else (T,)
    pos = torch.randint(0, cfg["max_seq"], pshape, generator=g, device=DEV)
    if cfg["cache_mode"] is None:
        qo, ko = ra.rope_with_cos_sin_cache(pos, q, k, cache, cfg["sec"], H, cfg["neox"])
    else:
        qo, ko = ra.rope_with_cos_sin_cache_v2(pos, q, k, cache, cfg["sec"], H, cfg["neox"],
                                               cfg["cache_mode"])
    torch.cuda.synchronize()
    compare_cache(pos.cpu(), q.cpu(), k.cpu(), cache.cpu(), cfg["sec"], H, cfg["neox"],
                  qo.cpu(), ko.cpu(), f"fuzz {seed}: {cfg}", cfg["cache_mode"])


def cache_fuzz_long(seed):
    """rotaryDim either side of 16384, where a token's cos|sin row no longer fits the tile
    kernel's LDS and each item reads the cache row directly (an own generator, so the seeds
    above keep their configurations)."""
    rng = np.random.default_rng(4000 + seed)
    dt = [torch.float32, torch.float16, torch.bfloat16][int(rng.integers(3))]
    align = 64 // torch.empty(0, dtype=dt).element_size()
    rd = align * int(rng.integers(16384 // align - 3, 24576 // align + 1))
    H = rd + align * int(rng.integers(0, 3))
    return dict(dt=dt, neox=bool(rng.integers(0, 2)), rd=rd, H=H, nq=int(rng.integers(1, 4)),
                nk=int(rng.integers(1, 3)), T=int(rng.integers(1, 24)),
                max_seq=int(rng.integers(1, 48)),
                pad_q=int(rng.integers(0, 3)) * align if rng.random() < 0.4 else 0,
                v2=bool(rng.integers(0, 2)))


@pytest.mark.parametrize("seed", range(24))
def test_cache_fuzz_long_rotary_dim(seed):
    cfg = cache_fuzz_long(seed)
    g = W.generator(5000 + seed, DEV)
    T, H, rd, dt = cfg["T"], cfg["H"], cfg["rd"], cfg["dt"]
    qbig = W.randn((T, cfg["nq"] * H + cfg["pad_q"]), dt, g)
    q = qbig[:, :cfg["nq"] * H]
    k = W.randn((T, cfg["nk"] * H), dt, g)
    cache = W.randn((cfg["max_seq"], rd), dt, g)
    pos = torch.randint(0, cfg["max_seq"], (T,), generator=g, device=DEV)
    if cfg["v2"]:
        qo, ko = ra.rope_with_cos_sin_cache_v2(pos, q, k, cache, None, H, cfg["neox"], 0)
    else:
        qo, ko = ra.rope_with_cos_sin_cache(pos, q, k, cache, None, H, cfg["neox"])
    torch.cuda.synchronize()
    compare_cache(pos.cpu(), q.cpu(), k.cpu(), cache.cpu(), None, H, cfg["neox"], qo.cpu(),
                  ko.cpu(), f"long-rd fuzz {seed}: {cfg}")


def cache_fuzz_scalar_row(seed):
    """GPT-J rope mode with a 128-byte cos|sin row and at least 2048 tokens, so that every launch
    has eight or more wavefronts per compute unit and each wavefront reads its token's row with
    scalar loads (an own generator, so the seeds above keep their configurations)."""
    rng = np.random.default_rng(6000 + seed)
    dt = [torch.float32, torch.float16, torch.bfloat16][int(rng.integers(3))]
    align = 64 // torch.empty(0, dtype=dt).element_size()
    rd = 2 * align
    H = rd + align * int(rng.integers(0, 4))
    nq, nk = int(rng.integers(1, 9)), int(rng.integers(1, 9))
    if rng.random() < 0.2:
        nq, nk = int(rng.integers(9, 33)), int(rng.integers(1, 9))
    return dict(dt=dt, rd=rd, H=H, nq=nq, nk=nk, T=int(rng.integers(2048, 4097)),
                max_seq=int(rng.integers(1, 3000)),
                pad_q=int(rng.integers(1, 3)) * align if rng.random() < 0.3 else 0,
                v2=bool(rng.integers(0, 2)))


@pytest.mark.parametrize("seed", range(24))
def test_cache_fuzz_gptj_scalar_row(seed):
    cfg = cache_fuzz_scalar_row(seed)
    g = W.generator(7000 + seed, DEV)
    T, H, rd, dt = cfg["T"], cfg["H"], cfg["rd"], cfg["dt"]
    qbig = W.randn((T, cfg["nq"] * H + cfg["pad_q"]), dt, g)
    q = qbig[:, :cfg["nq"] * H]
    k = W.randn((T, cfg["nk"] * H), dt, g)
    cache = W.randn((cfg["max_seq"], rd), dt, g)
    pos = torch.randint(0, cfg["max_seq"], (T,), generator=g, device=DEV)
    if cfg["v2"]:
        qo, ko = ra.rope_with_cos_sin_cache_v2(pos, q, k, cache, None, H, False, 0)
    else:
        qo, ko = ra.rope_with_cos_sin_cache(pos, q, k, cache, None, H, False)
    torch.cuda.synchronize()
    compare_cache(pos.cpu(), q.cpu(), k.cpu(), cache.cpu(), None, H, False, qo.cpu(), ko.cpu(),
                  f"scalar-row fuzz {seed}: {cfg}")
