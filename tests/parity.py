"""Comparison helpers for the GPU parity tests (test-side only).

Tolerances (written out here, applied element by element):
  * bf16 / f16 outputs: the ordered-integer distance between the GPU bits and the oracle's
    bits (float32 arithmetic, one round-to-nearest-even) is at most 1; NaN must meet NaN.
  * f32 outputs: |gpu - exact| <= 2e-6 * (|p| + |q|) where exact is the oracle's float64 twin
    and p, q are the two products of the element's formula (the scale of a sum that may
    cancel); infinities must match, NaN must meet NaN.
  * data outside the rotated range: bit-exact.
The kernels use the oracle's operation order, so exact agreement is expected; the counts of
bit-exact elements are returned for reporting.
"""
from __future__ import annotations

import numpy as np
import torch

F32_REL = 2e-6


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16)


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def _is_nan16(b, dtype):
    e = b & 0x7FFF
    return e > (0x7C00 if dtype == torch.float16 else 0x7F80)


def ordered16(b: np.ndarray) -> np.ndarray:
    v = (b & 0x7FFF).astype(np.int32)
    return np.where(b & 0x8000, -v, v)


def check_half(gpu: torch.Tensor, ref: torch.Tensor, what: str) -> int:
    """gpu vs oracle bits for bf16/f16 outputs; returns the count of bit-exact elements."""
    g, r = bits(gpu).ravel(), bits(ref).ravel()
    gn, rn = _is_nan16(g, gpu.dtype), _is_nan16(r, ref.dtype)
    assert (gn == rn).all(), f"{what}: NaN placement differs at {np.flatnonzero(gn != rn)[:8]}"
    ok = ~gn
    d = np.abs(ordered16(g[ok]) - ordered16(r[ok]))
    worst = int(d.max()) if d.size else 0
    assert worst <= 1, (f"{what}: {int((d > 1).sum())} elements beyond 1 ulp, worst {worst} "
                        f"at {np.flatnonzero(ok)[np.argmax(d)]}")
    return int((g == r).sum())


def check_f32(gpu: torch.Tensor, exact64: np.ndarray, scale: np.ndarray, what: str) -> int:
    g = as_f64(gpu).ravel()
    e = np.asarray(exact64, dtype=np.float64).ravel()
    s = np.asarray(scale, dtype=np.float64).ravel()
    gn, en = np.isnan(g), np.isnan(e)
    assert (gn == en).all(), f"{what}: NaN placement differs"
    ok = ~gn
    inf = np.isinf(e) & ok
    assert (g[inf] == e[inf]).all(), f"{what}: infinities differ"
    fin = ok & ~inf
    with np.errstate(invalid="ignore", over="ignore"):
        err = np.abs(g[fin] - e[fin])
        bound = F32_REL * s[fin]
    bad = ~(err <= bound)
    assert not bad.any(), (f"{what}: {int(bad.sum())} f32 elements beyond 2e-6 relative; "
                           f"first at {np.flatnonzero(fin)[np.flatnonzero(bad)[:4]]}")
    return int(fin.sum())


def check_bits_equal(a: torch.Tensor, b: torch.Tensor, what: str):
    ba, bb = bits(a), bits(b)
    same = ba == bb
    assert same.all(), f"{what}: {int((~same).sum())} elements differ bit-wise"


# ---- magnitude scales of the two products of every output element (for the f32 bound) ----

def inplace_scale(x: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor, start: int, end: int,
                  mode: int = 1, backward: bool = False):
    """[..., L] scale of the rotated slice for the pairs (j, k) of the mode ((2i, 2i+1)
    interleave, (i, i + L/2) half): forward |x_j c_j| + |x_k s_j| and |x_k c_k| + |x_j s_k|;
    backward |x_j c_j| + |x_k s_k| and |x_k c_k| + |x_j s_j|."""
    xs = as_f64(x)[..., start:end]
    L = end - start
    c = np.broadcast_to(as_f64(cos), xs.shape[:-1] + (L,))
    s = np.broadcast_to(as_f64(sin), xs.shape[:-1] + (L,))
    if mode == 1:
        j, k = np.arange(0, L, 2), np.arange(1, L, 2)
    else:
        j, k = np.arange(L // 2), np.arange(L // 2, L)
    a, b = xs[..., j], xs[..., k]
    out = np.empty_like(xs)
    if not backward:
        out[..., j] = np.abs(a * c[..., j]) + np.abs(b * s[..., j])
        out[..., k] = np.abs(b * c[..., k]) + np.abs(a * s[..., k])
    else:
        out[..., j] = np.abs(a * c[..., j]) + np.abs(b * s[..., k])
        out[..., k] = np.abs(b * c[..., k]) + np.abs(a * s[..., j])
    return out


def cache_scale(x: torch.Tensor, cos_t: np.ndarray, sin_t: np.ndarray, H: int, rd: int,
                neox: bool):
    """[T, n*H] scale; cos_t/sin_t are the per-token [T, rd/2] tables the formula uses."""
    X = as_f64(x).reshape(x.shape[0], -1, H)
    out = np.abs(X.copy())
    c, s = cos_t[:, None, :], sin_t[:, None, :]
    if neox:
        a, b = X[..., : rd // 2], X[..., rd // 2: rd]
        out[..., : rd // 2] = np.abs(a * c) + np.abs(b * s)
        out[..., rd // 2: rd] = np.abs(b * c) + np.abs(a * s)
    else:
        a, b = X[..., 0:rd:2], X[..., 1:rd:2]
        out[..., 0:rd:2] = np.abs(a * c) + np.abs(b * s)
        out[..., 1:rd:2] = np.abs(b * c) + np.abs(a * s)
    return out.reshape(x.shape[0], -1)


def gathered_tables(cache: torch.Tensor, positions: torch.Tensor, mrope_section,
                    cache_mode: int = 0):
    """Per-token cos/sin tables in float64 (for the f32 scale only)."""
    C = as_f64(cache)
    P = positions.detach().cpu().numpy()
    rd = C.shape[1]
    if not mrope_section or mrope_section[0] <= 0:
        return C[P, : rd // 2], C[P, rd // 2:]
    if cache_mode == 1:
        i = np.arange(rd // 2)
        sec = np.where(i < 3 * mrope_section[1], i % 3, 0)
    else:
        edges = np.cumsum(mrope_section)
        sec = np.searchsorted(edges, np.arange(rd // 2), side="right")
    rows = P[sec, :].T                                        # [T, rd/2]
    idx = np.arange(rd // 2)[None, :]
    return C[rows, idx], C[rows, rd // 2 + idx]
