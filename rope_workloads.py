"""Seeded synthetic inputs for the RoPE apply path.

This module only draws inputs; it holds none of the rotation arithmetic.  Both the GPU
tests/benchmark and the CPU oracle are fed from here, as CPU tensors (PyTorch is used as
host memory and as a seeded normal generator).

Inputs follow the workloads the pages describe: BSND activations with a partial slice on
the head dim for the in-place op, 2-D query/key rows with a [maxSeqLen, rotaryDim] cos|sin
cache for the cache op, and the mrope position layout (text tokens with three equal rows,
image tokens with temporal/height/width grid indices).  Activations are N(0, 1) in float32,
rounded to the tensor dtype by PyTorch's own conversion.  cos/sin tables hold the standard
RoPE angles pos * theta^(-2i/d) (theta = 10000), computed in float64 and rounded once to
the table dtype, so both sides of a comparison read the very same bytes.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

THETA = 10000.0

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def generator(seed: int, device="cpu") -> torch.Generator:
    """Seeded generator on the device the inputs are drawn on (large inputs are drawn
    directly in GPU memory; host copies of the very same bytes feed the oracle)."""
    return torch.Generator(device=torch.device(device)).manual_seed(seed)


def randn(shape, dtype, gen):
    return torch.randn(tuple(shape), generator=gen, dtype=torch.float32,
                       device=gen.device).to(dtype)


def angles(pos: np.ndarray, n_freq: int, dim: int) -> np.ndarray:
    """float64 [len(pos), n_freq] angles pos * theta^(-2i/dim), i < n_freq."""
    inv = THETA ** (-2.0 * np.arange(n_freq, dtype=np.float64) / dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]


def pairwise_tables(pos: np.ndarray, length: int, dtype) -> tuple[torch.Tensor, torch.Tensor]:
    """cos/sin rows of `length` elements for the interleave layout: the angle of pair i is
    repeated on elements 2i and 2i+1.  Returns float64-derived tensors of `dtype`."""
    a = angles(pos, length // 2, length)
    c = torch.from_numpy(np.cos(a)).to(dtype)
    s = torch.from_numpy(np.sin(a)).to(dtype)
    return (torch.stack([c, c], dim=2).reshape(len(a), length),
            torch.stack([s, s], dim=2).reshape(len(a), length))


def half_tables(pos: np.ndarray, length: int, dtype) -> tuple[torch.Tensor, torch.Tensor]:
    """cos/sin rows of `length` elements for the half (rotate-half) layout: the angles of the
    length/2 frequencies, written twice (element i and element i + length/2 share one)."""
    a = angles(pos, length // 2, length)
    c, s = np.cos(a), np.sin(a)
    return (torch.from_numpy(np.concatenate([c, c], axis=1)).to(dtype),
            torch.from_numpy(np.concatenate([s, s], axis=1)).to(dtype))


def cos_sin_cache(max_seq: int, rotary_dim: int, dtype) -> torch.Tensor:
    """[max_seq, rotary_dim] cache: cos of the rotary_dim/2 angles, then their sin."""
    a = angles(np.arange(max_seq), rotary_dim // 2, rotary_dim)
    return torch.from_numpy(np.concatenate([np.cos(a), np.sin(a)], axis=1)).to(dtype)


# ------------------------------------------------------------------------------------------
# The in-place op
# ------------------------------------------------------------------------------------------

@dataclasses.dataclass
class InplaceCase:
    name: str
    x: torch.Tensor
    cos: torch.Tensor
    sin: torch.Tensor
    partial_slice: list | None
    tokens: int           # B*S
    algo_bytes: int       # bytes the op must move (slice read+write, cos, sin)
    backward: bool = False  # run the gradient op (x is then the incoming gradient)
    rotary_mode: int = 1    # 1 interleave, 0 half


def inplace_case(name, B, S, N, D, xdtype, cdtype, partial_slice, cos_shape=None, seed=0,
                 table="angles", device="cpu", rotary_mode=1):
    """x ~ N(0,1) of shape [B,S,N,D]; cos/sin of `cos_shape` (default BS1D) over the slice.

    table="angles": cos/sin from angle s * theta^(-2i/L) (s = sequence index of the row),
    laid out for the mode: repeated per pair (interleave) or written once per half (half);
    table="randn": independent N(0,1) values (per-element cos/sin).
    """
    g = generator(seed, device)
    x = randn((B, S, N, D), xdtype, g)
    start, end = (0, D) if partial_slice is None else partial_slice
    L = end - start
    cshape = list(cos_shape) if cos_shape is not None else [B, S, 1, L]
    if table == "angles":
        pos = np.arange(cshape[1]) if cshape[1] > 1 else np.zeros(1)
        tables = pairwise_tables if rotary_mode == 1 else half_tables
        c, s = tables(pos, L, cdtype)                    # [Sc, L]
        c = c.reshape(1, cshape[1], 1, L).expand(cshape).contiguous().to(device)
        s = s.reshape(1, cshape[1], 1, L).expand(cshape).contiguous().to(device)
    else:
        c = randn(cshape, cdtype, g)
        s = randn(cshape, cdtype, g)
    xs = x.element_size()
    cs = c.element_size()
    rows = B * S * N
    crow_count = int(np.prod(cshape[:3]))
    algo = rows * L * xs * 2 + 2 * crow_count * L * cs
    return InplaceCase(name, x, c, s, partial_slice, B * S, algo, rotary_mode=rotary_mode)


def inplace_f32_small(device="cpu"):
    """fp32 x [1,16,2,64], slice [0,64), cos/sin fp32 [1,16,1,64] from angles per pair."""
    return inplace_case("inplace_f32_1x16x2x64", 1, 16, 2, 64, torch.float32, torch.float32,
                        [0, 64], seed=1001, device=device)


def inplace_f32_scaled(device="cpu"):
    """The [1,16,2,64] fp32 layout with S = 524288, so that one launch moves 768 MiB, above the
    256 MB Infinity Cache: the streaming rate of the same kernel configuration."""
    return inplace_case("inplace_f32_1x524288x2x64", 1, 524288, 2, 64, torch.float32,
                        torch.float32, [0, 64], seed=1009, device=device)


def inplace_bf16_slice(device="cpu"):
    """bf16 x [8,4096,1,576], slice [512,576), cos/sin fp32 [8,4096,1,64] (pos = s)."""
    return inplace_case("inplace_bf16x_f32cs_8x4096x1x576_slice512_576", 8, 4096, 1, 576,
                        torch.bfloat16, torch.float32, [512, 576], seed=1002, device=device)


# ------------------------------------------------------------------------------------------
# The cache op
# ------------------------------------------------------------------------------------------

@dataclasses.dataclass
class CacheCase:
    name: str
    positions: torch.Tensor
    query: torch.Tensor
    key: torch.Tensor
    cache: torch.Tensor
    mrope_section: list | None
    head_size: int
    is_neox: bool
    tokens: int
    algo_bytes: int
    cache_mode: int | None = None  # None: the V1 call; 0/1: the V2 call with that cacheMode


def cache_algo_bytes(T, nq, nk, H, rd, es, npos_rows):
    """q/k rows read and written in full, one gathered rd-row per token, positions."""
    return T * ((nq + nk) * H * es * 2 + rd * es + 8 * npos_rows)


def cache_case(name, T, nq, nk, H, rd, dtype, is_neox, max_seq, seed, mrope_section=None,
               positions=None, device="cpu", cache_mode=None):
    g = generator(seed, device)
    q = randn((T, nq * H), dtype, g)
    k = randn((T, nk * H), dtype, g)
    cache = cos_sin_cache(max_seq, rd, dtype).to(device)
    if positions is None:
        positions = torch.randint(0, max_seq, (T,), generator=g, dtype=torch.int64,
                                  device=g.device)
    else:
        positions = positions.to(device)
    nrows = 1 if positions.dim() == 1 else positions.shape[0]
    es = q.element_size()
    return CacheCase(name, positions, q, k, cache, mrope_section, H, is_neox, T,
                     cache_algo_bytes(T, nq, nk, H, rd, es, nrows), cache_mode)


def mrope_positions(T_text: int, frames: int, grid_h: int, grid_w: int, m: int = 3):
    """[m, T] positions: text tokens carry their index on every row; image tokens carry
    (frame, row, column) grid indices on rows 0/1/2 (a 4th row, if asked, repeats row 0)."""
    T_img = frames * grid_h * grid_w
    text = torch.arange(T_text, dtype=torch.int64)
    idx = torch.arange(T_img, dtype=torch.int64)
    t_idx = idx // (grid_h * grid_w)
    h_idx = (idx // grid_w) % grid_h
    w_idx = idx % grid_w
    rows = [torch.cat([text, t_idx]), torch.cat([text, h_idx]), torch.cat([text, w_idx])]
    if m == 4:
        rows.append(torch.cat([text, t_idx]))
    return torch.stack(rows).contiguous()


def cache_rope_neox(device="cpu"):
    """rope NeoX bf16: T=8192, q [8192, 32*128], k [8192, 8*128], cache [32768, 128]."""
    return cache_case("cache_rope_neox_bf16_T8192_q32_k8_H128", 8192, 32, 8, 128, 128,
                      torch.bfloat16, True, 32768, seed=1003, device=device)


def cache_rope_gptj_partial(device="cpu"):
    """rope GPT-J fp16 partial: T=32768, q/k [T, 32*128], rd 64, cache [65536, 64]."""
    return cache_case("cache_rope_gptj_f16_T32768_q32_k32_H128_rd64", 32768, 32, 32, 128, 64,
                      torch.float16, False, 65536, seed=1004, device=device)


def cache_mrope(device="cpu"):
    """mrope [16,24,24] NeoX bf16: T=16384, q [T, 28*128], k [T, 4*128], cache [32768, 128]."""
    pos = mrope_positions(8192, 2, 64, 64)
    return cache_case("cache_mrope_16_24_24_neox_bf16_T16384_q28_k4_H128", 16384, 28, 4, 128,
                      128, torch.bfloat16, True, 32768, seed=1005, mrope_section=[16, 24, 24],
                      positions=pos, device=device)


def cache_mrope_interleaved(device="cpu"):
    """mrope [24,20,20] interleaved stitching (V2, cacheMode 1), NeoX bf16: the shapes of the
    sectioned mrope workload, T=16384, q [T, 28*128], k [T, 4*128], cache [32768, 128]."""
    pos = mrope_positions(8192, 2, 64, 64)
    return cache_case("cache_mrope_interleaved_24_20_20_neox_bf16_T16384_q28_k4_H128", 16384,
                      28, 4, 128, 128, torch.bfloat16, True, 32768, seed=1006,
                      mrope_section=[24, 20, 20], positions=pos, device=device, cache_mode=1)


def inplace_half_bf16_slice(device="cpu"):
    """Half mode (rotary_mode 0) on the key-side slice shape: bf16 x [8,4096,1,576], slice
    [512,576), fp32 rotate-half cos/sin [8,4096,1,64]."""
    return inplace_case("inplace_half_bf16x_f32cs_8x4096x1x576_slice512_576", 8, 4096, 1, 576,
                        torch.bfloat16, torch.float32, [512, 576], seed=1007, device=device,
                        rotary_mode=0)


def inplace_heads_bf16_bs1d(device="cpu"):
    """Query-side shape of the same layout family: bf16 x [4,2048,32,192], rope slice
    [128,192) in each of 32 heads, fp32 cos/sin [4,2048,1,64] shared by the heads (BS1D)."""
    return inplace_case("inplace_heads_bf16x_f32cs_4x2048x32x192_slice128_192_bs1d", 4, 2048, 32,
                        192, torch.bfloat16, torch.float32, [128, 192], seed=1008,
                        device=device)


def inplace_bf16_slice_backward(device="cpu"):
    """The gradient op on the key-side slice shape: incoming gradient bf16 [8,4096,1,576]."""
    case = inplace_bf16_slice(device)
    case.name = "inplace_backward_bf16_8x4096x1x576_s512"
    case.backward = True
    return case


CONFIGS = {
    "inplace_f32_1x16x2x64": inplace_f32_small,
    "inplace_bf16_8x4096x1x576_s512": inplace_bf16_slice,
    "cache_rope_neox_bf16_t8192": cache_rope_neox,
    "cache_rope_gptj_f16_t32768_rd64": cache_rope_gptj_partial,
    "cache_mrope_neox_bf16_t16384": cache_mrope,
}
CONFIGS["inplace_backward_bf16_8x4096x1x576_s512"] = inplace_bf16_slice_backward
CONFIGS["cache_mrope_interleaved_neox_bf16_t16384"] = cache_mrope_interleaved
CONFIGS["inplace_half_bf16_8x4096x1x576_s512"] = inplace_half_bf16_slice
CONFIGS["inplace_heads_bf16_4x2048x32x192_s128_bs1d"] = inplace_heads_bf16_bs1d
CONFIGS["inplace_f32_1x524288x2x64"] = inplace_f32_scaled

