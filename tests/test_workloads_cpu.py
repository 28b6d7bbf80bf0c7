"""The synthetic-input recipe (rope_workloads.py), on the CPU: seeded draws are reproducible,
the RoPE tables hold the angles the recipe states (checked against an independent float64
evaluation with Python's math module), the mrope positions follow the text + image layout,
and the workloads carry the shapes and algorithmic byte counts the benchmark reports."""
import math
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import rope_workloads as W  # noqa: E402


def test_seeded_draws_repeat_and_differ():
    a = W.cache_case("a", 33, 3, 2, 64, 64, torch.bfloat16, True, 50, seed=9)
    b = W.cache_case("b", 33, 3, 2, 64, 64, torch.bfloat16, True, 50, seed=9)
    c = W.cache_case("c", 33, 3, 2, 64, 64, torch.bfloat16, True, 50, seed=10)
    for x, y in ((a.query, b.query), (a.key, b.key), (a.positions, b.positions)):
        assert torch.equal(x.view(torch.int16) if x.dtype != torch.int64 else x,
                           y.view(torch.int16) if y.dtype != torch.int64 else y)
    assert not torch.equal(a.query.view(torch.int16), c.query.view(torch.int16))
    i1 = W.inplace_case("i", 2, 3, 4, 32, torch.float16, torch.float32, [8, 24], seed=4)
    i2 = W.inplace_case("i", 2, 3, 4, 32, torch.float16, torch.float32, [8, 24], seed=4)
    assert torch.equal(i1.x.view(torch.int16), i2.x.view(torch.int16))


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_cache_table_holds_cos_then_sin_of_the_angles(dtype):
    max_seq, rd = 37, 64
    cache = W.cos_sin_cache(max_seq, rd, dtype)
    assert cache.shape == (max_seq, rd) and cache.dtype == dtype
    for p in (0, 1, 17, 36):
        for i in (0, 1, 15, 31):
            ang = p * 10000.0 ** (-2.0 * i / rd)
            want_c = torch.tensor(math.cos(ang), dtype=torch.float64).to(dtype)
            want_s = torch.tensor(math.sin(ang), dtype=torch.float64).to(dtype)
            assert cache[p, i].item() == want_c.item()
            assert cache[p, rd // 2 + i].item() == want_s.item()


def test_inplace_tables_repeat_each_pair_angle():
    case = W.inplace_case("t", 2, 5, 3, 32, torch.bfloat16, torch.float32, [0, 32], seed=3)
    L = 32
    assert case.cos.shape == (2, 5, 1, L)
    for b in (0, 1):
        for s in (0, 2, 4):
            for i in (0, 3, 15):
                ang = s * 10000.0 ** (-2.0 * i / L)   # position = sequence index
                c = torch.tensor(math.cos(ang), dtype=torch.float64).to(torch.float32).item()
                sn = torch.tensor(math.sin(ang), dtype=torch.float64).to(torch.float32).item()
                assert case.cos[b, s, 0, 2 * i].item() == c == case.cos[b, s, 0, 2 * i + 1].item()
                assert case.sin[b, s, 0, 2 * i].item() == sn == case.sin[b, s, 0, 2 * i + 1].item()


def test_mrope_positions_text_then_image_grid():
    T_text, frames, gh, gw = 10, 2, 3, 4
    pos = W.mrope_positions(T_text, frames, gh, gw)
    assert pos.shape == (3, T_text + frames * gh * gw) and pos.dtype == torch.int64
    for t in range(T_text):
        assert pos[:, t].tolist() == [t, t, t]
    k = T_text
    for f in range(frames):
        for h in range(gh):
            for w in range(gw):
                assert pos[:, k].tolist() == [f, h, w]
                k += 1
    pos4 = W.mrope_positions(T_text, frames, gh, gw, m=4)
    assert torch.equal(pos4[3], pos4[0])


def test_key_side_slice_workload_shape_and_bytes():
    case = W.CONFIGS["inplace_bf16_8x4096x1x576_s512"]("cpu")
    assert case.x.shape == (8, 4096, 1, 576) and case.x.dtype == torch.bfloat16
    assert case.cos.shape == (8, 4096, 1, 64) and case.cos.dtype == torch.float32
    assert case.partial_slice == [512, 576] and case.tokens == 32768
    # slice read + write (2 x 128 B) + cos and sin rows (2 x 256 B) per token
    assert case.algo_bytes == 32768 * 768 == 25_165_824


@pytest.mark.parametrize("args,per_token", [
    ((8192, 32, 8, 128, 128, 2, 1), 20_744),    # rope NeoX bf16
    ((32768, 32, 32, 128, 64, 2, 1), 32_904),   # GPT-J f16, rd 64 of 128
    ((16384, 28, 4, 128, 128, 2, 3), 16_664),   # mrope bf16, three position rows
])
def test_cache_workload_bytes_per_token(args, per_token):
    T = args[0]
    assert W.cache_algo_bytes(*args) == T * per_token
