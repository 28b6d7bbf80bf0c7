"""Host logic of bench.py (CPU only): the one-GPU refusal, the kernel-code hash that keys the
committed traffic figures, the traffic lookup, the kernel a workload is reported under, and
the buffer rotation count."""
import json
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import rope_workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_code_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    code = "int f(int a) {\n  return a + 1;\n}\n"
    src = tmp_path / "k.hip"
    src.write_text(code)
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src)])
    base = bench.kernel_code_hash()
    src.write_text("// a comment\n\nint f(int a) {  // trailing\n  return a + 1;   \n}\n\n")
    assert bench.kernel_code_hash() == base
    src.write_text("int f(int a) {\n  return a + 2;\n}\n")
    assert bench.kernel_code_hash() != base


def test_traffic_only_for_the_code_it_was_measured_on(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    good = {"kernel_code_sha256_16": bench.kernel_code_hash(), "hbm_bytes_per_launch": 1234}
    (tmp_path / "profiles" / "traffic_w1.json").write_text(json.dumps(good))
    stale = dict(good, kernel_code_sha256_16="0" * 16)
    (tmp_path / "profiles" / "traffic_w2.json").write_text(json.dumps(stale))
    assert bench.traffic_for("w1") == 1234
    assert bench.traffic_for("w2") is None
    assert bench.traffic_for("w3") is None


@pytest.mark.parametrize("H,rd,neox,dt,want", [
    (128, 128, True, torch.bfloat16, "cos_sin_cache_wave_kernel"),    # 8 units per head
    (128, 64, False, torch.float16, "cos_sin_cache_wave_kernel"),     # 16 units
    (1024, 1024, True, torch.bfloat16, "cos_sin_cache_wave_kernel"),  # 64 units
    (2048, 1024, True, torch.bfloat16, "cos_sin_cache_kernel"),       # 128 units
    (1024, 512, False, torch.float16, "cos_sin_cache_kernel"),        # 128 units
])
def test_cache_kernel_name(H, rd, neox, dt, want):
    case = W.cache_case("name", 3, 2, 1, H, rd, dt, neox, 16, seed=1)
    assert bench.kernel_name(case) == want


def test_inplace_kernel_name_and_rotation():
    case = W.inplace_case("name", 1, 2, 1, 64, torch.float32, torch.float32, [0, 64], seed=1)
    assert bench.kernel_name(case) == "inplace_rope_kernel"
    assert bench.n_sets_for(bench.MALL_DEFEAT_BYTES) == 1
    assert bench.n_sets_for(bench.MALL_DEFEAT_BYTES - 1) == 2
    assert bench.n_sets_for(25_165_824) == 86   # the headline launch: 86 buffer sets


def test_headline_is_the_largest_configuration():
    """The headline is the configuration with the most algorithmic bytes per launch (the
    1 GiB GPT-J fp16 one); every other workload is reported under `kernels`."""
    sizes = {
        "inplace_f32_1x16x2x64": 16 * (2 * 64 * 4 * 2 + 2 * 64 * 4),
        "inplace_bf16_8x4096x1x576_s512": 32768 * (64 * 2 * 2 + 2 * 64 * 4),
        "cache_rope_neox_bf16_t8192": W.cache_algo_bytes(8192, 32, 8, 128, 128, 2, 1),
        "cache_rope_gptj_f16_t32768_rd64": W.cache_algo_bytes(32768, 32, 32, 128, 64, 2, 1),
        "cache_mrope_neox_bf16_t16384": W.cache_algo_bytes(16384, 28, 4, 128, 128, 2, 3),
    }
    assert bench.WORKLOADS[0] == bench.HEADLINE == max(sizes, key=sizes.get)
    assert set(sizes) <= set(bench.WORKLOADS)
    assert len(set(bench.WORKLOADS)) == len(bench.WORKLOADS)
    assert all(w in W.CONFIGS for w in bench.WORKLOADS)


@pytest.mark.parametrize("shape,sl,xdt,cdt,want", [
    # bf16 x beside f32 cos/sin: 8-byte x lanes, one cos/sin row per row (N = 1), streamed
    ((2, 5, 1, 576), [512, 576], torch.bfloat16, torch.float32,
     dict(rows=10, row_bytes=1152, off=1024, len=128, lane_bytes=8, rows_per_lane=1,
          side_bytes=256, rows_per_side=1, side_stream=1)),
    # 32 heads sharing each (b, s) cos/sin row: 4 heads per lane of 8-byte chunks
    ((2, 3, 32, 192), [128, 192], torch.bfloat16, torch.float32,
     dict(rows=192, row_bytes=384, off=256, len=128, lane_bytes=8, rows_per_lane=4,
          side_bytes=256, rows_per_side=32, side_stream=0)),
    # fp32 throughout: 16-byte lanes, 2 heads per lane (their one cos/sin row streamed)
    ((1, 16, 2, 64), [0, 64], torch.float32, torch.float32,
     dict(rows=32, row_bytes=256, off=0, len=256, lane_bytes=16, rows_per_lane=2,
          side_bytes=256, rows_per_side=2, side_stream=1)),
    # 6 heads of 16-byte chunks: 2 per lane
    ((2, 3, 6, 64), [0, 64], torch.bfloat16, torch.bfloat16,
     dict(rows=36, row_bytes=128, off=0, len=128, lane_bytes=16, rows_per_lane=2,
          side_bytes=128, rows_per_side=6, side_stream=0)),
])
def test_inplace_access_pattern_matches_the_kernel(shape, sl, xdt, cdt, want):
    B, S, N, D = shape
    case = W.inplace_case("pat", B, S, N, D, xdt, cdt, sl, seed=1)
    assert bench.inplace_pattern(case) == want
    # the pattern moves the workload's algorithmic bytes: slice read + write, cos + sin rows
    moved = want["rows"] * want["len"] * 2 + 2 * (want["rows"] // want["rows_per_side"]) * \
        want["side_bytes"]
    assert moved == case.algo_bytes


def test_host_cpu_model_is_named():
    name = bench.host_cpu_model()
    assert name and name != "x86_64" or not os.path.exists("/proc/cpuinfo")


def test_read_write_split_of_the_algorithmic_bytes():
    inp = W.inplace_case("rw", 2, 5, 3, 96, torch.bfloat16, torch.float32, [32, 96], seed=2)
    assert bench.read_write_bytes(inp) == (2 * 5 * 3 * 64 * 2 + 2 * 2 * 5 * 64 * 4,
                                           2 * 5 * 3 * 64 * 2)
    cc = W.cache_case("rw", 7, 3, 2, 128, 64, torch.float16, False, 50, seed=3)
    rd, wr = bench.read_write_bytes(cc)
    assert wr == 7 * 5 * 128 * 2 and rd == wr + 7 * (64 * 2 + 8)


@pytest.mark.skipif(not os.path.exists(bench.CEILING_LIB), reason="libbench_ceiling.so not built")
def test_ceiling_kernels_refuse_arguments_outside_their_form():
    """bench_ceiling's entry points check their arguments before any launch (so these calls
    run without a GPU): null or misaligned buffers, sizes that are not whole lanes, a slice past
    the row, lane widths and rows per lane outside {8, 16} and {1, 2, 4}, an x of 2^31 bytes or
    more (the row pattern's store offsets are 32-bit)."""
    lib = bench.load_ceiling()
    buf = torch.zeros((1 << 16) + 256, dtype=torch.uint8)
    p = (buf.data_ptr() + 255) // 256 * 256  # 256-byte aligned, with 64 KiB behind it
    assert lib.ceiling_copy(None, p, 1024, None) == -1
    assert lib.ceiling_copy(p, p + 8, 1024, None) == -1            # misaligned source
    assert lib.ceiling_copy(p, p + 4096, 1000, None) == -1         # not whole 16-byte lanes
    assert lib.ceiling_copy(p, p + 4096, 0, None) == -1

    def rows(**kw):
        a = dict(x=p, rows=8, row_bytes=384, off=256, len=128, lane=8, rpl=4, sa=p + 8192,
                 sb=p + 12288, side=256, rps=32, stream_side=0)
        a.update(kw)
        return lib.ceiling_rows(a["x"], a["rows"], a["row_bytes"], a["off"], a["len"], a["lane"],
                                a["rpl"], a["sa"], a["sb"], a["side"], a["rps"], a["stream_side"],
                                None)
    assert rows(x=None) == -1
    assert rows(lane=4) == -1                  # lane width outside {8, 16}
    assert rows(rpl=3) == -1                   # rows per lane outside {1, 2, 4}
    assert rows(rows=6) == -1                  # rows not a multiple of rows per lane
    assert rows(off=320) == -1                 # slice past the end of the row
    assert rows(len=100) == -1                 # not whole lanes
    assert rows(side=200) == -1                # side bytes not whole 16-byte loads per lane
    assert rows(rps=2) == -1                   # rows per lane sharing different side rows
    assert rows(sa=p + 8) == -1                # misaligned side array
    assert rows(rows=1 << 23, row_bytes=256, off=0, len=128, rps=32) == -1  # x of 2^31 bytes:
    # beyond the 32-bit store offsets (refused before any launch, so no memory is touched)
    assert lib.ceiling_pairs(p, p + 8192, 4, 256, 3, None) == -1       # rows per lane
    assert lib.ceiling_pairs(p, p + 8192, 4, 240, 2, None) == -1       # not whole 32-byte units
    assert lib.ceiling_pairs(p, p + 8192, 4, 4096, 2, None) == -1      # more than 64 lanes a head
    assert lib.ceiling_pairs(p + 8, p + 8192, 4, 256, 2, None) == -1   # misaligned


def test_code_hash_covers_the_launch_plans(tmp_path, monkeypatch):
    """A change to the plan code (which kernel, grid or layout a workload gets) also detaches
    the traffic figures measured before it."""
    k, plan = tmp_path / "k.hip", tmp_path / "plan.cpp"
    k.write_text("int f(int a) { return a; }\n")
    plan.write_text("int rows = 2;\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(k), str(plan)])
    base = bench.kernel_code_hash()
    plan.write_text("int rows = 1;\n")
    assert bench.kernel_code_hash() != base


def test_cache_buffer_sets_copy_every_input():
    """Each buffer set of the cache op has its own q, k, positions and cos/sin table (so no
    launch finds an input its predecessors left in the caches); set 0 is the case's own."""
    seen = []

    class FakeBinding:
        @staticmethod
        def prepare_with_cos_sin_cache(p, q, k, c, msec, H, neox, qo, ko, cache_mode=None):
            seen.append((p, q, k, c, qo, ko))
            return lambda: None

    case = W.cache_case("sets", 5, 2, 1, 64, 64, torch.bfloat16, True, 40, seed=4)
    bench.cache_calls(FakeBinding, torch, case, 3)
    assert len(seen) == 3
    assert all(a is b for a, b in zip(seen[0][:4], (case.positions, case.query, case.key,
                                                 case.cache)))
    for j in range(6):
        ptrs = {s[j].data_ptr() for s in seen}
        assert len(ptrs) == 3, f"argument {j} shared between buffer sets"
    for s in seen[1:]:
        assert torch.equal(s[3], case.cache) and torch.equal(s[0], case.positions)
