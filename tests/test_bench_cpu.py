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
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
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
