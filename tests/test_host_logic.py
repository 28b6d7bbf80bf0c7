"""CPU tests of the library's host-side index arithmetic (no GPU).

The kernels decode flat work-item indices with a multiply-high division by run-time
invariant divisors (rope_plan.h).  A wrong quotient would address memory outside a tensor,
so the formula is checked here, compiled from the library's own header, against `/`.
"""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_fastdiv_matches_integer_division(tmp_path):
    exe = tmp_path / "fastdiv_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "rope_partial_inplace_amd", "csrc"),
                    os.path.join(ROOT, "tests", "fastdiv_check.cpp"), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok")


def test_inplace_plan_covers_every_slice_element_once(tmp_path):
    """The in-place launch plan and the kernel's item decode (written out for the host in
    tests/inplace_plan_check.cpp): every slice element is touched by exactly one work item and
    paired with its own cos/sin element, over both modes, every dtype pair and broadcast
    layout, vector and element paths and 1-8 heads per lane; a 2^32-item plan takes the
    64-bit decode and stays in bounds."""
    exe = tmp_path / "inplace_plan_check"
    csrc = os.path.join(ROOT, "rope_partial_inplace_amd", "csrc")
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    os.path.join(ROOT, "tests", "inplace_plan_check.cpp"),
                    os.path.join(csrc, "rope_plan.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok")


def test_cache_plan_covers_every_output_once(tmp_path):
    """The cos/sin-cache launch plan and the kernel's tile / item / staging walk (written out
    for the host in tests/cache_plan_check.cpp): every output element written once from its
    own input position, rotated elements paired with their own cos|sin index, every LDS
    element staged once with the position row the stitching assigns, over every dtype,
    style, mrope list and cacheMode, pass-through parts and ragged last tiles."""
    exe = tmp_path / "cache_plan_check"
    csrc = os.path.join(ROOT, "rope_partial_inplace_amd", "csrc")
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    os.path.join(ROOT, "tests", "cache_plan_check.cpp"),
                    os.path.join(csrc, "rope_plan.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok")
