"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only; gcc/g++, no GPU
code is built here).

- The CPU oracle, driven by tests/oracle_sanitize_check.c over seeded random configurations of
  both operations with exact-size buffers (and a few calls it must refuse).
- The library's host planning and validation code (rope_partial_inplace_amd/csrc/rope_plan.cpp)
  through the three host plan checks, which build thousands of plans and walk the kernels'
  index decoding for each (every 16th divisor and plan for the two longest checks).
Any out-of-bounds access, use of freed memory, leak, signed overflow or other undefined
behaviour fails the test.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, exe, timeout, args=()):
    subprocess.run(cmd, check=True, cwd=ROOT)
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=timeout, env=ENV)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout[-2000:] + r.stderr[-4000:]
    return r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize_check")
    out = _run(["gcc", "-std=c99", "-ffp-contract=off", *SAN,
                os.path.join(ROOT, "oracle", "rope_oracle.c"),
                os.path.join(ROOT, "tests", "oracle_sanitize_check.c"), "-lm", "-o", exe],
               exe, 600)
    assert int(out.split()[1]) > 10000


@pytest.mark.parametrize("check", ["fastdiv_check", "inplace_plan_check", "cache_plan_check"])
def test_host_plans_under_asan_ubsan(tmp_path, check):
    exe = str(tmp_path / check)
    inc = ["-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "rope_partial_inplace_amd", "csrc")]
    srcs = [os.path.join(ROOT, "tests", f"{check}.cpp")]
    if check != "fastdiv_check":
        srcs.append(os.path.join(ROOT, "rope_partial_inplace_amd", "csrc", "rope_plan.cpp"))
    # the plain runs (test_host_logic) cover every case; here a sample of them is enough to
    # exercise each code path under the sanitizers
    _run(["g++", "-std=c++17", *SAN, *inc, *srcs, "-o", exe], exe, 900,
         () if check == "inplace_plan_check" else ("16",))
