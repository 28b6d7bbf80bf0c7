"""Build librope_amd.so in-tree for gfx950 (MI355X).

``python rope_partial_inplace_amd/build.py`` or ``build()``.  hipcc cross-compiles without
a GPU.  Code object version 5 is emitted so that the kernels load under the HIP runtime the
process already uses (PyTorch ships its own, older than this compiler).  Device code is
compiled with: no fused multiply-add contraction (the formulas are
separately rounded products and sums), float32 denormals kept, and the packed-fp32 feature
disabled (so the compiler never emits packed fp32 adds/multiplies).
"""
from __future__ import annotations

import hashlib
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "librope_amd.so")
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, "rope_plan.cpp"), os.path.join(CSRC, "rope_kernels.hip")]
# Everything the library is built from; its digest is written beside the library (STAMP_PATH)
# so that a library older than its sources is noticed before it is tested.
BUILD_INPUTS = SOURCES + [os.path.join(CSRC, "rope_plan.h"), os.path.join(INCLUDE, "rope.h"),
                          os.path.abspath(__file__)]
STAMP_PATH = LIB_PATH + ".sources"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-mcode-object-version=5", "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden", "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def bundled_targets(path: str) -> list[str]:
    """Target ids of the clang offload bundle embedded in a built library."""
    import struct
    with open(path, "rb") as f:
        data = f.read()
    i = data.find(b"__CLANG_OFFLOAD_BUNDLE__")
    if i < 0:
        return []
    n = struct.unpack_from("<Q", data, i + 24)[0]
    off, out = i + 32, []
    for _ in range(n):
        _, _, idlen = struct.unpack_from("<QQQ", data, off)
        off += 24
        out.append(data[off:off + idlen].decode())
        off += idlen
    return out


def source_digest() -> str:
    """sha256 of the library's build inputs (names and contents)."""
    h = hashlib.sha256()
    for path in BUILD_INPUTS:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def up_to_date() -> bool:
    """The library exists and was built from the sources as they are now."""
    if not (os.path.exists(LIB_PATH) and os.path.exists(STAMP_PATH)):
        return False
    with open(STAMP_PATH) as f:
        return f.read().strip() == source_digest()


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile the host planning code and the kernels separately (one hipcc call that mixes
    languages silently falls back to the default offload target), link, and check that the
    device code in the result is for gfx950 only."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    plan_o = os.path.join(objdir, "rope_plan.o")
    kern_o = os.path.join(objdir, "rope_kernels.o")
    tmp = LIB_PATH + ".tmp"
    inc = ["-I", INCLUDE, "-I", CSRC]
    _run(["g++", *HOST_FLAGS, *inc, "-c", SOURCES[0], "-o", plan_o], verbose)
    _run([hipcc(), *HIPCC_FLAGS, *(extra_flags or []), *inc, "-c", SOURCES[1], "-o", kern_o],
         verbose)
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", kern_o, plan_o, "-o", tmp],
         verbose)
    devices = [t for t in bundled_targets(tmp) if not t.startswith("host-")]
    if devices != [f"hipv4-amdgcn-amd-amdhsa--{ARCH}"]:
        raise RuntimeError(f"built library carries device code for {devices}, expected {ARCH}")
    digest = source_digest()
    os.replace(tmp, LIB_PATH)
    with open(STAMP_PATH, "w") as f:
        f.write(digest + "\n")
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
