"""Build the CPU oracle library (test infrastructure only).

``python -m oracle.build`` or ``oracle.build.build()`` compiles ``rope_oracle.c`` with gcc.
The flags keep IEEE semantics: no contraction into fused multiply-add, no fast-math.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rope_oracle.c")
# ROPE_ORACLE_LIB points the tests at another build of this file (the mutation tests load
# deliberately broken copies to show that the pins catch them).
LIB_PATH = os.environ.get("ROPE_ORACLE_LIB") or os.path.join(HERE, "librope_oracle.so")
CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
