"""Build the CPU oracle library (test infrastructure only).

``python -m oracle.build`` or ``oracle.build.build()`` compiles ``rope_oracle.c`` with gcc.
The flags keep IEEE semantics: no contraction into fused multiply-add, no fast-math.
"""
from __future__ import annotations

import hashlib
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rope_oracle.c")
# ROPE_ORACLE_LIB points the tests at another build of this file (the mutation tests load
# deliberately broken copies to show that the pins catch them).
LIB_PATH = os.environ.get("ROPE_ORACLE_LIB") or os.path.join(HERE, "librope_oracle.so")
CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror"]
# digest of the source and this script, written beside the library when it is built
STAMP_PATH = LIB_PATH + ".sources"


def source_digest() -> str:
    h = hashlib.sha256()
    for path in (SRC, os.path.abspath(__file__)):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def up_to_date() -> bool:
    """The library exists and was built from the source as it is now."""
    if not (os.path.exists(LIB_PATH) and os.path.exists(STAMP_PATH)):
        return False
    with open(STAMP_PATH) as f:
        return f.read().strip() == source_digest()


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    digest = source_digest()
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    with open(STAMP_PATH, "w") as f:
        f.write(digest + "\n")
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
