"""Builds the CPU oracle shared library (test infrastructure only).

Compiles ``pkv_oracle.c`` with gcc at -O2, IEEE semantics (no fast-math, no
FMA contraction so every product and sum rounds as written), OpenMP for the
timing runs.  The result lands in ``oracle/_build/libpkv_oracle.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pkv_oracle.c")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libpkv_oracle.so")


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [
        "gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
        "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
        "-o", tmp, SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
