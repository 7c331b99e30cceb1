"""Build the CPU oracle (test infrastructure): ``oracle/liboracle.so`` from ``qdg_oracle.c``.

Plain gcc, no fast-math, no contraction of ``a*b+c`` (the only fused
multiply-adds are the explicit ``fmaf`` calls), OpenMP for the row loop.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qdg_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fno-finite-math-only", "-frounding-math", "-fopenmp"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
