"""Build the CPU oracle shared library (test infrastructure only).

gcc, -O2, no fast-math, no contraction of a*b+c into fma (the pipeline calls
fma() where it means one), OpenMP for whole-tile parallelism.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "wq8_oracle.c")
LIB = os.path.join(HERE, "libwq8_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wno-unknown-pragmas",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built() -> str:
    deps = [SRC, os.path.join(HERE, "wq8_oracle_body.h")]
    if not os.path.exists(LIB) or any(os.path.getmtime(d) > os.path.getmtime(LIB) for d in deps):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
