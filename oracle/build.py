"""Build the C oracle (test infrastructure) into oracle/liboracle.so with gcc.

Flags: -O2 with -ffp-contract=off and no fast-math, so every float operation
in the oracle is a single IEEE binary32 operation (x86-64 SSE, no excess
precision, no fused multiply-add). OpenMP is only used to split element loops.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dp_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fno-unsafe-math-optimizations", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Wextra", "-Wno-unknown-pragmas", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
