"""Compile the CPU oracle (plain C, gcc) into oracle/liboracle.so.

The oracle is test infrastructure: the tests, the smoke check and the
benchmark's CPU-baseline leg load it; the library's product path never does.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pc_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# No fast-math, no contraction, SSE arithmetic: binary32 evaluated as written.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
          "-ffp-contract=off", "-msse2", "-mfpmath=sse", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
