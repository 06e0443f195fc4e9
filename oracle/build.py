"""Build the CPU oracle library (test infrastructure only).

Compiles ``gemm_oracle.c`` with gcc into ``liboracle_gemm.so`` beside it.
``-ffp-contract=off`` keeps every product and every addition a separately
rounded binary64 operation (no fused multiply-add), and no fast-math flag is
used, so the sum is the plain sequential one the source describes.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemm_oracle.c")
LIB = os.path.join(HERE, "liboracle_gemm.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-pthread", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile the oracle; returns the path of the shared library."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
