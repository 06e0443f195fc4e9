"""Write ``workload_digests.json``: the SHA-256 of each workload's fp16 input
bytes (A then B, row-major), as the seeded generator draws them.

The digests pin the inputs themselves, so that the oracle, the GPU tests and
the benchmark provably see the same bits on every machine.  This script uses
only the input generator (no arithmetic of the product); run it from the
repository root:

    python tests/golden/make_workload_digests.py
"""
from __future__ import annotations

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from dense_fp16_gemm_04_amd import workloads  # noqa: E402


def main() -> None:
    out = {
        "what": "SHA-256 of A's then B's fp16 bytes (row-major, little-endian) per workload",
        "generator": "numpy.random.Generator(PCG64(20261202 + index)); A then B, "
                     "standard_normal * K**-0.25 rounded to float16",
        "digests": {},
    }
    for w in workloads.WORKLOADS:
        a, b = workloads.workload_inputs(w)
        out["digests"][w.name] = {"M": w.M, "N": w.N, "K": w.K, "seed": w.seed,
                                  "sha256": workloads.digest(a, b)}
        print(w.name, out["digests"][w.name]["sha256"], flush=True)
    with open(os.path.join(HERE, "workload_digests.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
