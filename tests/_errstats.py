"""Error distribution of a GPU result against the oracle's binary64 sum.

Parity tests call ``record`` on each Gaussian workload; ``tests/conftest.py``
prints the collected rows as a table at the end of the session and, when the
environment variable GEMM_ERROR_REPORT names a file, writes them there as
JSON.  Beside the GPU's error the table gives the error of the oracle's own
fp16 rounding, rne(C64) - C64: the least any fp16 output can have, and the
quantity the pages' fp32-accumulation figures measure ("6. Four Consumers,
FP16 Accumulation, and a TMA Epilogue", "The Register Budget Problem").
"""
from __future__ import annotations

import numpy as np

RECORDS = []


def _p99(x: np.ndarray) -> float:
    k = int(0.99 * (x.size - 1))
    return float(np.partition(x.ravel(), k)[k])


def record(label: str, got16: np.ndarray, c64: np.ndarray, c16: np.ndarray, K: int) -> dict:
    got = got16.astype(np.float64)
    diff = got - c64
    err = np.abs(diff)
    floor = np.abs(c16.astype(np.float64) - c64)
    rec = {
        "workload": label,
        "K": int(K),
        "outputs": int(err.size),
        "mean": float(err.mean()),
        "p99": _p99(err),
        "max": float(err.max()),
        "signed_mean": float(diff.mean()),
        "bit_equal_to_rne_c64": float(np.mean(got16.view(np.uint16) == c16.view(np.uint16))),
        "rne_floor_mean": float(floor.mean()),
        "rne_floor_max": float(floor.max()),
        "var_c64": float(c64.var()),
    }
    RECORDS.append(rec)
    print("errors %s: mean %.4g p99 %.4g max %.4g signed %.3g bit-equal %.5f (rne floor: mean %.4g max %.4g)"
          % (label, rec["mean"], rec["p99"], rec["max"], rec["signed_mean"], rec["bit_equal_to_rne_c64"],
             rec["rne_floor_mean"], rec["rne_floor_max"]), flush=True)
    return rec
