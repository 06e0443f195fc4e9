"""Accumulation precision: why the path accumulates in fp32.

The pages move their last kernel to fp16 accumulation to free registers and
report what it costs in accuracy at K = 8192 with unit-variance outputs ("6.
Four Consumers, FP16 Accumulation, and a TMA Epilogue", section "The Register
Budget Problem"): mean |error| 0.0023, p99 0.0117, max 0.047 against an
fp32-accumulating library, versus mean 0.00014 and max 0.0020 with fp32
accumulation.  This library keeps fp32 accumulation (CDNA4's fp16 MFMA
accumulates in fp32 anyway).  These CPU tests reproduce both sets of figures
from their mechanisms, so the report can put the two side by side:

* fp16 accumulation: a tensor-core MMA adds a block of 16 products to the
  accumulator and rounds once to fp16; over K = 8192 that is 512 fp16
  roundings of a running sum that grows to |C| ~ 1..4;
* fp32 accumulation with one final fp16 cast: the error is the fp16 rounding
  of the result (the oracle's C16 against C64).

The emulation is plain numpy and is not part of the oracle.
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
from dense_fp16_gemm_04_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def fp16_accumulate(a, b, block=16):
    """C[m, n] with an fp16 accumulator: each block of `block` products is
    summed exactly and added to the accumulator with one fp16 rounding."""
    a64 = a.astype(np.float64)
    b64 = b.astype(np.float64)
    K = a.shape[1]
    acc = np.zeros((a.shape[0], b.shape[0]), dtype=np.float16)
    for k0 in range(0, K, block):
        part = a64[:, k0:k0 + block] @ b64[:, k0:k0 + block].T
        acc = (acc.astype(np.float64) + part).astype(np.float16)
    return acc


def _figures():
    with open(os.path.join(GOLDEN, "pages_error_figures.json")) as f:
        return json.load(f)


def test_fp16_accumulation_reproduces_the_pages_figures():
    fig = _figures()["fp16_accumulation_vs_fp32_library"]
    a, b = workloads.gaussian(96, 96, 8192, seed=workloads.HEADLINE.seed)
    c64, _ = oracle.gemm_nt(a, b)
    err = np.abs(fp16_accumulate(a, b).astype(np.float64) - c64)
    mean, p99 = float(err.mean()), float(np.percentile(err, 99))
    print("fp16 accumulation: mean %.5f p99 %.5f max %.5f" % (mean, p99, err.max()))
    assert abs(mean - fig["mean_abs"]) < 0.2 * fig["mean_abs"]
    assert abs(p99 - fig["p99_abs"]) < 0.3 * fig["p99_abs"]
    assert err.max() < fig["tolerance_used_by_the_pages"]


def test_fp32_accumulation_is_an_order_of_magnitude_tighter():
    fig = _figures()
    a, b = workloads.gaussian(96, 96, 8192, seed=workloads.HEADLINE.seed)
    c64, c16 = oracle.gemm_nt(a, b)
    e32 = np.abs(c16.astype(np.float64) - c64)
    e16 = np.abs(fp16_accumulate(a, b).astype(np.float64) - c64)
    assert e32.max() <= fig["fp32_accumulation_vs_fp32_reference"]["max_abs"]
    assert e16.mean() > 10 * e32.mean()


def test_fp16_accumulation_of_one_block_is_one_rounding():
    """With K = 16 the emulation is a single fp16 rounding of the exact sum,
    i.e. the oracle's C16."""
    a, b = workloads.gaussian(40, 24, 16, seed=7)
    _, c16 = oracle.gemm_nt(a, b)
    assert np.array_equal(fp16_accumulate(a, b).view(np.uint16), c16.view(np.uint16))


STUDY_K = (1024, 4096, 8192, 16384)


def accumulation_table(ks=STUDY_K, m=96, n=96):
    """Error against the exact sum for fp16 accumulation (blocks of 16) and
    for fp32 accumulation with one final fp16 cast, at unit-variance outputs
    for each K (inputs N(0, K**-0.5) as in every workload): one row per K
    with the mean, p99 and max of |error|."""
    rows = []
    for K in ks:
        a, b = workloads.gaussian(m, n, K, seed=workloads.SEED_BASE + K)
        c64, c16 = oracle.gemm_nt(a, b)
        e16 = np.abs(fp16_accumulate(a, b).astype(np.float64) - c64)
        e32 = np.abs(c16.astype(np.float64) - c64)
        rows.append({"K": K,
                     "fp16_acc": (float(e16.mean()), float(np.percentile(e16, 99)), float(e16.max())),
                     "fp32_acc": (float(e32.mean()), float(np.percentile(e32, 99)), float(e32.max()))})
    return rows


def test_accumulation_error_across_k():
    """fp16 accumulation rounds a running sum of size ~1 once per block of
    16 products, so its error grows with the number of blocks, K / 16 (as a
    random walk of roundings, roughly with its square root); fp32
    accumulation leaves only the final cast, whose error does not depend on
    K.  At K = 8192 both match the pages' figures."""
    rows = accumulation_table()
    print("\n    K | fp16 accumulation mean / p99 / max | fp32 accumulation, one fp16 cast: mean / p99 / max")
    for r in rows:
        print("%5d | %.5f / %.5f / %.4f | %.6f / %.6f / %.5f" % ((r["K"],) + r["fp16_acc"] + r["fp32_acc"]))
    means16 = [r["fp16_acc"][0] for r in rows]
    assert all(x < y for x, y in zip(means16, means16[1:]))
    # a random walk of K / 16 roundings: the mean grows by about sqrt(2) per doubling of K
    assert 2.5 < means16[-1] / means16[0] < 6.0  # 16x the blocks
    for r in rows:
        mean32, _, max32 = r["fp32_acc"]
        assert 1.1e-4 < mean32 < 1.7e-4 and max32 <= 2.0e-3
        assert r["fp16_acc"][0] > 5 * mean32
    fig = _figures()["fp16_accumulation_vs_fp32_library"]
    at8192 = [r for r in rows if r["K"] == 8192][0]
    assert abs(at8192["fp16_acc"][0] - fig["mean_abs"]) < 0.2 * fig["mean_abs"]
