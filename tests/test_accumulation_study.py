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
