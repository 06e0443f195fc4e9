"""Seeded synthetic inputs for the fp16 product C = A * B^T.

This module only draws random numbers and rounds them to fp16; it holds none
of the product's arithmetic.  Both the GPU path's tests and the oracle's tests
take their inputs from here, so both sides see the same bits.

The workload family is the one the pages measure on: square fp16 problems up
to M = N = K = 8192 ("0. A Minimal Hopper Matmul", section "Performance"),
with unit-variance outputs at K = 8192 for the error figures ("6. Four
Consumers, FP16 Accumulation, and a TMA Epilogue", section "The Register
Budget Problem").  Unit-variance outputs need Var(A) * Var(B) * K = 1, so each
entry is drawn from N(0, 1/sqrt(K)) read as a *variance*: standard deviation
K**-0.25.  A is drawn first, then B, from one PCG64 stream per workload.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

SEED_BASE = 20261202


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    index: int

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


# The problem sizes: three square throughput points, the 8192 cube (headline
# throughput and the long-K error point), a ragged shape whose sizes are
# multiples of no tile size (partial tiles in M, N and K), and the two
# one-GPU shares of the cube.
WORKLOADS = (
    Workload("square_256", 256, 256, 256, 0),
    Workload("square_1024", 1024, 1024, 1024, 1),
    Workload("square_4096", 4096, 4096, 4096, 2),
    Workload("square_8192", 8192, 8192, 8192, 3),
    Workload("ragged_5000x3000x6000", 5000, 3000, 6000, 4),
    # one GPU's share of the 8192 cube split eight ways along M (A's rows) or
    # along N (B's rows): what a single GPU runs when the product is sharded
    Workload("share_m_1024x8192x8192", 1024, 8192, 8192, 5),
    Workload("share_n_8192x1024x8192", 8192, 1024, 8192, 6),
)

HEADLINE = WORKLOADS[3]


def by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def gaussian(M: int, N: int, K: int, seed: int):
    """A [M, K] and B [N, K], fp16, entries N(0, variance K**-0.5), A first."""
    g = np.random.Generator(np.random.PCG64(seed))
    std = float(K) ** -0.25 if K > 0 else 1.0
    a = (g.standard_normal((M, K)) * std).astype(np.float16)
    b = (g.standard_normal((N, K)) * std).astype(np.float16)
    return a, b


def workload_inputs(w: Workload):
    return gaussian(w.M, w.N, w.K, w.seed)


def small_integers(M: int, N: int, K: int, seed: int, lo: int = -1, hi: int = 1):
    """fp16 A [M, K] and B [N, K] with integer entries in [lo, hi].

    With |entries| <= 2 and K small enough that every partial sum stays an
    integer below 2**24 in magnitude, any fp32 summation order is exact, so a
    correct kernel reproduces the exact result bit for bit.
    """
    g = np.random.Generator(np.random.PCG64(seed))
    a = g.integers(lo, hi + 1, size=(M, K)).astype(np.float16)
    b = g.integers(lo, hi + 1, size=(N, K)).astype(np.float16)
    return a, b


def digest(*arrays) -> str:
    """SHA-256 over the raw bytes of the given arrays (in order)."""
    h = hashlib.sha256()
    for x in arrays:
        h.update(np.ascontiguousarray(x).tobytes())
    return h.hexdigest()
