"""CPU oracle for C = A * B^T in fp16 (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never import it, and it imports nothing from them.

It wraps ``gemm_oracle.c`` (plain C, built with gcc by ``oracle/build.py``):

* ``gemm_nt(a16, b16)`` -> ``(c64, c16)``: the plain definition
  ``C64[m, n] = sum_k dec(A[m, k]) * dec(B[n, k])`` in binary64 with a
  sequential k order, and ``C16 = rne_fp16(C64)``.  This is the operation of
  "0. A Minimal Hopper Matmul", section "Block Tiling" (C = A x B^T, A is
  (M, K), B is (N, K), both K-major), accumulated wider than the fp16 inputs
  and cast to fp16 once at the end (same page, "Walkthrough" / "Epilogue").
* ``gemm_nt_entries(a16, b16, rows, cols)``: the same sum for selected
  outputs only.
* ``decode`` / ``encode_rne``: the oracle's own IEEE 754 binary16 codec.

Every function here is pinned by ``tests/test_oracle.py`` against things
other than itself (numpy's conversions, exact rational arithmetic, closed
forms and algebraic invariants).  Individual output values of the Gaussian
workloads have no printed value on the pages to compare with: that part is
pinned only through the codec, exact arithmetic and the invariants.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_gemm.so")
_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_f16_decode.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_decode.restype = ctypes.c_double
    lib.oracle_f16_encode_rne.argtypes = [ctypes.c_double]
    lib.oracle_f16_encode_rne.restype = ctypes.c_uint16
    lib.oracle_f16_decode_array.argtypes = [_p, _p, _i64]
    lib.oracle_f16_decode_array.restype = None
    lib.oracle_f16_encode_array.argtypes = [_p, _p, _i64]
    lib.oracle_f16_encode_array.restype = None
    lib.oracle_gemm_nt_f16.argtypes = [_p, _p, _i64, _i64, _i64, _p, _p, ctypes.c_int]
    lib.oracle_gemm_nt_f16.restype = ctypes.c_int
    lib.oracle_gemm_nt_f64.argtypes = [_p, _p, _i64, _i64, _i64, _p, ctypes.c_int]
    lib.oracle_gemm_nt_f64.restype = ctypes.c_int
    lib.oracle_gemm_nt_f16_entries.argtypes = [_p, _p, _i64, _i64, _i64, _p, _p, _i64, _p]
    lib.oracle_gemm_nt_f16_entries.restype = ctypes.c_int
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _bits(x) -> np.ndarray:
    """fp16 array (or uint16 bit patterns) -> contiguous uint16 bits."""
    x = np.asarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    if x.dtype != np.uint16:
        raise TypeError("expected float16 values or uint16 bit patterns, got %s" % x.dtype)
    return np.ascontiguousarray(x)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def decode(h) -> np.ndarray:
    """binary16 bit patterns (or fp16 values) -> exact binary64 values."""
    h = _bits(h)
    out = np.empty(h.shape, dtype=np.float64)
    _load().oracle_f16_decode_array(_ptr(h), _ptr(out), h.size)
    return out


def encode_rne(x) -> np.ndarray:
    """binary64 values -> binary16 bit patterns, round to nearest, ties to even."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_f16_encode_array(_ptr(x), _ptr(out), x.size)
    return out


def gemm_nt(a16, b16, threads: int | None = None):
    """C = A * B^T for fp16 A [M, K] and B [N, K].

    Returns ``(c64, c16)``: the binary64 sum (float64 [M, N]) and its
    round-to-nearest-even fp16 rounding (float16 [M, N]).
    """
    a = _bits(a16)
    b = _bits(b16)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("need A [M, K] and B [N, K], got %s and %s" % (a.shape, b.shape))
    M, K = a.shape
    N = b.shape[0]
    c64 = np.zeros((M, N), dtype=np.float64)
    c16 = np.zeros((M, N), dtype=np.uint16)
    rc = _load().oracle_gemm_nt_f16(_ptr(a), _ptr(b), M, N, K, _ptr(c64), _ptr(c16),
                                    threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_gemm_nt_f16 failed with %d" % rc)
    return c64, c16.view(np.float16)


def gemm_nt_f64(a, b, threads: int | None = None) -> np.ndarray:
    """The same sum on binary64 inputs (no fp16 decode): float64 [M, N]."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    b = np.ascontiguousarray(np.asarray(b, dtype=np.float64))
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("need a [M, K] and b [N, K], got %s and %s" % (a.shape, b.shape))
    M, K = a.shape
    N = b.shape[0]
    c = np.zeros((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_nt_f64(_ptr(a), _ptr(b), M, N, K, _ptr(c),
                                    threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_gemm_nt_f64 failed with %d" % rc)
    return c


def gemm_nt_entries(a16, b16, rows, cols) -> np.ndarray:
    """C64[rows[i], cols[i]] for each i: selected outputs of the same sum."""
    a = _bits(a16)
    b = _bits(b16)
    M, K = a.shape
    N = b.shape[0]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in shape")
    out = np.empty(rows.shape, dtype=np.float64)
    rc = _load().oracle_gemm_nt_f16_entries(_ptr(a), _ptr(b), M, N, K, _ptr(rows),
                                            _ptr(cols), rows.size, _ptr(out))
    if rc != 0:
        raise RuntimeError("oracle_gemm_nt_f16_entries failed with %d" % rc)
    return out
