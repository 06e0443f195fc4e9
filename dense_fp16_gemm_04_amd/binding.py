"""ctypes binding of ``libgemm_nt_f16.so`` (argument marshalling only).

Every function mirrors an entry point of ``include/gemm_nt_f16.h`` by name.
PyTorch supplies device memory and the current stream; all arithmetic runs in
the library's HIP kernels.  A missing library raises ``RuntimeError``: there
is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgemm_nt_f16.so")

_lib = None
_lock = threading.Lock()

# Functions declared in include/gemm_nt_f16.h, with their ctypes signatures.
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_p = ctypes.c_void_p
SIGNATURES = {
    "gemm_nt_f16": ([_p, _p, _p, _i64, _i64, _i64, _p], ctypes.c_int),
    "gemm_nt_f16_ex": ([_p, _p, _p, _i64, _i64, _i64, _i32, _p], ctypes.c_int),
    "gemm_nt_f16_variant_count": ([], _i32),
    "gemm_nt_f16_variant_name": ([_i32], ctypes.c_char_p),
    "gemm_nt_f16_select": ([_i64, _i64, _i64], _i32),
    "gemm_nt_f16_plan": ([_i64, _i64, _i64, ctypes.POINTER(_i64), ctypes.POINTER(_i32)], _i32),
    "gemm_nt_f16_config_name": ([_i64, _i64, _i64], ctypes.c_char_p),
    "gemm_nt_f16_version": ([], ctypes.c_int),
}


class GemmError(RuntimeError):
    """A non-zero hipError_t returned by the library."""

    def __init__(self, func: str, code: int):
        super().__init__("%s failed with hipError_t %d" % (func, code))
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                "libgemm_nt_f16.so is not built (%s); run "
                "`python -c 'import __graft_entry__ as g; g.build()'`" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def gemm_nt_f16_version() -> int:
    return load().gemm_nt_f16_version()


def variants():
    lib = load()
    return [lib.gemm_nt_f16_variant_name(i).decode() for i in range(lib.gemm_nt_f16_variant_count())]


def gemm_nt_f16_config_name(M: int, N: int, K: int):
    name = load().gemm_nt_f16_config_name(M, N, K)
    return None if name is None else name.decode()


def gemm_nt_f16_select(M: int, N: int, K: int) -> int:
    return load().gemm_nt_f16_select(M, N, K)


def gemm_nt_f16_plan(M: int, N: int, K: int):
    """(variant, rows, rest): ``variant`` runs rows [0, rows) of C and, if
    rows < M, ``rest`` runs the others (-1 otherwise); variant -1 for invalid
    sizes."""
    rows = ctypes.c_int64(0)
    rest = ctypes.c_int32(0)
    v = load().gemm_nt_f16_plan(M, N, K, ctypes.byref(rows), ctypes.byref(rest))
    return v, rows.value, rest.value


def _check(a, b, out):
    import torch
    if not (isinstance(a, torch.Tensor) and isinstance(b, torch.Tensor)):
        raise TypeError("a and b must be torch tensors")
    if a.dtype != torch.float16 or b.dtype != torch.float16:
        raise TypeError("a and b must be float16")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("need a [M, K] and b [N, K], got %s and %s" % (tuple(a.shape), tuple(b.shape)))
    index = a.get_device()  # -1 for host memory
    if not a.is_cuda or b.get_device() != index:
        raise ValueError("a and b must be on the same GPU")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous (row-major, K innermost)")
    M, N = a.shape[0], b.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=a.device)
    elif (not isinstance(out, torch.Tensor) or out.dtype != torch.float16 or out.dim() != 2
          or out.shape[0] != M or out.shape[1] != N or out.get_device() != index or not out.is_contiguous()):
        raise ValueError("out must be a contiguous float16 [M, N] tensor on a's device")
    return out


_raw_stream_of = None


def _stream(index: int) -> int:
    """The HIP stream handle of the current stream of device `index` (torch's
    own accessor for it; the public Stream object where that is missing)."""
    global _raw_stream_of
    if _raw_stream_of is None:
        import torch
        _raw_stream_of = getattr(torch._C, "_cuda_getCurrentRawStream", None) or (
            lambda i: torch.cuda.current_stream(i).cuda_stream)
    return _raw_stream_of(index)


def _launch(name, a, b, out, *extra):
    """Check the tensors, then call entry point `name` on a's device and its
    current stream; the library plans for the current device, so another
    device is made current for the call."""
    import torch
    out = _check(a, b, out)
    M, K = a.shape
    N = b.shape[0]
    fn = getattr(load(), name)
    index = a.get_device()
    if index == torch.cuda.current_device():
        rc = fn(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, *extra, _stream(index))
    else:
        with torch.cuda.device(index):
            rc = fn(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, *extra, _stream(index))
    if rc != 0:
        raise GemmError(name, rc)
    return out


def gemm_nt_f16(a, b, out=None):
    """out[M, N] = a[M, K] @ b[N, K]^T in fp16 with fp32 accumulation.

    Enqueued on the current stream of a's device; returns ``out``.
    """
    return _launch("gemm_nt_f16", a, b, out)


def gemm_nt_f16_ex(a, b, out=None, variant: int = -1):
    """``gemm_nt_f16`` with an explicit kernel variant (index into ``variants()``)."""
    return _launch("gemm_nt_f16_ex", a, b, out, int(variant))
