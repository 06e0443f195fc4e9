"""fp16 C = A * B^T on AMD Instinct MI355X (gfx950).

The product runs in hand-written HIP kernels behind a C ABI
(``include/gemm_nt_f16.h``, built into ``libgemm_nt_f16.so`` in this
package).  The Python functions here only marshal arguments; the library is
loaded on first use and an error is raised if it is missing.
"""
from __future__ import annotations

__all__ = [
    "gemm_nt_f16",
    "gemm_nt_f16_ex",
    "gemm_nt_f16_config_name",
    "gemm_nt_f16_select",
    "gemm_nt_f16_version",
    "variants",
    "library_path",
    "load",
    "GemmError",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
