"""Build the gfx950 libraries in this package directory: ``libgemm_nt_f16.so``
(the GEMM kernels and their C ABI) and ``libpower_probe.so`` (the power
probe, a measuring instrument that the GEMM path never loads).

One hipcc invocation per library compiles it ahead of time for gfx950 only.  ``-Xclang -target-feature -Xclang -packed-fp32-ops`` keeps the
compiler from emitting packed fp32 arithmetic (v_pk_*_f32); the host pass
warns that it does not know the feature, which is harmless.

The same invocation asks the compiler for each kernel's resource usage
(``-Rpass-analysis=kernel-resource-usage``: registers, scratch, spills,
occupancy, LDS).  The build fails if any kernel in the library uses scratch
memory or spills registers: a spill puts per-lane scratch traffic into the
K loop and slows a kernel by tens of percent without changing its results,
so nothing else would notice.  The table is written beside each library as
``<library>.resources.json``.
"""
from __future__ import annotations

import json
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "gemm_nt_f16.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgemm_nt_f16.so")
RESOURCES = os.path.join(HERE, "libgemm_nt_f16.resources.json")
PROBE_SRC = os.path.join(HERE, "csrc", "power_probe.hip")
PROBE_LIB = os.path.join(HERE, "libpower_probe.so")
PROBE_RESOURCES = os.path.join(HERE, "libpower_probe.resources.json")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def flags():
    return [
        "--offload-arch=" + ARCH,
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-Wall",
        "-Wno-unused-command-line-argument",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
    ]


_FIELDS = {
    "TotalSGPRs": "sgprs",
    "VGPRs": "vgprs",
    "AGPRs": "agprs",
    "ScratchSize [bytes/lane]": "scratch_bytes_per_lane",
    "Occupancy [waves/SIMD]": "waves_per_simd",
    "SGPRs Spill": "sgpr_spill",
    "VGPRs Spill": "vgpr_spill",
    "LDS Size [bytes/block]": "lds_bytes",
}


def parse_resource_usage(stderr: str) -> dict:
    """The compiler's kernel-resource-usage remarks -> {kernel symbol: {field: int}}."""
    kernels, cur = {}, None
    for line in stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(.+?): (\S+) \[-Rpass-analysis=kernel-resource-usage\]", line)
        if m and cur is not None and m.group(1).strip() in _FIELDS:
            try:
                cur[_FIELDS[m.group(1).strip()]] = int(m.group(2))
            except ValueError:
                pass
    return kernels


def spilling(kernels: dict) -> list:
    """Kernels that use scratch memory or spill registers."""
    return sorted(k for k, r in kernels.items()
                  if r.get("scratch_bytes_per_lane", 0) or r.get("vgpr_spill", 0) or r.get("sgpr_spill", 0))


def compile_library(src: str, lib: str, resources: str, verbose: bool = False, extra=()) -> str:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *flags(), "-Rpass-analysis=kernel-resource-usage", *extra, src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("is not a recognized feature for this target", "kernel-resource-usage")
    err = "\n".join(l for l in res.stderr.splitlines()
                    if not any(n in l for n in noise) and not re.match(r"^\s*(\d+ \||\|)", l))
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, err))
    kernels = parse_resource_usage(res.stderr)
    if not kernels:
        os.remove(tmp)
        raise RuntimeError("hipcc printed no kernel resource usage; cannot check for spills")
    bad = spilling(kernels)
    if bad:
        os.remove(tmp)
        raise RuntimeError("kernels use scratch memory or spill registers:\n" +
                           "\n".join("  %s: %s" % (k, kernels[k]) for k in bad))
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    with open(resources + ".tmp", "w") as f:
        json.dump({"arch": ARCH, "kernels": kernels}, f, indent=1, sort_keys=True)
    os.replace(resources + ".tmp", resources)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, extra=()) -> str:
    """Both libraries (`extra` flags for the GEMM library only); returns the
    GEMM library's path."""
    compile_library(SRC, LIB, RESOURCES, verbose, extra)
    compile_library(PROBE_SRC, PROBE_LIB, PROBE_RESOURCES, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
