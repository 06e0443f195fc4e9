"""Reading the AMD assembly of a library built here: the gfx950 code object
is taken out of the shared library's HIP fat binary and disassembled with the
ROCm LLVM tools (no GPU needed)."""
from __future__ import annotations

import collections
import os
import re
import subprocess

import pytest

LLVM = "/opt/rocm/llvm/bin"
TOOLS = ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")


def disassemble(lib: str, tmp_path) -> str:
    """The gfx950 disassembly of `lib`; skips the test when the library or
    the tools are missing."""
    if not os.path.exists(lib):
        pytest.skip("%s not built" % os.path.basename(lib))
    for t in TOOLS:
        if not os.path.exists(os.path.join(LLVM, t)):
            pytest.skip("%s not installed" % t)
    fatbin = str(tmp_path / "fatbin.bin")
    co = str(tmp_path / "gfx950.o")
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section=.hip_fatbin=" + fatbin, lib,
                    str(tmp_path / "copy.so")], check=True, capture_output=True)
    subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o", "--input=" + fatbin,
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", "--output=" + co], check=True, capture_output=True)
    out = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", co],
                         check=True, capture_output=True, text=True)
    return out.stdout


def kernel(asm: str, parts) -> list:
    """(address, mnemonic, branch target address or None) of the one kernel
    whose symbol contains every string in `parts`."""
    lines = asm.splitlines()
    starts = [i for i, l in enumerate(lines) if l.endswith(">:") and all(p in l for p in parts)]
    assert len(starts) == 1, "expected one kernel matching %s, found %d" % (parts, len(starts))
    ins = []
    for l in lines[starts[0] + 1:]:
        if not l.strip():
            break
        m = re.match(r"\s+(\S+).*?//\s*([0-9A-F]+):", l)
        if not m:
            continue
        t = re.search(r"\+0x([0-9a-f]+)>\s*$", l) if "branch" in m.group(1) else None
        ins.append((int(m.group(2), 16), m.group(1), int(t.group(1), 16) if t else None))
    base = ins[0][0]
    return [(a, mn, None if t is None else base + t) for a, mn, t in ins]


def loops(ins, mfmas: int) -> list:
    """Instruction counts (mnemonic -> count) of every loop, closed by a
    backward branch, that holds exactly `mfmas` MFMAs."""
    out = []
    for a, _, t in ins:
        if t is not None and t <= a:
            body = collections.Counter(m for x, m, _ in ins if t <= x <= a)
            if sum(v for k, v in body.items() if k.startswith("v_mfma")) == mfmas:
                out.append(body)
    return out
