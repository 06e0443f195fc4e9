"""The default kernel's K loop, read from the gfx950 code object of the built
library (no GPU).

With one wave per SIMD, every scalar or vector instruction beyond what the
matrix core's issue slots hide stalls that SIMD's MFMAs, so the lean kernel
unrolls its K loop over the five positions of the LDS ring and keeps every
address in an immediate offset.  A compiler change or an edit that brings
arithmetic back into that loop would cost clock and busy cycles without
breaking parity; this test catches it on the CPU, from the AMD assembly of
the library built here.
"""
from __future__ import annotations

import _isa
from dense_fp16_gemm_04_amd import binding

# gemm_nt_f16_ordered_persist<TileShape<256,256,64,2,2,2,1,0,16>, RS=3, LS=8, kLean>
LEAN_SYMBOL = ("gemm_nt_f16_ordered_persist", "ILi256ELi256ELi64ELi2ELi2ELi2ELi1ELi0ELi16EEELi3ELi8ELi16EEE")

# One cycle of five K steps: 256 x 256 x 64 per step on four waves, each wave
# 128 x 128 as 8 x 8 tiles of 16 x 16, two K halves of 32.
MFMA_PER_CYCLE = 5 * 8 * 8 * 2
READS_PER_CYCLE = 5 * 2 * (8 + 8)  # one b128 fragment per 16-row tile and K half
LOADS_PER_CYCLE = 5 * (8 + 8)      # A and B: 8 x 16 bytes per lane each


def test_lean_k_loop_holds_only_mfma_lds_loads_and_a_few_scalar_adds(tmp_path):
    ins = _isa.kernel(_isa.disassemble(binding.library_path(), tmp_path), LEAN_SYMBOL)
    found = _isa.loops(ins, MFMA_PER_CYCLE)
    assert found, "no loop of %d MFMAs in the lean kernel" % MFMA_PER_CYCLE
    for body in found:
        assert body["v_mfma_f32_16x16x32_f16"] == MFMA_PER_CYCLE, body
        # no vector arithmetic at all: every v_ instruction is an MFMA
        vector = {k: v for k, v in body.items() if k.startswith("v_") and not k.startswith("v_mfma")}
        assert not vector, vector
        assert body["ds_read_b128"] == READS_PER_CYCLE, body
        assert body["buffer_load_dwordx4"] == LOADS_PER_CYCLE, body
        assert body["s_barrier"] == 5, body
        # the ring's slots and the K offset live in immediates; what the
        # scalar unit still does (M0 for the loads, the K offset, the loop
        # test) stays under one instruction in sixteen MFMAs
        scalar = sum(v for k, v in body.items() if k.startswith("s_") and k not in ("s_waitcnt", "s_barrier"))
        assert scalar <= MFMA_PER_CYCLE // 16, body
        other = {k: v for k, v in body.items() if not k.startswith(("v_mfma", "ds_read_b128", "buffer_load_dwordx4", "s_"))}
        assert not other, other
