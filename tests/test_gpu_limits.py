"""Parity at the size limits where the path changes form (needs an MI355X).

The kernels address their operand tiles and C through 32-bit buffer offsets:

* an operand tile of 256 rows spans 256 * 2K bytes, under 2^31 for every K
  below 2^22, the limit of the MFMA path; K = 2^22 - 8 is the largest K on
  it, with a ragged last K step;
* C rows leave through buffer stores while N <= 2^22 (a 256-row tile of C
  then spans at most 2^31 bytes), through 64-bit pointer stores beyond, and
  the persistent kernel hands such products to its one-tile form;
* from K = 2^22 the per-element kernel takes the product, and forcing an
  MFMA kernel there is an error;
* the per-element kernel (K % 8 != 0, unaligned operands, K >= 2^22) walks
  a one-dimensional grid over 16 x 16 blocks of C, so M may exceed the
  65535 x 16 rows a two-dimensional grid would reach.

Each case runs the library's own plan and each kernel the plan can choose,
on integer inputs in {-1, 0, 1}: every partial sum is an integer below
2^24, exact in fp32, so the result must equal the oracle's C16 bit for bit.
Only those kernels run here; the ablation variants are not part of the
product path.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from dense_fp16_gemm_04_amd import binding

pytestmark = pytest.mark.gpu

SELECTABLE = [
    "mfma16_256x256x64_w4_r5_persistent_lean",
    "mfma16_256x128x64_w8x_s3_l4_ordered",
    "mfma16_128x128x64_w8_s3_l4_ordered",
    "mfma16_64x64x64_w4_s3",
    "simple_f32_per_element",
]
MAX_K = 1 << 22


@pytest.fixture(scope="module", autouse=True)
def _lib():
    return binding.load()  # raises if the HIP library is missing


def ints(rows, cols, seed):
    """fp16 [rows, cols] with entries drawn uniformly from {-1, 0, 1}
    (generated as int8, so a billion entries stay within a few GB)."""
    g = np.random.Generator(np.random.PCG64(seed))
    return g.integers(-1, 2, size=(rows, cols), dtype=np.int8).astype(np.float16)


def check(a, b, label, names=SELECTABLE):
    import torch

    _, c16 = oracle.gemm_nt(a, b)
    want = c16.view(np.uint16)
    ids = {n: i for i, n in enumerate(binding.variants())}
    ta = torch.from_numpy(a).to("cuda:0")
    tb = torch.from_numpy(b).to("cuda:0")
    for name in [None] + list(names):
        print("case", label, a.shape[0], b.shape[0], a.shape[1], name or "plan", flush=True)
        if name is None:
            c = binding.gemm_nt_f16(ta, tb)
        else:
            c = binding.gemm_nt_f16_ex(ta, tb, variant=ids[name])
        torch.cuda.synchronize()
        got = c.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want), (label, name)
        del c
    return ta, tb


def test_widest_c_on_the_buffer_store_path():
    """N = 2^22: a full 256-row tile row of C spans exactly 2^31 bytes."""
    check(ints(256, 8, 71), ints(1 << 22, 8, 72), "widest-buffer-C")


def test_n_past_the_buffer_store_limit():
    """N = 2^22 + 8: pointer stores, the persistent kernel's one-tile form,
    a ragged last tile column and a masked K tail."""
    check(ints(40, 72, 73), ints((1 << 22) + 8, 72, 74), "pointer-C")


def test_largest_k_on_the_mfma_path():
    """K = 2^22 - 8: 256-row operand tiles of nearly 2^31 bytes, 65536 K
    steps of 64 with the last one cut short."""
    check(ints(256, MAX_K - 8, 75), ints(16, MAX_K - 8, 76), "largest-K")


def test_k_at_the_limit_takes_the_per_element_kernel():
    import torch

    ta, tb = check(ints(24, MAX_K, 77), ints(16, MAX_K, 78), "K-limit", names=["simple_f32_per_element"])
    ids = {n: i for i, n in enumerate(binding.variants())}
    for name in SELECTABLE[:-1]:
        with pytest.raises(binding.GemmError):
            binding.gemm_nt_f16_ex(ta, tb, variant=ids[name])
    torch.cuda.synchronize()


def test_per_element_kernel_past_65535_row_blocks():
    """M = 1,048,577 rows with K = 7 (K % 8 != 0: only the per-element kernel
    takes it): more blocks of 16 rows than a grid dimension of 65535 holds,
    so the kernel's grid-stride loop must reach them, and the last block
    holds a single row."""
    check(ints(1048577, 7, 79), ints(3, 7, 80), "many-rows", names=["simple_f32_per_element"])
