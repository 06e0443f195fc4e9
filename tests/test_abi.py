"""The C ABI library without a GPU: it loads, exports what the header
declares, and rejects bad arguments on the host before enqueuing anything."""
from __future__ import annotations

import os
import re

import pytest

from dense_fp16_gemm_04_amd import binding, workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_nt_f16.h")

INVALID = 1  # hipErrorInvalidValue


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_nt_f16\w*)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return binding.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert "gemm_nt_f16" in names and "gemm_nt_f16_ex" in names
    for name in names:
        assert hasattr(lib, name), name
    # and the binding wraps exactly those
    assert sorted(binding.SIGNATURES) == names


def test_version_matches_header(lib):
    m = re.search(r"#define\s+GEMM_NT_F16_VERSION\s+(\d+)", open(HEADER).read())
    assert lib.gemm_nt_f16_version() == int(m.group(1))


def test_variant_table(lib):
    n = lib.gemm_nt_f16_variant_count()
    assert n >= 2
    names = [lib.gemm_nt_f16_variant_name(i) for i in range(n)]
    assert all(isinstance(x, bytes) and x for x in names)
    assert len(set(names)) == n
    assert lib.gemm_nt_f16_variant_name(n) is None
    assert lib.gemm_nt_f16_variant_name(-1) is None


def test_selection(lib):
    n = lib.gemm_nt_f16_variant_count()
    for w in workloads.WORKLOADS:
        v = lib.gemm_nt_f16_select(w.M, w.N, w.K)
        assert 0 <= v < n
        assert binding.gemm_nt_f16_config_name(w.M, w.N, w.K).startswith("mfma")
    name = binding.gemm_nt_f16_config_name
    assert name(8192, 8192, 8192) == "mfma16_256x256x64_w4_r5_persistent_lean"
    assert name(4096, 4096, 4096) == "mfma16_256x256x64_w4_r5_persistent_lean"
    assert name(5000, 3000, 6000) == "mfma16_256x256x64_w4_r5_persistent_lean"
    assert name(4096, 4096, 1024) == "mfma16_256x256x64_w4_r5_persistent_lean"
    assert name(2048, 2048, 8192) == "mfma16_128x128x64_w8_s3_l4_ordered"
    assert name(2048, 2048, 2048) == "mfma16_128x128x64_w8_s3_l4_ordered"
    assert name(1024, 1024, 1024) == "mfma16_64x64x64_w4_s3"
    assert name(256, 256, 256) == "mfma16_64x64x64_w4_s3"
    # 256-row products: 128 tiles of 128x128 leave half the CUs idle, which
    # the model credits with a faster per-CU rate; 64x64 would take 512 tiles
    assert name(256, 8192, 8192) == "mfma16_128x128x64_w8_s3_l4_ordered"
    assert name(8192, 256, 8192) == "mfma16_128x128x64_w8_s3_l4_ordered"
    assert name(1024, 1024, 8192) == "mfma16_64x64x64_w4_s3"
    # one GPU's share of an 8192^3 product split eight ways along M or N
    assert name(1024, 8192, 8192) == "mfma16_256x128x64_w8x_s3_l4_ordered"
    assert name(8192, 1024, 8192) == "mfma16_256x128x64_w8x_s3_l4_ordered"
    # K not a multiple of 8 cannot use the MFMA kernels
    assert binding.gemm_nt_f16_config_name(64, 64, 7).startswith("simple")
    assert lib.gemm_nt_f16_select(-1, 4, 4) == -1
    assert lib.gemm_nt_f16_config_name(4, -4, 4) is None


FAKE_A = 0x10000
FAKE_B = 0x200000
FAKE_C = 0x4000000


def call(lib, a, b, c, M, N, K, variant=None):
    if variant is None:
        return lib.gemm_nt_f16(a, b, c, M, N, K, None)
    return lib.gemm_nt_f16_ex(a, b, c, M, N, K, variant, None)


def test_negative_dimensions_rejected(lib):
    for M, N, K in [(-1, 4, 4), (4, -1, 4), (4, 4, -1)]:
        assert call(lib, FAKE_A, FAKE_B, FAKE_C, M, N, K) == INVALID


def test_null_pointers_rejected(lib):
    assert call(lib, None, FAKE_B, FAKE_C, 4, 4, 4) == INVALID
    assert call(lib, FAKE_A, None, FAKE_C, 4, 4, 4) == INVALID
    assert call(lib, FAKE_A, FAKE_B, None, 4, 4, 4) == INVALID


def test_empty_output_is_a_no_op(lib):
    # nothing to write: success without touching any pointer or the GPU
    assert call(lib, None, None, None, 0, 5, 5) == 0
    assert call(lib, None, None, None, 5, 0, 5) == 0


def test_overlap_rejected(lib):
    # C [4 x 4] fp16 = 32 bytes starting inside A or B
    assert call(lib, FAKE_A, FAKE_B, FAKE_A + 16, 4, 4, 8) == INVALID
    assert call(lib, FAKE_A, FAKE_B, FAKE_B + 8, 4, 4, 8) == INVALID
    assert call(lib, FAKE_A, FAKE_B, FAKE_A - 16, 4, 4, 8) == INVALID


def test_odd_pointer_rejected(lib):
    assert call(lib, FAKE_A + 1, FAKE_B, FAKE_C, 4, 4, 8) == INVALID


def test_too_large_rejected(lib):
    assert call(lib, FAKE_A, FAKE_B, FAKE_C, 1 << 31, 4, 8) == INVALID


def test_variant_checks(lib):
    n = lib.gemm_nt_f16_variant_count()
    assert call(lib, FAKE_A, FAKE_B, FAKE_C, 4, 4, 8, variant=n) == INVALID
    # an MFMA variant needs 16-byte aligned A and B and K % 8 == 0
    assert call(lib, FAKE_A + 2, FAKE_B, FAKE_C, 4, 4, 8, variant=0) == INVALID
    assert call(lib, FAKE_A, FAKE_B, FAKE_C, 4, 4, 6, variant=0) == INVALID


def test_binding_rejects_bad_tensors():
    torch = pytest.importorskip("torch")
    a = torch.zeros((4, 8), dtype=torch.float16)
    b = torch.zeros((4, 8), dtype=torch.float32)
    with pytest.raises(TypeError):
        binding.gemm_nt_f16(a, b)
    with pytest.raises(ValueError):
        binding.gemm_nt_f16(a, torch.zeros((4, 9), dtype=torch.float16))
    with pytest.raises(ValueError):  # CPU tensors: no GPU path here
        binding.gemm_nt_f16(a, torch.zeros((4, 8), dtype=torch.float16))


def test_launch_plan_invariants_on_random_shapes(lib):
    """Over 2000 seeded random shapes: a plan is one kernel on all rows, or a
    256x256 kernel on the most whole tile rows whose tiles fit in some number
    of waves over the chip's 256 CUs, plus a kernel the model picks (possibly
    the same one) on the rest."""
    import numpy as np

    names = binding.variants()
    g = np.random.Generator(np.random.PCG64(2024))
    splits = 0
    for _ in range(2000):
        M, N = (int(x) for x in g.integers(1, 20000, size=2))
        K = int(g.choice([8, 64, 72, 256, 1000, 1024, 2048, 4096, 6000, 8192]))
        v, rows, rest = binding.gemm_nt_f16_plan(M, N, K)
        assert 0 <= v < len(names) and names[v] != "simple_f32_per_element", (M, N, K)
        assert v == binding.gemm_nt_f16_select(M, N, K)
        if rest == -1:
            assert rows == M, (M, N, K)
            continue
        splits += 1
        assert names[v] == "mfma16_256x256x64_w4_r5_persistent_lean", (M, N, K)
        assert 0 < rows < M and rows % 256 == 0, (M, N, K, rows)
        assert 0 <= rest < len(names) and names[rest] != "simple_f32_per_element", (M, N, K)
        # w waves hold the first rows' tiles, and one more tile row would not fit
        tiles_n = (N + 255) // 256
        r = rows // 256
        w = -(-r * tiles_n // 256)
        assert r * tiles_n <= w * 256 < (r + 1) * tiles_n, (M, N, K, rows)
    assert splits > 0


def test_launch_plan(lib):
    """The row split of gemm_nt_f16 (host logic only)."""
    names = binding.variants()
    plan = binding.gemm_nt_f16_plan
    # full waves of 256x256 tiles, or one wave: one kernel on all of C
    for shape in [(8192, 8192, 8192), (4096, 4096, 4096), (12288, 12288, 4096), (5000, 3000, 6000)]:
        v, rows, rest = plan(*shape)
        assert (rows, rest) == (shape[0], -1), shape
        assert v == binding.gemm_nt_f16_select(*shape)
    # a small last wave: whole waves over the first rows, the rest apart
    for shape in [(6144, 6144, 6144), (4352, 4352, 2048), (4104, 4096, 2048), (4200, 4352, 1024)]:
        v, rows, rest = plan(*shape)
        assert names[v] == "mfma16_256x256x64_w4_r5_persistent_lean", shape
        assert 0 < rows < shape[0] and rows % 256 == 0 and 0 <= rest < len(names), shape
        # the most whole tile rows that fit in w waves of 256 tiles
        tiles_n = (shape[1] + 255) // 256
        r = rows // 256
        w = -(-r * tiles_n // 256)
        assert (r + 1) * tiles_n > w * 256, shape
        assert v == binding.gemm_nt_f16_select(*shape)
    assert plan(64, 64, 7) == (binding.gemm_nt_f16_select(64, 64, 7), 64, -1)
    assert plan(-1, 4, 4)[0] == -1


def test_no_kernel_uses_scratch_or_spills(lib):
    """The build records every kernel's resource usage (the compiler's
    kernel-resource-usage remarks) beside the library and refuses to
    produce a library in which any kernel spills; check the record of the
    library that is loaded: every kernel present, none with scratch."""
    import json

    from dense_fp16_gemm_04_amd import build

    if not os.path.exists(build.RESOURCES):
        build.build()
    with open(build.RESOURCES) as f:
        kernels = json.load(f)["kernels"]
    # every kernel family the launch plan can run is in the record (a
    # variant may instantiate more than one kernel: the persistent ones
    # carry their one-tile fallback)
    assert len(kernels) >= 10
    for family in ("gemm_nt_f16_ordered_persist", "gemm_nt_f16_ordered", "gemm_nt_f16_mfma", "gemm_nt_f16_simple"):
        assert any(family in k for k in kernels), family
    assert build.spilling(kernels) == []
    for name, r in kernels.items():
        assert r["scratch_bytes_per_lane"] == 0 and r["vgpr_spill"] == 0 and r["sgpr_spill"] == 0, name
        assert r["vgprs"] + r["agprs"] <= 512 and r["lds_bytes"] <= 160 * 1024, name
    # the 8-wave persistent kernels (2 x 4 waves) run two waves per SIMD
    persist8 = [k for k in kernels if "ordered_persist" in k and "Li256ELi256ELi64ELi2ELi4E" in k]
    assert persist8 and all(kernels[k]["waves_per_simd"] >= 2 for k in persist8)


def test_spill_gate_flags_a_spilling_kernel():
    """The gate's parser on remarks in the compiler's format, one kernel
    clean and one with scratch and spilled registers."""
    from dense_fp16_gemm_04_amd import build

    text = "\n".join([
        "k.hip:10:1: remark: Function Name: clean_kernel [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:10:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:10:1: remark:     AGPRs: 128 [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:10:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]",
        "   10 | {",
        "k.hip:20:1: remark: Function Name: spilling_kernel [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:20:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:20:1: remark:     ScratchSize [bytes/lane]: 44 [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:20:1: remark:     VGPRs Spill: 10 [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:20:1: remark:     Occupancy [waves/SIMD]: 1 [-Rpass-analysis=kernel-resource-usage]",
    ])
    k = build.parse_resource_usage(text)
    assert k["clean_kernel"]["vgprs"] == 128 and k["clean_kernel"]["scratch_bytes_per_lane"] == 0
    assert k["spilling_kernel"]["scratch_bytes_per_lane"] == 44 and k["spilling_kernel"]["waves_per_simd"] == 1
    assert build.spilling(k) == ["spilling_kernel"]
