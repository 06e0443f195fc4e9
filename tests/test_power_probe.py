"""The power probe: its modes and argument checks, the instruction mix of its
loops against the default kernel's K loop (read from both libraries' gfx950
code objects), and power_ceiling.py's run order and table (no GPU); one
short launch of every mode on the GPU."""
from __future__ import annotations

import ctypes
import os

import pytest

import _isa
from dense_fp16_gemm_04_amd import binding, power_ceiling

HIP_ERROR_INVALID_VALUE = 1
LEAN_SYMBOL = ("gemm_nt_f16_ordered_persist", "ILi256ELi256ELi64ELi2ELi2ELi2ELi1ELi0ELi16EEELi3ELi8ELi16EEE")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(power_ceiling.PROBE_LIB):
        pytest.skip("libpower_probe.so not built")
    return power_ceiling.load_probe()


def test_modes_match_the_rows_of_power_ceiling(lib):
    assert power_ceiling.probe_modes(lib) == [n for n, _ in power_ceiling.ROWS]
    assert lib.power_probe_mode_name(-1) is None
    assert lib.power_probe_mode_name(len(power_ceiling.ROWS)) is None


def test_launch_rejects_arguments_outside_its_ranges(lib):
    """Each call is refused before anything reaches the GPU (the pointers are
    never dereferenced)."""
    fake = ctypes.c_void_p(0x1000)
    mib = 1 << 20
    good = dict(mode=5, src=fake, nbytes=64 * mib, sink=fake, grid=256, steps=4)
    for bad in [dict(mode=-1), dict(mode=len(power_ceiling.ROWS)), dict(src=None), dict(sink=None),
                dict(nbytes=32 * mib), dict(nbytes=96 * mib), dict(nbytes=2048 * mib), dict(grid=0),
                dict(grid=5000), dict(steps=0)]:
        a = {**good, **bad}
        rc = lib.power_probe_launch(a["mode"], a["src"], a["nbytes"], a["sink"], a["grid"], a["steps"], None)
        assert rc == HIP_ERROR_INVALID_VALUE, bad


def test_probe_kernels_do_not_spill(lib):
    """The build gate covers the probe library too: every mode's kernel is
    in its resource record, none with scratch, one wave per SIMD."""
    import json

    from dense_fp16_gemm_04_amd import build

    with open(build.PROBE_RESOURCES) as f:
        kernels = json.load(f)["kernels"]
    assert len(kernels) == len(power_ceiling.ROWS)
    assert build.spilling(kernels) == []
    for name, r in kernels.items():
        assert r["agprs"] == 256 and r["waves_per_simd"] == 1, (name, r)


def _probe_loop(asm, flags):
    found = _isa.loops(_isa.kernel(asm, ("power_probe_kernelILi%dE" % flags,)), 128)
    assert len(found) == 1, (flags, found)
    return found[0]


def test_full_mix_issues_what_the_default_k_loop_issues(tmp_path):
    """Per 128 MFMAs the probe's full mix issues the reads, loads and barrier
    of the default kernel's five-step K loop (640 MFMAs), and almost no
    other arithmetic; the partial modes issue only their parts."""
    (tmp_path / "probe").mkdir()
    (tmp_path / "gemm").mkdir()
    probe = _isa.disassemble(power_ceiling.PROBE_LIB, tmp_path / "probe")
    gemm = _isa.disassemble(binding.library_path(), tmp_path / "gemm")
    lean = _isa.loops(_isa.kernel(gemm, LEAN_SYMBOL), 640)
    assert lean
    mix = _probe_loop(probe, 7)
    for k in ("ds_read_b128", "buffer_load_dwordx4", "s_barrier"):
        assert 5 * mix[k] == lean[0][k], (k, mix[k], lean[0][k])
    vector = sum(v for k, v in mix.items() if k.startswith("v_") and not k.startswith("v_mfma"))
    scalar = sum(v for k, v in mix.items() if k.startswith("s_") and k not in ("s_waitcnt", "s_barrier"))
    assert vector <= 1 and scalar <= 16, mix
    parts = {8: (0, 0), 0: (0, 0), 1: (32, 0), 2: (0, 16), 3: (32, 16)}
    for flags, (reads, loads) in parts.items():
        body = _probe_loop(probe, flags)
        assert body["ds_read_b128"] == reads and body["buffer_load_dwordx4"] == loads, (flags, body)
        assert body["s_barrier"] == 0, (flags, body)
    direct = _probe_loop(probe, 32)
    assert direct["buffer_load_dwordx4"] == 16 and direct["ds_read_b128"] == 0 and direct["s_barrier"] == 0, direct
    wide = _isa.loops(_isa.kernel(probe, ("power_probe_mfma32",)), 64)
    assert len(wide) == 1 and wide[0]["v_mfma_f32_32x32x16_f16"] == 64, wide
    assert not [k for k in wide[0] if k.startswith(("v_", "ds_", "buffer_")) and not k.startswith("v_mfma")], wide


def test_rows_run_forward_then_backward():
    assert power_ceiling.order(3, 1) == [0, 1, 2]
    assert power_ceiling.order(3, 2) == [0, 1, 2, 2, 1, 0]
    assert power_ceiling.order(2, 3) == [0, 1, 1, 0, 0, 1]


def test_a_row_reports_the_mean_of_its_passes():
    passes = [{"tflops": 1500.0, "sclk_mhz_median": 1650.0, "power_w_mean": 1300.0, "pct_of_peak_at_sclk": 89.0},
              {"tflops": 1540.0, "sclk_mhz_median": 1690.0, "power_w_mean": 1310.0, "pct_of_peak_at_sclk": 90.0}]
    r = power_ceiling.combine("k_loop_mix", "all", passes)
    assert r["tflops"] == 1520.0 and r["sclk_mhz_median"] == 1670.0 and r["power_w_mean"] == 1305.0
    assert r["pct_of_peak_at_sclk"] == 89.5 and r["tflops_passes"] == [1500.0, 1540.0]
    # a pass without clock samples leaves the clock columns empty, the rate not
    r = power_ceiling.combine("k_loop_mix", "all", [passes[0], {"tflops": 1540.0}])
    assert r["tflops"] == 1520.0 and r["sclk_mhz_median"] is None


def test_table_reads_against_mfma_only():
    recs = [{"name": "mfma_zero_data", "what": "zeros", "tflops": 2400.0, "tflops_passes": [2390.0, 2410.0],
             "sclk_mhz_median": 2390.0, "power_w_mean": 700.0, "pct_of_peak_at_sclk": 96.0},
            {"name": "mfma", "what": "Gaussian", "tflops": 1800.0, "sclk_mhz_median": 1870.0,
             "power_w_mean": 1330.0, "pct_of_peak_at_sclk": 94.0},
            {"name": "k_loop_mix", "what": "all", "tflops": 1500.0},
            {"name": "gemm", "what": "the GEMM"}]
    t = power_ceiling.table(recs).splitlines()
    assert len(t) == 2 + len(recs)
    assert t[0].count("|") == t[2].count("|") == 10
    assert "| 2400.0 | 2390.0 / 2410.0 | 95.4% | 2390 | 700 | 96.0% | +33.3% |" in t[2]
    assert "| 1800.0 | 1800.0 | 71.5% |" in t[3] and t[3].endswith("| +0.0% |")
    assert "| 1500.0 | 1500.0 | 59.6% | - | - | - | -16.7% |" in t[4]
    assert t[5].endswith("| the GEMM | - | - | - | - | - | - | - |")


def test_power_ceiling_rejects_bad_arguments_before_starting_anything(capsys):
    for bad in (["--steps", "0"], ["--window", "0"], ["--settle", "-1"], ["--passes", "0"]):
        assert power_ceiling.main(bad) == 2, bad
    assert "power_ceiling:" in capsys.readouterr().err


@pytest.mark.gpu
def test_every_mode_launches_and_finishes(lib):
    import torch
    dev = torch.device("cuda:0")
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    src = (torch.randn(32 << 20, device=dev) * 0.1).to(torch.float16)
    sink = torch.full((grid * 256,), float("nan"), device=dev)
    stream = torch.cuda.current_stream()
    for m, (name, _) in enumerate(power_ceiling.ROWS):
        print("power probe mode %s" % name, flush=True)
        rc = lib.power_probe_launch(m, src.data_ptr(), src.numel() * 2, sink.data_ptr(), grid, 8,
                                    ctypes.c_void_p(stream.cuda_stream))
        assert rc == 0, name
        torch.cuda.synchronize()
        assert torch.isfinite(sink).all(), name
        sink.fill_(float("nan"))
