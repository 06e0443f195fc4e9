"""The rate the board sustains under its power limit for each part of the
default kernel's K loop, beside the GEMM itself.

An MI355X holds its engine clock at the level its power limit allows under
the load it runs, so what a kernel reaches depends on the energy of each
instruction it issues as well as on how densely it issues MFMAs.  The power
probe (``csrc/power_probe.hip``, its own library) replays the default
kernel's K loop on every CU one part at a time: MFMAs alone (with zero
fragments, then with Gaussian ones at the workload's scale), then the LDS
fragment reads, the global->LDS loads and the barrier of the real loop.  Each
row runs back to back for --settle seconds, then for a --window of seconds
while a child process samples the engine clock and board power with amd-smi
(``clock.py``); the last row is the GEMM itself, the library's own plan on
the workload, measured the same way.  The chip drifts over a run, so the
rows run in --passes passes, alternately forward and backward, and each
row reports the mean of its passes.

The percentage of the peak at the clock is the share of cycles in which the
matrix cores worked: every flop of a row is an MFMA's, and the peak at clock
f is 1024 SIMDs x 1024 flop per cycle x f.

Run (needs a GPU):

    python -m dense_fp16_gemm_04_amd.power_ceiling [--window 3] [--settle 1] [--workload square_8192]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
if __package__ in (None, ""):
    sys.path.insert(0, os.path.dirname(HERE))

from dense_fp16_gemm_04_amd import clock  # noqa: E402

PROBE_LIB = os.path.join(HERE, "libpower_probe.so")
# 256 CUs x 4096 dense fp16 flop per clock per CU x 2.4 GHz
PEAK_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
MFMA_FLOP = 2 * 16 * 16 * 32  # one v_mfma_f32_16x16x32_f16

ROWS = [
    ("mfma_zero_data", "MFMAs only, fragments of zeros"),
    ("mfma", "MFMAs only, Gaussian fragments at the workload's scale"),
    ("mfma_lds_reads", "MFMAs + 32 fragment reads from LDS per 128 MFMAs"),
    ("mfma_loads", "MFMAs + 16 global->LDS loads per 128 MFMAs (L2-resident), no reads"),
    ("mfma_lds_reads_loads", "MFMAs + the reads + the loads"),
    ("k_loop_mix", "MFMAs + reads + loads + one barrier per 128 MFMAs: the default kernel's K-loop mix"),
    ("mfma32", "MFMAs only as 32x32x16 (64 per step, the same flops), Gaussian fragments"),
    ("mfma_vgpr_loads", "MFMAs + the same 16 loads per 128 MFMAs into VGPRs (the B fragments), no LDS"),
]


def load_probe():
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError("libpower_probe.so is not built (%s); run "
                           "`python -c 'import __graft_entry__ as g; g.build()'`" % PROBE_LIB)
    lib = ctypes.CDLL(PROBE_LIB)
    lib.power_probe_mode_count.restype = ctypes.c_int32
    lib.power_probe_mode_name.restype = ctypes.c_char_p
    lib.power_probe_mode_name.argtypes = [ctypes.c_int32]
    lib.power_probe_launch.restype = ctypes.c_int
    lib.power_probe_launch.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    return lib


def probe_modes(lib) -> list:
    return [lib.power_probe_mode_name(i).decode() for i in range(lib.power_probe_mode_count())]


def table(records) -> str:
    """Markdown table of the rows' records (dicts with name, what, tflops,
    sclk_mhz_median, power_w_mean, pct_of_peak_at_sclk)."""
    base = next((r["tflops"] for r in records if r["name"] == "mfma" and r.get("tflops")), None)
    out = ["| row | what runs | TFLOP/s | each pass | % of the 2516.6 peak | engine MHz (median) | board W (mean) | "
           "matrix cores busy (% of the peak at that clock) | vs MFMAs only |",
           "|---|---|---|---|---|---|---|---|---|"]
    for r in records:
        if r.get("tflops") is None:
            out.append("| `%s` | %s | - | - | - | - | - | - | - |" % (r["name"], r["what"]))
            continue
        mhz = r.get("sclk_mhz_median")
        each = " / ".join("%.1f" % t for t in r.get("tflops_passes", [r["tflops"]]) if t is not None)
        out.append("| `%s` | %s | %.1f | %s | %.1f%% | %s | %s | %s | %s |" % (
            r["name"], r["what"], r["tflops"], each, 100 * r["tflops"] / PEAK_TFLOPS,
            "%.0f" % mhz if mhz else "-",
            "%.0f" % r["power_w_mean"] if r.get("power_w_mean") else "-",
            "%.1f%%" % r["pct_of_peak_at_sclk"] if r.get("pct_of_peak_at_sclk") else "-",
            "%+.1f%%" % (100 * (r["tflops"] / base - 1)) if base else "-"))
    return "\n".join(out)


def timed_only(seconds, step, stream, flops):
    """The rate alone, when amd-smi is not available."""
    import torch
    s0 = torch.cuda.Event(enable_timing=True)
    e0 = torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step()
        n += 20
        torch.cuda.synchronize()
    e0.record(stream)
    torch.cuda.synchronize()
    ms = s0.elapsed_time(e0) / n
    return {"seconds": seconds, "launches": n, "ms_per_launch": ms, "tflops": flops / (ms * 1e-3) / 1e12}


def combine(name, what, passes) -> dict:
    """One row's record from its passes: the means of the rate, the median
    clock, the power and the busy share; each pass's rate kept."""
    out = {"name": name, "what": what, "passes": passes,
           "tflops_passes": [r.get("tflops") for r in passes]}
    for key in ("tflops", "sclk_mhz_median", "power_w_mean", "pct_of_peak_at_sclk"):
        vals = [r[key] for r in passes if r.get(key) is not None]
        out[key] = sum(vals) / len(vals) if len(vals) == len(passes) else None
    return out


def order(n: int, passes: int) -> list:
    """Row indices in run order: forward, then backward, and so on, so that a
    drift linear in time weighs every row's mean alike."""
    seq = []
    for p in range(passes):
        seq += list(range(n)) if p % 2 == 0 else list(range(n - 1, -1, -1))
    return seq


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--settle", type=float, default=1.0, metavar="SECONDS")
    p.add_argument("--window", type=float, default=3.0, metavar="SECONDS")
    p.add_argument("--passes", type=int, default=2,
                   help="passes over the rows, alternately forward and backward (the rows' means are reported)")
    p.add_argument("--steps", type=int, default=512, help="probe steps (128 MFMAs per wave each) per launch")
    p.add_argument("--workload", default="square_8192")
    p.add_argument("--json", default="", help="also write the records to this file")
    args = p.parse_args(argv)
    if args.steps < 1 or args.window <= 0 or args.settle < 0 or args.passes < 1:
        print("power_ceiling: --steps and --passes must be >= 1, --window > 0, --settle >= 0", file=sys.stderr)
        return 2
    # the sampler starts before this process touches the GPU, and serves every window
    sampler = clock.start_sampler()
    try:
        return measure(args, sampler)
    finally:
        clock.stop_sampler(sampler)


def measure(args, sampler) -> int:
    import torch

    from dense_fp16_gemm_04_amd import binding, workloads

    lib = load_probe()
    names = probe_modes(lib)
    if names != [n for n, _ in ROWS]:
        raise RuntimeError("probe modes %s do not match the rows %s" % (names, [n for n, _ in ROWS]))
    if not torch.cuda.is_available():
        print("power_ceiling: needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(0)
    w = workloads.by_name(args.workload)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    std = float(w.K) ** -0.25 if w.K > 0 else 1.0  # the workload's entries: N(0, K**-0.5)
    src = (torch.randn(32 << 20, device=dev, generator=g) * std).to(torch.float16)  # 64 MiB
    grid = props.multi_processor_count
    sink = torch.empty(grid * 256, device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream()
    a, b = workloads.workload_inputs(w)
    A = torch.from_numpy(a).to(dev)
    B = torch.from_numpy(b).to(dev)
    C = torch.empty(w.M, w.N, device=dev, dtype=torch.float16)
    kernel = binding.gemm_nt_f16_config_name(w.M, w.N, w.K)

    def run_row(step, flops, label):
        step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.settle:
            for _ in range(10):
                step()
            torch.cuda.synchronize()
        if sampler is not None and sampler.poll() is None:
            rec = clock.clock_window(sampler, args.window, step, stream, flops, props, PEAK_TFLOPS,
                                     label="power_ceiling: " + label, keep=True)
            if rec is not None:
                return rec
        rec = timed_only(args.window, step, stream, flops)
        print("power_ceiling: %s: %.1f TFLOP/s (no clock samples)" % (label, rec["tflops"]), file=sys.stderr,
              flush=True)
        return rec

    def probe_step(m, name):
        def step():
            rc = lib.power_probe_launch(m, src.data_ptr(), src.numel() * 2, sink.data_ptr(), grid, args.steps,
                                        ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError("power_probe_launch(%s) returned hipError_t %d" % (name, rc))
        return step

    def gemm():
        binding.gemm_nt_f16(A, B, C)

    probe_flops = float(grid) * 4 * args.steps * 128 * MFMA_FLOP
    items = [(name, what, probe_step(m, name), probe_flops) for m, (name, what) in enumerate(ROWS)]
    items.append(("gemm", "the GEMM on %s (%d x %d x %d), the library's plan: `%s`" % (w.name, w.M, w.N, w.K, kernel),
                  gemm, 2.0 * w.M * w.N * w.K))
    runs = [[] for _ in items]
    for i in order(len(items), args.passes):
        name, _, step, flops = items[i]
        runs[i].append(run_row(step, flops, name))
    records = [combine(name, what, runs[i]) for i, (name, what, _, _) in enumerate(items)]
    print(table(records))
    print(json.dumps({"workload": w.name, "grid": grid, "steps": args.steps, "passes": args.passes,
                      "records": records}))
    if args.json:
        with open(args.json, "w") as f:
            json.dump(records, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
