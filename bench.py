#!/usr/bin/env python3
"""Throughput of fp16 C = A * B^T on one MI355X, as one JSON line.

One step is one call of ``gemm_nt_f16`` (the whole path: tile scheduling,
global->LDS staging, MFMA loop, epilogue) on M = N = K = 8192 by default, with
seeded synthetic fp16 inputs already resident in HBM.  Method, following the
pages' own ("6. Four Consumers, FP16 Accumulation, and a TMA Epilogue",
section "Performance"): warm-up launches, a cool-down pause, then a window of
back-to-back launches bracketed by events on the launch stream.

The line carries a ``roofline`` object for the MFMA kernel (algorithmic
2*M*N*K flop per launch over the measured launch time, against the dense
fp16 MFMA peak) and a ``cpu_baseline`` object: the CPU oracle timed on a
bounded slab of the same product on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOP/s fp16 GEMM C=A·Bᵀ at M=N=K=8192; % of MI355X dense fp16 MFMA peak"
# 256 CUs x 4096 dense fp16 flop per clock per CU x 2.4 GHz (AMD's 2.5 PFLOP/s)
PEAK_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
# HBM bytes per launch measured with rocprofv3 (FETCH_SIZE x 2.000 plus
# WRITE_SIZE x 1.000, the factors read off a plain 1 GiB device copy) for one
# kernel on one workload.  Reported only for that pair; reset to None when the
# kernel changes.
TRAFFIC = {"workload": "square_8192", "kernel": "mfma16_256x256x64_w8_r5_l4_persistent", "bytes": 1.812e9}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, 16))


def cpu_baseline(a, b, rows: int):
    """Time the oracle on rows [0, rows) of A against all of B."""
    import oracle

    threads = cpu_threads()
    a_s = a[:rows]
    t0 = time.perf_counter()
    oracle.gemm_nt(a_s, b, threads=threads)
    dt = time.perf_counter() - t0
    flops = 2.0 * a_s.shape[0] * b.shape[0] * a.shape[1]
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "rows [0, %d) of A against all %d rows of B, K=%d (%.3g flop, %.1f s)"
                  % (a_s.shape[0], b.shape[0], a.shape[1], flops, dt),
    }


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="square_8192")
    p.add_argument("--variant", type=int, default=-1, help="kernel variant index (-1: automatic)")
    p.add_argument("--cooldown", type=float, default=3.0, help="seconds idle before the timed window")
    p.add_argument("--cpu-rows", type=int, default=8192,
                   help="rows of A in the oracle's timed slab (0 skips the CPU baseline)")
    p.add_argument("--throttle-check", type=int, default=100, metavar="N",
                   help="after the timed window, time N more back-to-back launches (0: skip); "
                        "reported beside the result, never as the result")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after timing, run one plain device copy of this many MiB (a kernel of "
                        "known traffic, to scale hardware byte counters against)")
    p.add_argument("--repeat", type=int, default=1, metavar="R",
                   help="run the measurement in R fresh processes, one after the other, and "
                        "report the median (the pages quote the median of three)")
    args = p.parse_args(argv)

    if args.gpus != 1:
        print("bench.py: this benchmark runs on one GPU only; --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0 or args.repeat < 1:
        print("bench.py: --steps and --repeat must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
    if args.repeat > 1:
        return repeated(args, argv if argv is not None else sys.argv[1:])

    import numpy as np
    import torch

    from dense_fp16_gemm_04_amd import binding, workloads

    if not os.path.exists(binding.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    binding.load()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1

    w = workloads.by_name(args.workload)
    dev = torch.device("cuda:0")
    log("bench: generating %s (M=%d N=%d K=%d, seed %d)" % (w.name, w.M, w.N, w.K, w.seed))
    a, b = workloads.workload_inputs(w)
    ta = torch.from_numpy(a).to(dev)
    tb = torch.from_numpy(b).to(dev)
    out = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    names = binding.variants()
    if args.variant >= 0:
        vid, rows, rest = args.variant, w.M, -1
    else:  # the library's own plan, as gemm_nt_f16 runs it
        vid, rows, rest = binding.gemm_nt_f16_plan(w.M, w.N, w.K)
    vname = names[vid]
    plan = vname if rows == w.M else "%s on rows [0, %d) + %s" % (vname, rows, names[rest])
    log("bench: %s" % plan)

    def step():
        if args.variant >= 0:
            binding.gemm_nt_f16_ex(ta, tb, out=out, variant=vid)
        else:
            binding.gemm_nt_f16(ta, tb, out=out)

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.cooldown > 0:
        time.sleep(args.cooldown)

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    tflops = w.flops / (ms * 1e-3) / 1e12
    log("bench: %.4f ms per launch (%.1f TFLOP/s, %.1f%% of peak); host wall %.4f ms per step"
        % (ms, tflops, 100 * tflops / PEAK_TFLOPS, 1e3 * wall / args.steps))
    if not torch.isfinite(out.float()).all().item():
        print("bench.py: non-finite output", file=sys.stderr)
        return 1

    # The engine clock is power-managed: after the idle pause the first
    # launches run fast, the clock then dips below its settled value and
    # recovers over ~20 ms.  A longer back-to-back window shows where it
    # settles; the result above keeps the 30-launch window of the protocol.
    throttle = None
    if args.throttle_check > 0:
        s2 = torch.cuda.Event(enable_timing=True)
        e2 = torch.cuda.Event(enable_timing=True)
        s2.record(stream)
        for _ in range(args.throttle_check):
            step()
        e2.record(stream)
        torch.cuda.synchronize()
        ms2 = s2.elapsed_time(e2) / args.throttle_check
        throttle = {"launches": args.throttle_check, "ms_per_launch": ms2,
                    "tflops": w.flops / (ms2 * 1e-3) / 1e12,
                    "window": "back-to-back launches right after the timed ones"}
        log("bench: next %d launches: %.4f ms per launch (%.1f TFLOP/s)"
            % (args.throttle_check, ms2, throttle["tflops"]))

    if args.copy_calibration > 0:
        n = args.copy_calibration * 2 ** 20 // 2
        src = torch.ones(n, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("bench: copied %d MiB device to device (reads and writes %d bytes each)"
            % (args.copy_calibration, 2 * n))
        del src, dst

    roof = {
        "bound": "mfma",
        "achieved": tflops,
        "peak": PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": tflops / PEAK_TFLOPS,
        "traffic": (TRAFFIC["bytes"] if TRAFFIC and TRAFFIC["workload"] == w.name
                    and TRAFFIC["kernel"] == vname and rows == w.M else None),
    }
    rec = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "seed": w.seed,
                   "inputs": "iid N(0, 1/sqrt(K)) fp16, K-major", "accumulate": "f32",
                   "output": "f16", "kernel": plan, "pct_of_peak": 100 * tflops / PEAK_TFLOPS},
        "roofline": roof,
    }
    if throttle is not None:
        rec["throttle_check"] = throttle
    if args.cpu_rows > 0:
        rows = min(args.cpu_rows, w.M)
        log("bench: timing the CPU oracle on %d rows ..." % rows)
        rec["cpu_baseline"] = cpu_baseline(a, b, rows)
        log("bench: oracle %.4g TFLOP/s on %d threads" % (rec["cpu_baseline"]["value"],
                                                           rec["cpu_baseline"]["cores"]))
    print(json.dumps(rec), flush=True)
    return 0


def repeated(args, argv) -> int:
    """The measurement in args.repeat fresh child processes, one after the
    other (this process never touches the GPU); the record of the median
    run, with every run's value beside it."""
    child = []
    skip = False
    for x in argv:  # drop --repeat and --cpu-rows from the child's arguments
        if skip:
            skip = False
            continue
        if x in ("--repeat", "--cpu-rows"):
            skip = True
            continue
        if x.startswith("--repeat=") or x.startswith("--cpu-rows="):
            continue
        child.append(x)
    recs = []
    for i in range(args.repeat):
        log("bench: process %d of %d" % (i + 1, args.repeat))
        res = subprocess.run([sys.executable, os.path.abspath(__file__), *child, "--repeat", "1",
                              "--cpu-rows", "0"], stdout=subprocess.PIPE, text=True)
        if res.returncode != 0:
            print("bench.py: run %d failed (%d)" % (i + 1, res.returncode), file=sys.stderr)
            return res.returncode
        recs.append(json.loads(res.stdout.strip().splitlines()[-1]))
    values = [r["value"] for r in recs]
    rec = sorted(recs, key=lambda r: r["value"])[len(recs) // 2]
    rec["repeat"] = {"processes": args.repeat, "values": values, "range": [min(values), max(values)],
                     "reported": "median"}
    if args.cpu_rows > 0:
        from dense_fp16_gemm_04_amd import workloads
        w = workloads.by_name(args.workload)
        a, b = workloads.workload_inputs(w)
        rows = min(args.cpu_rows, w.M)
        log("bench: timing the CPU oracle on %d rows ..." % rows)
        rec["cpu_baseline"] = cpu_baseline(a, b, rows)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
