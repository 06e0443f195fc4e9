#!/usr/bin/env python3
"""Throughput of fp16 C = A * B^T on one MI355X, as one JSON line.

One step is one call of ``gemm_nt_f16`` (the whole path: tile scheduling,
global->LDS staging, MFMA loop, epilogue) on M = N = K = 8192 by default, with
seeded synthetic fp16 inputs already resident in HBM.

The engine clock is power-managed: from idle, the first launches run at a
high clock, the clock then dips below the level it settles at and recovers
over tens of milliseconds.  So before the --warmup steps the benchmark
launches back to back for --settle seconds (untimed), and the --steps timed
launches, bracketed by events on the launch stream, measure the rate the
chip sustains.  After them it repeats the pages' own protocol ("6. Four
Consumers, FP16 Accumulation, and a TMA Epilogue", section "Performance": a
cool-down pause, then 30 back-to-back launches) and reports it beside the
result as ``pages_protocol``, never as the result.

The line carries a ``roofline`` object for the MFMA kernel (algorithmic
2*M*N*K flop per launch over the measured launch time, against the dense
fp16 MFMA peak) and a ``cpu_baseline`` object: the CPU oracle timed on a
bounded slab of the same product on this host's cores.  Last comes a
``clock_window``: three seconds of back-to-back launches while amd-smi, run
from a child process started before this one touches the GPU, samples the
engine clock and board power, so the result can also be read against the
peak at the clock the chip holds under this load.
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
# Bytes per launch between the L2s and the memory controller, from two
# rocprofv3 --pmc runs of this benchmark: FETCH_SIZE x 2.000 + WRITE_SIZE x
# 1.000 (KiB per dispatch), the factors read off a plain 1 GiB device copy in
# the same process; TCC_EA0_RDREQ_DRAM_32B and TCC_EA0_WRREQ_64B give the same
# bytes.  The memory-side cache sits behind that point, so this bounds HBM
# traffic from above.  Valid only for the kernel source it was measured on
# (source_digest: comments and whitespace aside): null once that changes.
TRAFFIC = {"workload": "square_8192", "kernel": "mfma16_256x256x64_w4_r5_persistent_lean", "bytes": 1.841e9,
           "source_sha256_16": "1b96a223308de091"}
SOURCE = os.path.join(ROOT, "dense_fp16_gemm_04_amd", "csrc", "gemm_nt_f16.hip")


def source_digest() -> str:
    """SHA-256 (16 hex digits) of the kernel source's code: comments removed
    and whitespace collapsed, so an edit to a comment keeps the record."""
    import hashlib
    import re
    try:
        with open(SOURCE, encoding="utf-8") as f:
            text = f.read()
    except OSError:
        return ""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_configs():
    """The oracle on every workload of five configurations, whole products,
    on this host's cores (capped as for the baseline), and on one thread for
    the two smallest: wall time and GFLOP/s each."""
    import oracle
    from dense_fp16_gemm_04_amd import workloads

    threads = cpu_threads()
    rows = []
    for w in workloads.WORKLOADS[:5]:
        a, b = workloads.workload_inputs(w)
        for t in ([threads, 1] if w.M * w.N * w.K <= 1 << 30 else [threads]):
            t0 = time.perf_counter()
            oracle.gemm_nt(a, b, threads=t)
            dt = time.perf_counter() - t0
            rows.append({"workload": w.name, "threads": t, "seconds": dt, "gflops": w.flops / dt / 1e9})
            log("bench: oracle on %s, %d thread(s): %.3f s, %.2f GFLOP/s" % (w.name, t, dt, w.flops / dt / 1e9))
    return {"cpu_model": cpu_model(), "nproc": os.cpu_count(), "threads": threads, "runs": rows}


def under_profiler() -> bool:
    """True inside rocprofv3 (which sets ROCPROF_* variables): its preloaded
    library follows every child process, so the clock window, which starts
    children, is skipped there."""
    return any(k.startswith("ROCPROF") for k in os.environ)


# the amd-smi sampler child and the clock window live in the package (the
# power-ceiling probe uses them too); bench.py --smi-sampler runs the child
from dense_fp16_gemm_04_amd import clock as _clock  # noqa: E402
from dense_fp16_gemm_04_amd.clock import samples_of, smi_command, smi_sampler, tell  # noqa: E402,F401


def clock_window(sampler, seconds, step, stream, flops, props):
    """Back-to-back launches for `seconds` while the sampler child polls
    amd-smi: the engine clock and board power under sustained load, and the
    fraction of the peak at that clock."""
    return _clock.clock_window(sampler, seconds, step, stream, flops, props, PEAK_TFLOPS)


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="square_8192")
    p.add_argument("--variant", default="-1",
                   help="kernel variant, by index or name (-1: the library's own launch plan)")
    p.add_argument("--settle", type=float, default=1.0, metavar="SECONDS",
                   help="launch back to back for this long before the warm-up steps (untimed), so the "
                        "timed window sees the clock the chip sustains")
    p.add_argument("--cooldown", type=float, default=0.0,
                   help="seconds idle between the warm-up and the timed window (the pages' protocol "
                        "pauses 3 s; it is also reported separately, see --pages-protocol)")
    p.add_argument("--pages-protocol", type=float, default=3.0, metavar="SECONDS",
                   help="after the timed window, pause this long and time 30 back-to-back launches, as "
                        "the pages do; reported beside the result (0: skip)")
    p.add_argument("--cpu-rows", type=int, default=8192,
                   help="rows of A in the oracle's timed slab (0 skips the CPU baseline)")
    p.add_argument("--throttle-check", type=int, default=0, metavar="N",
                   help="after the timed window, time N more back-to-back launches (0: skip); "
                        "reported beside the result, never as the result")
    p.add_argument("--clock-window", type=float, default=3.0, metavar="SECONDS",
                   help="after the throttle check, launch back to back for this long while sampling "
                        "the engine clock and board power with amd-smi (0: skip)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after timing, run one plain device copy of this many MiB (a kernel of "
                        "known traffic, to scale hardware byte counters against)")
    p.add_argument("--repeat", type=int, default=1, metavar="R",
                   help="run the measurement in R fresh processes, one after the other, and "
                        "report the median (the pages quote the median of three)")
    p.add_argument("--cpu-configs", action="store_true",
                   help="also time the oracle on every configuration (whole products; about a minute "
                        "more): cpu_baseline.per_config")
    p.add_argument("--smi-sampler", action="store_true", help=argparse.SUPPRESS)
    args = p.parse_args(argv)
    if args.smi_sampler:
        return smi_sampler()

    if args.gpus != 1:
        print("bench.py: this benchmark runs on one GPU only; --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0 or args.repeat < 1:
        print("bench.py: --steps and --repeat must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
    if args.repeat > 1:
        return repeated(args, argv if argv is not None else sys.argv[1:])

    # the clock sampler starts before this process touches the GPU
    sampler = None
    if (args.clock_window > 0 and os.path.exists("/dev/kfd") and not under_profiler()
            and smi_command() is not None):
        sampler = subprocess.Popen([sys.executable, os.path.abspath(__file__), "--smi-sampler"],
                                   stdin=subprocess.PIPE, stdout=subprocess.PIPE, text=True)
    try:
        return measure(args, sampler)
    finally:
        if sampler is not None and sampler.poll() is None:
            sampler.stdin.close()  # end of input: the sampler exits
            try:
                sampler.wait(timeout=60)
            except subprocess.TimeoutExpired:
                sampler.kill()


def measure(args, sampler) -> int:
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
    forced = int(args.variant) if args.variant.lstrip("-").isdigit() else names.index(args.variant)
    if forced >= 0:
        vid, rows, rest = forced, w.M, -1
    else:  # the library's own plan, as gemm_nt_f16 runs it
        vid, rows, rest = binding.gemm_nt_f16_plan(w.M, w.N, w.K)
    vname = names[vid]
    plan = vname if rows == w.M else "%s on rows [0, %d) + %s" % (vname, rows, names[rest])
    log("bench: %s" % plan)

    def step():
        if forced >= 0:
            binding.gemm_nt_f16_ex(ta, tb, out=out, variant=vid)
        else:
            binding.gemm_nt_f16(ta, tb, out=out)

    stream = torch.cuda.current_stream(dev)
    settle = None
    if args.settle > 0:
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.settle:
            for _ in range(10):
                step()
            n += 10
            torch.cuda.synchronize()
        settle = {"seconds": time.perf_counter() - t0, "launches": n,
                  "note": "untimed back-to-back launches before the warm-up steps"}
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.cooldown > 0:
        time.sleep(args.cooldown)

    def window(k):
        """k back-to-back launches between events on the launch stream:
        (ms per launch, host wall seconds)."""
        s0 = torch.cuda.Event(enable_timing=True)
        e0 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        s0.record(stream)
        for _ in range(k):
            step()
        e0.record(stream)
        torch.cuda.synchronize()
        return s0.elapsed_time(e0) / k, time.perf_counter() - t0

    ms, wall = window(args.steps)
    tflops = w.flops / (ms * 1e-3) / 1e12
    log("bench: %.4f ms per launch (%.1f TFLOP/s, %.1f%% of peak); host wall %.4f ms per step"
        % (ms, tflops, 100 * tflops / PEAK_TFLOPS, 1e3 * wall / args.steps))
    if not torch.isfinite(out.float()).all().item():
        print("bench.py: non-finite output", file=sys.stderr)
        return 1

    pages = None
    if args.pages_protocol > 0:
        time.sleep(args.pages_protocol)
        ms_p, _ = window(30)
        pages = {"cooldown_s": args.pages_protocol, "launches": 30, "ms_per_launch": ms_p,
                 "tflops": w.flops / (ms_p * 1e-3) / 1e12,
                 "note": "after an idle pause the clock dips below its settled value for ~20 ms"}
        log("bench: pages' protocol (%.0f s pause, 30 launches): %.4f ms per launch (%.1f TFLOP/s)"
            % (args.pages_protocol, ms_p, pages["tflops"]))

    throttle = None
    if args.throttle_check > 0:
        ms2, _ = window(args.throttle_check)
        throttle = {"launches": args.throttle_check, "ms_per_launch": ms2,
                    "tflops": w.flops / (ms2 * 1e-3) / 1e12,
                    "window": "back-to-back launches after the timed ones"}
        log("bench: next %d launches: %.4f ms per launch (%.1f TFLOP/s)"
            % (args.throttle_check, ms2, throttle["tflops"]))

    clock = None
    if sampler is not None:
        clock = clock_window(sampler, args.clock_window, step, stream, w.flops,
                             torch.cuda.get_device_properties(dev))

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
                    and TRAFFIC["kernel"] == vname and rows == w.M
                    and TRAFFIC["source_sha256_16"] == source_digest() else None),
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
    if settle is not None:
        rec["settle"] = settle
    if pages is not None:
        rec["pages_protocol"] = pages
    if throttle is not None:
        rec["throttle_check"] = throttle
    if clock is not None:
        rec["clock_window"] = clock
    if args.cpu_rows > 0:
        rows = min(args.cpu_rows, w.M)
        log("bench: timing the CPU oracle on %d rows ..." % rows)
        rec["cpu_baseline"] = cpu_baseline(a, b, rows)
        log("bench: oracle %.4g TFLOP/s on %d threads" % (rec["cpu_baseline"]["value"],
                                                           rec["cpu_baseline"]["cores"]))
        if args.cpu_configs:
            rec["cpu_baseline"]["per_config"] = cpu_configs()
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
        if args.cpu_configs:
            rec["cpu_baseline"]["per_config"] = cpu_configs()
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
