"""Ablation ladder: the design steps of the pages, re-made for CDNA4, timed
and counted on one workload.

The pages build their kernel in steps ("0. A Minimal Hopper Matmul" through
"6. Four Consumers, FP16 Accumulation, and a TMA Epilogue", section
"Summary"): a first tiled kernel whose copy and math never overlap, then a
multi-stage ring, producer/consumer warps, a larger tile, more consumers,
a grouped tile raster and a staged epilogue.  The rungs below take the same
steps with this library's kernels, each one design choice away from the
rung before it, and R8 adds one of CDNA4's own (one wave per SIMD with a K
loop free of scalar and vector arithmetic; the side row without that loop
separates its two changes); the side rows change one thing of R7 or R8.

Run (needs a GPU):

    python -m dense_fp16_gemm_04_amd.ladder [--workload square_8192]

Each kernel is launched back to back for --settle seconds, then --warmup
and --launches timed launches (events on the launch stream), so every row
is read at the clock the chip sustains under that kernel.  Counters come
from separate runs under rocprofv3, one counter set per run, with no settle
(every launch is then a counted dispatch), summarised without a GPU:

    rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_ANY \\
        SQ_INSTS_LDS SQ_INSTS_SALU SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE \\
        --output-format csv -d DIR1 -o run -- \\
        python3 -m dense_fp16_gemm_04_amd.ladder --settle 0 --warmup 1 --launches 2
    rocprofv3 --pmc GRBM_GUI_ACTIVE TCC_EA0_RDREQ_DRAM_32B_sum TCC_EA0_WRREQ_sum \\
        TCC_EA0_WRREQ_64B_sum --output-format csv -d DIR2 -o run -- \\
        python3 -m dense_fp16_gemm_04_amd.ladder --settle 0 --warmup 1 --launches 2
    rocprofv3 --pmc GRBM_GUI_ACTIVE TCC_HIT_sum TCC_REQ_sum --output-format csv -d DIR3 \\
        -o run -- python3 -m dense_fp16_gemm_04_amd.ladder --settle 0 --warmup 1 --launches 2
    python -m dense_fp16_gemm_04_amd.ladder --summarize DIR1 DIR2 DIR3 --warmup 1 --launches 2 \\
        [--times ladder.json]

The summary assigns GEMM dispatches to rows in launch order, which this
script fixes: every row gets warmup + launches dispatches, in table order,
and nothing else launches a kernel whose name contains gemm_nt_f16.

Counter readings (GRBM_GUI_ACTIVE counts cycles on each of the 8 XCDs; the
matrix-core busy cycles, per SIMD, are over 1024 SIMDs): MFMA busy =
SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 * 1024), a fraction of
cycles whatever the clock; the implied clock is the one at which the timed
rate and that fraction agree, TFLOP/s / (busy * 1048.576 TFLOP/s per GHz)
(counted dispatches run one at a time, not at the sustained clock);
bytes read beyond L2 = 32 * TCC_EA0_RDREQ_DRAM_32B_sum and bytes written =
64 * TCC_EA0_WRREQ_64B_sum + 32 * (TCC_EA0_WRREQ_sum - TCC_EA0_WRREQ_64B_sum),
factors read off a plain 1 GiB device copy, which these counters report as
exactly 1 GiB read and 1 GiB written.  The memory-side cache (MALL) sits behind that point, so
these are requests that leave the L2s for the memory controller: an upper
bound on HBM traffic.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# (variant, rung, what it adds to the rung above; the pages' step it mirrors)
LADDER = [
    ("simple_f32_per_element", "R0",
     "one thread per output, fp32 FMAs from global memory: no tiling, no matrix cores"),
    ("mfma16_128x128x64_w4_s1_one_per_cu", "R1",
     "128x128 tiles in LDS, 4 waves of 16x16x32 MFMAs, one workgroup per CU; one stage: "
     "load, wait, compute (V0: the copy runs, then everyone waits)"),
    ("mfma16_128x128x64_w4_s3", "R2",
     "3-stage ring: the loads of later steps overlap the MFMAs (V2's multi-stage ring)"),
    ("mfma16_128x128x64_w8_s3_l4_ordered", "R3",
     "8 waves, 4 of them issue the loads, every instruction placed by hand "
     "(V3's warp specialization: on CDNA4 the loading waves also compute)"),
    ("mfma16_256x128x64_w8x_s3_l4_ordered", "R4",
     "256x128 tile: more reuse per loaded byte (V5's 128x256 with two consumer groups)"),
    ("mfma16_256x256x64_w8_s2_l4_ordered", "R5",
     "256x256 tile, 2-stage ring (V6's tile; the accumulators fill half the register file)"),
    ("mfma16_256x256x64_w8_r5_l4_ordered", "R6",
     "five single-operand LDS slots: a step's loads spread over the whole step"),
    ("mfma16_256x256x64_w8_r5_l4_persistent", "R7",
     "persistent: one workgroup per CU walks its tiles, the next tile's loads start "
     "under this tile's last steps, C staged through LDS"),
    ("mfma16_256x256x64_w4_r5_persistent_lean", "R8",
     "4 waves of 128x128, one per SIMD (accumulators in all 256 AGPRs, a third fewer LDS reads "
     "per MFMA), with a K loop that holds no scalar or vector arithmetic: a cycle of five steps "
     "with constant slot offsets, addresses kept in registers (the default)"),
]

# (variant, what differs: from R1 for the first row, from R8 for the two
# 4-wave rows, else from R7)
SIDE = [
    ("mfma16_128x128x64_w4_s1",
     "R1 without the one-workgroup limit: its 32 KiB of LDS lets four workgroups share a CU, "
     "and they overlap each other's copies and MFMAs (CDNA4's way to hide a load without a ring)"),
    ("mfma16_256x256x64_w8_r5_l4_persistent_direct",
     "C stored straight from registers as 8-byte pieces, no LDS staging "
     "(V6's 'Serialized Shared-Memory Epilogue', undone)"),
    ("mfma16_256x256x64_w8_r5_l4_persistent_group4",
     "raster groups of 4 tile rows instead of 8 (V5's width; V6 raised it to 8)"),
    ("mfma16_256x256x64_w8_r5_l4_persistent_noxcd",
     "the pages' grouped raster (8 rows) without renumbering tiles per XCD"),
    ("mfma16_256x256x64_w8_r5_l4_persistent_linear",
     "tiles in row-major order: no grouped raster, no XCD renumbering"),
    ("mfma16_256x256x64_w8_r5_l4_persistent_columns",
     "MFMAs down every column of blocks top to bottom, not back up every second one: at each "
     "column's end both fragments change"),
    ("mfma16_256x256x64_w8_r5_l4_persistent_vacc",
     "accumulators in VGPRs instead of AGPRs (the epilogue converts them without moving them first)"),
    ("mfma16_256x256x64_w4_r5_persistent_rs2",
     "R8 without the lean K loop: every step computes its slot offsets, M0 values and load "
     "addresses (a lone wave per SIMD pays for that arithmetic between its MFMAs)"),
    ("mfma16_256x256x64_w4_r5_persistent_rs2_m0",
     "the same, with each group of four global->LDS loads sharing one LDS base (M0)"),
    ("mfma16_256x256x64_w8_s2",
     "compiler-scheduled 256x256, 8 waves, all loading, 2-stage ring (16x16x32 MFMAs)"),
    ("mfma32_256x256x64_w8_s2",
     "the same with 32x32x16 MFMAs"),
]


def rows(only=None):
    """The rows in table order; with `only` (variant names), just those."""
    r = [(v, r, w) for v, r, w in LADDER] + [(v, "side", w) for v, w in SIDE]
    if only:
        missing = set(only) - {v for v, _, _ in r}
        if missing:
            raise SystemExit("ladder: not a row: %s" % ", ".join(sorted(missing)))
        r = [x for x in r if x[0] in set(only)]
    return r


def run(args) -> int:
    import torch

    from dense_fp16_gemm_04_amd import binding, workloads

    binding.load()
    if not torch.cuda.is_available():
        print("ladder: no GPU visible", file=sys.stderr)
        return 1
    w = workloads.by_name(args.workload)
    dev = torch.device("cuda:0")
    a, b = workloads.workload_inputs(w)
    ta = torch.from_numpy(a).to(dev)
    tb = torch.from_numpy(b).to(dev)
    out = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    names = binding.variants()
    stream = torch.cuda.current_stream(dev)
    table = []
    for name, rung, what in rows(args.only):
        vid = names.index(name)

        def step():
            binding.gemm_nt_f16_ex(ta, tb, out=out, variant=vid)

        warmup, launches = args.warmup, args.launches
        t0 = time.perf_counter()
        first = True
        while args.settle > 0 and time.perf_counter() - t0 < args.settle:
            step()
            torch.cuda.synchronize()
            if first and time.perf_counter() - t0 > 0.02:  # a slow rung (the per-element kernel)
                warmup, launches = 1, 3
            first = False
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(launches):
            step()
        e.record(stream)
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / launches
        table.append({"variant": name, "rung": rung, "ms": ms, "tflops": w.flops / ms / 1e9, "launches": launches,
                      "what": what})
        print("ladder: %-4s %-46s %9.4f ms %8.1f TFLOP/s" % (rung, name, ms, w.flops / ms / 1e9),
              file=sys.stderr, flush=True)
    print(json.dumps({"workload": w.name, "settle": args.settle, "warmup": args.warmup,
                      "launches": args.launches, "rows": table}), flush=True)
    return 0


def _dispatches(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("ladder: no counter_collection.csv under %s" % d)
    disp = {}
    for r in csv.DictReader(open(files[0])):
        if "gemm_nt_f16" not in r["Kernel_Name"]:
            continue
        e = disp.setdefault(int(r["Dispatch_Id"]),
                            {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        e[r["Counter_Name"]] = float(r["Counter_Value"])
    return [disp[k] for k in sorted(disp)]


def summarize(dirs, warmup, launches, times=None, workload="square_8192", only=None) -> int:
    from dense_fp16_gemm_04_amd import workloads

    w = workloads.by_name(workload)
    order = rows(only)
    per = warmup + launches
    runs = {v: [] for v, _, _ in order}  # per row: one {counter: median} per counter run
    for d in dirs:
        disp = _dispatches(d)
        if len(disp) != per * len(order):
            print("ladder: %s holds %d GEMM dispatches, expected %d" % (d, len(disp), per * len(order)),
                  file=sys.stderr)
            return 1
        for i, (v, _, _) in enumerate(order):
            chunk = disp[i * per + warmup:(i + 1) * per]
            runs[v].append({c: statistics.median(x[c] for x in chunk) for c in chunk[0]})

    def get(v, *names):
        """The named counters of row v, all from the first run that counted
        every one of them (a ratio never mixes two runs), else None."""
        for r in runs[v]:
            if all(n in r for n in names):
                return [r[n] for n in names]
        return None

    timed = {}
    if times:
        with open(times) as f:
            timed = {r["variant"]: r for r in json.loads(f.read().strip().splitlines()[-1])["rows"]}
    mfmas = w.flops / 16384  # 16x16x32 MFMAs the product needs

    def ratio(v, f, *names):
        x = get(v, *names)
        try:
            return None if x is None else f(*x)
        except ZeroDivisionError:
            return None

    fmt = lambda x, f: "-" if x is None else f % x
    print("| rung | variant | TFLOP/s | % of peak | MFMA busy | implied clock MHz | waves waiting | "
          "LDS instr / MFMA | SALU / MFMA | LDS bank conflicts | read beyond L2 GB | written GB | "
          "L2 hit | what changes |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    for v, rung, what in order:
        busy = ratio(v, lambda m, g: 100 * m / (g / 8 * 1024), "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
        wait = ratio(v, lambda a, c: 100 * a / c, "SQ_WAIT_ANY", "SQ_WAVE_CYCLES")
        lds = ratio(v, lambda x: x / mfmas, "SQ_INSTS_LDS")
        salu = ratio(v, lambda x: x / mfmas, "SQ_INSTS_SALU")
        conf = ratio(v, lambda b, a: 100 * b / a, "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE")
        rd = ratio(v, lambda x: 32 * x / 1e9, "TCC_EA0_RDREQ_DRAM_32B_sum")
        wr = ratio(v, lambda a, b: (64 * b + 32 * (a - b)) / 1e9, "TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum")
        hit = ratio(v, lambda h, r: 100 * h / r, "TCC_HIT_sum", "TCC_REQ_sum")
        tf = timed.get(v, {}).get("tflops")
        # the clock at which the timed rate and the counted busy fraction
        # agree: TFLOP/s = busy * 1024 SIMDs * 1024 flop/clock * clock
        implied = tf / (busy / 100 * 1.048576) if tf and busy else None
        print("| %s | `%s` | %s | %s | %s | %s | %s | %s | %s | %s | %s | %s | %s | %s |" % (
            rung, v, fmt(tf, "%.1f"), fmt(None if tf is None else 100 * tf / 2516.5824, "%.1f"),
            fmt(busy, "%.1f%%"), fmt(implied, "%.0f"), fmt(wait, "%.1f%%"), fmt(lds, "%.3f"), fmt(salu, "%.3f"),
            fmt(conf, "%.2f%%"), fmt(rd, "%.3f"), fmt(wr, "%.3f"), fmt(hit, "%.1f%%"), what))
    # counters outside the main table, where a run collected them
    extra = [("scalar-unit instr per cycle per CU", lambda a, g: a / (g / 8) / 256, "%.3f",
              ("SQ_ACTIVE_INST_SCA", "GRBM_GUI_ACTIVE")),
             ("vector instr per MFMA (MFMAs included)", lambda x: x / mfmas, "%.3f", ("SQ_INSTS_VALU",)),
             ("waiting to issue an LDS instr", lambda a, c: 100 * a / c, "%.1f%%",
              ("SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES")),
             ("issue cycles per global->LDS load", lambda a, n: a / n, "%.2f",
              ("SQ_INST_CYCLES_VMEM_RD", "SQ_INSTS_VMEM_RD")),
             ("LDS busy", lambda a, g: 100 * a / (g / 8 * 256), "%.1f%%", ("SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE")),
             ("clock of the counted dispatches, MHz", lambda g, ns: g / 8 / (ns * 1e-9) / 1e6, "%.0f",
              ("GRBM_GUI_ACTIVE", "ns"))]
    present = [x for x in extra[:-1] if any(get(v, x[3][0]) is not None for v, _, _ in order)]
    if present:
        present.append(extra[-1])
        print()
        print("| variant | " + " | ".join(x[0] for x in present) + " |")
        print("|---|" + "---|" * len(present))
        for v, _, _ in order:
            vals = [fmt(ratio(v, f, *names), form) for _, f, form, names in present]
            print("| `%s` | %s |" % (v, " | ".join(vals)))
    return 0


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--workload", default="square_8192")
    p.add_argument("--settle", type=float, default=0.5, help="seconds of untimed launches before each row")
    p.add_argument("--launches", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--summarize", nargs="+", metavar="DIR", help="summarise rocprofv3 counter output")
    p.add_argument("--times", help="the JSON line of a timed run, for the TFLOP/s column")
    p.add_argument("--only", type=lambda x: x.split(","), metavar="V1,V2,...",
                   help="run (or summarise) only these rows, in table order")
    args = p.parse_args(argv)
    if args.summarize:
        return summarize(args.summarize, args.warmup, args.launches, args.times, args.workload, args.only)
    return run(args)


if __name__ == "__main__":
    sys.exit(main())
