"""Ablation ladder: every kernel variant of the library on one workload.

Each variant is one design choice away from its neighbours (tile size, wave
count, ring depth, fragment read distance, which waves load, persistence,
hand-scheduled issue order), so the table shows what each choice is worth on
MI355X.  The ladder follows the sequence of design steps the pages walk
through ("0. A Minimal Hopper Matmul" to "6. Four Consumers, FP16
Accumulation, and a TMA Epilogue", section "Summary"), re-made for CDNA4.

Run (needs a GPU):

    python -m dense_fp16_gemm_04_amd.ladder [--workload square_8192]

Under rocprofv3, with one counter set per run, and then summarised (no GPU
needed for the summary):

    rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_LDS_BANK_CONFLICT \\
        SQ_LDS_IDX_ACTIVE --output-format csv -d DIR1 -o run -- \\
        python3 -m dense_fp16_gemm_04_amd.ladder --launches 2 --warmup 1 --cooldown 0
    python -m dense_fp16_gemm_04_amd.ladder --summarize DIR1 [DIR2 ...]

The summary assigns GEMM dispatches to variants in launch order, which this
script fixes: every variant gets warmup + launches dispatches, in table
order, and nothing else launches a kernel whose name contains gemm_nt_f16.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# What each variant changes.  mfma32 variants use v_mfma_f32_32x32x16_f16,
# mfma16 ones v_mfma_f32_16x16x32_f16.
RUNGS = {
    "simple_f32_per_element": "one thread per output, no tiling (the naive baseline)",
    "mfma32_64x64x64_w4_s3": "64x64 tile, 4 waves, 3-stage ring",
    "mfma32_128x128x64_w4_s3": "128x128 tile: 2x the reuse per loaded byte",
    "mfma32_256x128x64_w4_s3": "256x128 tile",
    "mfma32_256x256x64_w4_s2": "256x256 tile, 4 waves (1 per SIMD, 256 accumulators each), 2 stages",
    "mfma32_256x256x64_w8_s2": "256x256 tile, 8 waves (2 per SIMD, 128 accumulators each)",
    "mfma32_256x256x32_w8_s5": "same, BK 32 with a 5-stage ring (loads 4 steps ahead)",
    "mfma32_256x256x32_w8_s4_d2": "BK 32, 4 stages, fragments read a whole step ahead, loads spread over the step",
    "mfma32_256x256x64_w8_s2_l4": "only 4 of the 8 waves issue global->LDS loads (a producer/consumer split)",
    "mfma32_256x256x32_w4_s5_e4": "4 waves, BK 32, 5 stages, half of each step's loads issued a step early",
    "mfma16_256x256x64_w4_s2": "16x16x32 MFMAs, 4 waves (1 per SIMD, 128x128 each, accumulators in all 256 AGPRs)",
    "mfma16_256x256x64_w8_s2": "16x16x32 MFMAs, 8 waves (2 per SIMD, 128x64 each)",
    "mfma16_256x256x32_w8_s4": "16x16x32 MFMAs, 8 waves, BK 32 with a 4-stage ring",
    "mfma16_256x256x64_w8x_s2": "16x16x32 MFMAs, 8 waves laid out 4x2 (64x128 each)",
    "mfma16_256x256x64_w8_s2_l4": "16x16x32 MFMAs, 8 waves, 4 of them loading",
    "mfma16_256x256x64_w4_s2_ordered": "4 waves again, every read and load placed by hand, one per 4 MFMAs",
    "mfma16_256x256x64_w8_s2_l4_ordered": "8 waves, 4 loading, every read and load placed by hand",
    "mfma16_256x256x64_w8_r5_l4_ordered": "same with a 5-slot ring: A loads half a step earlier, loads over the whole step",
    "mfma16_256x256x64_w8_r5_l4_persistent": "same, persistent: the next tile's first steps load during this tile's last, half the waves store C: the default",
    "mfma16_256x128x64_w4_s3": "16x16x32 MFMAs, 256x128 tile, 4 waves",
    "mfma16_256x128x64_w8_s3": "16x16x32 MFMAs, 256x128 tile, 8 waves",
    "mfma16_256x128x64_w4_s3_ordered": "256x128 tile, 4 waves, issue order fixed by hand",
    "mfma16_256x128x64_w8_s3_l4_ordered": "256x128 tile, 8 waves (2x4, 128x32 each), 4 loading, issue order fixed by hand",
    "mfma16_256x128x64_w8x_s3_l4_ordered": "same with the waves laid out 4x2 (64x64 each: a fifth fewer LDS reads per MFMA; default for one GPU's share)",
    "mfma16_128x128x64_w4_s3": "16x16x32 MFMAs, 128x128 tile, 4 waves",
    "mfma16_128x128x64_w8_s3": "16x16x32 MFMAs, 128x128 tile, 8 waves",
    "mfma16_128x128x64_w8_s3_l4_ordered": "128x128 tile, 8 waves, 4 loading, issue order fixed by hand (default for mid sizes)",
    "mfma16_64x64x64_w4_s3": "16x16x32 MFMAs, 64x64 tile (default for small sizes)",
}


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
    order = [n for n in names if n != "simple_f32_per_element" or args.with_simple]
    rows = []
    stream = torch.cuda.current_stream(dev)
    for name in order:
        vid = names.index(name)
        for _ in range(args.warmup):
            binding.gemm_nt_f16_ex(ta, tb, out=out, variant=vid)
        torch.cuda.synchronize()
        if args.cooldown > 0:
            time.sleep(args.cooldown)
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(args.launches):
            binding.gemm_nt_f16_ex(ta, tb, out=out, variant=vid)
        e.record(stream)
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / args.launches
        rows.append({"variant": name, "ms": ms, "tflops": w.flops / ms / 1e9,
                     "rung": RUNGS.get(name, "")})
        print("ladder: %-32s %8.4f ms %8.1f TFLOP/s" % (name, ms, w.flops / ms / 1e9),
              file=sys.stderr, flush=True)
    print(json.dumps({"workload": w.name, "warmup": args.warmup, "launches": args.launches,
                      "rows": rows}), flush=True)
    return 0


def summarize(dirs, warmup, launches, with_simple) -> int:
    from dense_fp16_gemm_04_amd import binding

    names = [n for n in binding.variants() if n != "simple_f32_per_element" or with_simple]
    per = warmup + launches
    table = {n: {} for n in names}
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            print("ladder: no counter_collection.csv under %s" % d, file=sys.stderr)
            return 1
        rows = list(csv.DictReader(open(files[0])))
        disp = {}
        for r in rows:
            if "gemm_nt_f16" not in r["Kernel_Name"]:
                continue
            disp.setdefault(int(r["Dispatch_Id"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
        ids = sorted(disp)
        if len(ids) != per * len(names):
            print("ladder: %s holds %d GEMM dispatches, expected %d" % (d, len(ids), per * len(names)),
                  file=sys.stderr)
            return 1
        for i, n in enumerate(names):
            chunk = [disp[k] for k in ids[i * per + warmup:(i + 1) * per]]
            for c in chunk[0]:
                table[n][c] = sum(x[c] for x in chunk) / len(chunk)
    print("| variant | MFMA busy | LDS bank conflicts | HBM read KiB | HBM write KiB | what changes |")
    print("|---|---|---|---|---|---|")
    for n in names:
        t = table[n]
        busy = (t["SQ_VALU_MFMA_BUSY_CYCLES"] / (t["GRBM_GUI_ACTIVE"] / 8 * 1024)
                if "SQ_VALU_MFMA_BUSY_CYCLES" in t and "GRBM_GUI_ACTIVE" in t else None)
        conf = (t["SQ_LDS_BANK_CONFLICT"] / t["SQ_LDS_IDX_ACTIVE"]
                if t.get("SQ_LDS_IDX_ACTIVE") else None)
        cell = lambda v, f: (f % v) if v is not None else "-"
        print("| `%s` | %s | %s | %s | %s | %s |" % (
            n, cell(None if busy is None else 100 * busy, "%.1f%%"), cell(None if conf is None else 100 * conf, "%.1f%%"),
            cell(t.get("FETCH_SIZE"), "%.0f"), cell(t.get("WRITE_SIZE"), "%.0f"), RUNGS.get(n, "")))
    return 0


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--workload", default="square_8192")
    p.add_argument("--launches", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--cooldown", type=float, default=1.0)
    p.add_argument("--with-simple", action="store_true", help="include the per-element kernel (slow)")
    p.add_argument("--summarize", nargs="+", metavar="DIR", help="summarise rocprofv3 counter output")
    args = p.parse_args(argv)
    if args.summarize:
        return summarize(args.summarize, args.warmup, args.launches, args.with_simple)
    return run(args)


if __name__ == "__main__":
    sys.exit(main())
