"""Shape sweep: the selected kernel, every selectable kernel and hipBLASLt.

For each shape the sweep times, in one process on one GPU, what the library
runs (one kernel, or two on blocks of rows), each of the kernels it chooses
from run alone on the whole product, and
hipBLASLt (``torch.matmul``, as context only), each as a CUDA-graph replay
of back-to-back launches.  It reports TFLOP/s and which kernel was fastest,
so the selection can be checked against measurement on square, non-square
and skinny shapes (the pages warn that their kernels were tuned for one
shape: "6. Four Consumers, FP16 Accumulation, and a TMA Epilogue", section
"Performance", the closing caution).  A caller who wants the fastest kernel
for a shape the selection gets wrong can pass the reported variant to
``gemm_nt_f16_ex``; ``autotune`` (or ``--autotune MxNxK``) measures that
choice for one shape.

Run (needs a GPU):

    python -m dense_fp16_gemm_04_amd.sweep [--shapes 8192x8192x8192,...] [--launches 50]
    python -m dense_fp16_gemm_04_amd.sweep --autotune 6144x6144x2048
"""
from __future__ import annotations

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# square, non-square, skinny and ragged shapes
DEFAULT_SHAPES = [
    "512x512x512", "1024x1024x1024", "2048x2048x2048", "3072x3072x3072", "4096x4096x4096",
    "6144x6144x6144", "8192x8192x8192", "3000x3000x3000", "5000x3000x6000", "2816x2816x4096",
    "4352x4352x2048", "6144x6144x2048", "4104x4096x2048", "8192x8192x1024", "4096x4096x1024",
    "4096x4096x16384", "2048x2048x8192",
    "1024x1024x8192", "256x8192x8192", "512x8192x8192", "1024x8192x8192", "2048x8192x8192",
    "8192x256x8192", "8192x1024x8192", "8192x8192x256", "16384x4096x4096", "4096x16384x4096",
]

# the kernels the selection chooses from (select_mfma's candidates)
CANDIDATES = [
    "mfma16_256x256x64_w4_r5_persistent_lean",
    "mfma16_256x128x64_w8x_s3_l4_ordered",
    "mfma16_128x128x64_w8_s3_l4_ordered",
    "mfma16_64x64x64_w4_s3",
]


def time_graph(torch, fn, launches):
    """Mean ms per launch of `launches` back-to-back calls replayed as one graph."""
    for _ in range(5):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(launches):
            fn()
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / launches


def autotune(M: int, N: int, K: int, launches: int = 20, repeats: int = 3):
    """Measure which way of running an M x N x K product is fastest here.

    Times the library's own plan (``gemm_nt_f16``) and each kernel it
    chooses from, run alone on the whole product through ``gemm_nt_f16_ex``,
    on seeded random fp16 inputs of the shape: graph replays of `launches`
    back-to-back calls, alternating between the contenders, `repeats` times,
    keeping each one's best.  Returns ``(variant, ms)``: variant -1 when the
    plan is fastest (call ``gemm_nt_f16``), else the index to pass to
    ``gemm_nt_f16_ex``; ``ms`` maps each contender's name ("plan" for the
    plan) to its best time per launch in milliseconds.
    """
    import torch

    from dense_fp16_gemm_04_amd import binding

    binding.load()
    if not torch.cuda.is_available():
        raise RuntimeError("autotune needs a GPU")
    if M < 1 or N < 1 or K < 1:
        raise ValueError("autotune needs M, N, K >= 1")
    names = binding.variants()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(M * 31 + N * 7 + K)
    a = (torch.randn(M, K, device="cuda", generator=gen) * K ** -0.25).half()
    b = (torch.randn(N, K, device="cuda", generator=gen) * K ** -0.25).half()
    out = torch.empty(M, N, dtype=torch.float16, device="cuda")
    fns = {"plan": lambda: binding.gemm_nt_f16(a, b, out=out)}
    if K % 8 == 0 and K < (1 << 22):  # the MFMA kernels' requirements
        for n in CANDIDATES:
            fns[n] = (lambda v: lambda: binding.gemm_nt_f16_ex(a, b, out=out, variant=v))(names.index(n))
    time_graph(torch, fns["plan"], launches)  # the first graph of a shape runs slow
    ms = {}
    for _ in range(max(1, repeats)):
        for label, fn in fns.items():
            t = time_graph(torch, fn, launches)
            ms[label] = min(ms.get(label, t), t)
    best = min(ms, key=ms.get)
    return (-1 if best == "plan" else names.index(best)), ms


def run(args) -> int:
    import torch

    from dense_fp16_gemm_04_amd import binding

    binding.load()
    if not torch.cuda.is_available():
        print("sweep: no GPU visible", file=sys.stderr)
        return 1
    names = binding.variants()
    cand = [names.index(n) for n in CANDIDATES]
    gen = torch.Generator(device="cuda")
    rows = []
    for shape in args.shapes.split(","):
        M, N, K = (int(t) for t in shape.split("x"))
        gen.manual_seed(M * 31 + N * 7 + K)
        a = (torch.randn(M, K, device="cuda", generator=gen) * K ** -0.25).half()
        b = (torch.randn(N, K, device="cuda", generator=gen) * K ** -0.25).half()
        out = torch.empty(M, N, dtype=torch.float16, device="cuda")
        sel, prows, rest = binding.gemm_nt_f16_plan(M, N, K)
        flop = 2.0 * M * N * K
        fns = [("selected", lambda: binding.gemm_nt_f16(a, b, out=out))]
        for vid in cand:
            fns.append((names[vid], (lambda v: lambda: binding.gemm_nt_f16_ex(a, b, out=out, variant=v))(vid)))
        fns.append(("hipBLASLt", lambda: torch.matmul(a, b.t(), out=out)))
        time_graph(torch, fns[0][1], args.launches)  # the first graph of a shape runs slow
        res = {}
        for label, fn in fns:
            ms = time_graph(torch, fn, args.launches)
            res[label] = flop / ms / 1e9
        best = max(CANDIDATES, key=lambda n: res[n])
        row = {"shape": shape, "selected": names[sel], "tflops": res}
        if prows < M:
            row["split"] = {"rows": prows, "rest": names[rest]}
        rows.append(row)
        label = names[sel] + ("" if prows == M else " rows<%d + %s" % (prows, names[rest]))
        print("sweep: %-18s selected %-40s %7.1f  best single %-40s %7.1f  hipBLASLt %7.1f" % (
            shape, label, res["selected"], best, res[best], res["hipBLASLt"]), file=sys.stderr, flush=True)
    print(json.dumps({"launches": args.launches, "rows": rows}), flush=True)
    return 0


def table(path) -> int:
    """Markdown table from the JSON line a run printed."""
    with open(path) as f:
        data = json.loads(f.read().strip().splitlines()[-1])
    short = {n: n.replace("mfma16_", "").replace("_ordered", " ord").replace("_persistent", " pers")
             for n in CANDIDATES}
    print("| shape | selected | selected TF/s | " + " | ".join(short[n] for n in CANDIDATES)
          + " | best single / selected | hipBLASLt | selected / hipBLASLt |")
    print("|---" * (len(CANDIDATES) + 6) + "|")
    for r in data["rows"]:
        t = r["tflops"]
        best = max(t[n] for n in CANDIDATES)
        sel = short.get(r["selected"], r["selected"])
        if "split" in r:
            sel += " (rows < %d) + %s" % (r["split"]["rows"], short.get(r["split"]["rest"], r["split"]["rest"]))
        print("| %s | %s | %.0f | %s | %.2f | %.0f | %.2f |" % (
            r["shape"], sel, t["selected"],
            " | ".join("%.0f" % t[n] for n in CANDIDATES), best / t["selected"], t["hipBLASLt"],
            t["selected"] / t["hipBLASLt"]))
    return 0


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--shapes", default=",".join(DEFAULT_SHAPES))
    p.add_argument("--launches", type=int, default=50)
    p.add_argument("--table", metavar="JSON", help="print a markdown table from a run's JSON output")
    p.add_argument("--autotune", metavar="MxNxK",
                   help="time the plan and each kernel on this shape; print the fastest as JSON")
    args = p.parse_args(argv)
    if args.table:
        return table(args.table)
    if args.autotune:
        M, N, K = (int(t) for t in args.autotune.split("x"))
        variant, ms = autotune(M, N, K, launches=args.launches)
        print(json.dumps({"shape": args.autotune, "variant": variant,
                          "use": "gemm_nt_f16" if variant < 0 else "gemm_nt_f16_ex(variant=%d)" % variant,
                          "ms": ms}), flush=True)
        return 0
    return run(args)


if __name__ == "__main__":
    sys.exit(main())
