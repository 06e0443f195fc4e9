"""Engine clock and board power under sustained load, read with amd-smi.

The engine clock is power-managed, so a throughput figure means most beside
the clock the chip held while it was taken.  A sampler child process, started
before the measuring process touches the GPU, queries ``amd-smi metric -c -p``
in a loop between a start and a stop line on its stdin; ``clock_window``
launches a step back to back meanwhile and returns the rate, the median
engine clock (averaged over the XCDs) and the board power.

Run as a script (``python clock.py``) this module is the sampler child.  It
imports nothing but the standard library, so the child starts in well under a
second and never loads a GPU runtime.
"""
from __future__ import annotations

import json
import os
import shutil
import statistics
import subprocess
import sys
import time


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def smi_command(*args):
    """amd-smi's command line, its Python entry script run directly by this
    interpreter; None when amd-smi is not installed."""
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    if not os.path.exists(exe):
        return None
    real = os.path.realpath(exe)
    return ([sys.executable, real] if real.endswith(".py") else [real]) + list(args)


def smi_json(*args):
    cmd = smi_command(*args, "--json")
    if cmd is None:
        return None
    try:
        res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True, timeout=30)
        out = res.stdout
        return json.loads(out[min(i for i in (out.find("{"), out.find("[")) if i >= 0):])
    except (OSError, ValueError, subprocess.SubprocessError):
        return None


def smi_sampler() -> int:
    """The sampler child, one window after another: it waits for a line on
    stdin, then queries amd-smi for every GPU's engine clocks and socket power
    until the next line (or end of input) arrives, and prints one line
    {"bdf": {gpu: PCI address}, "samples": [[gpu, MHz, W], ...]}.  It exits
    at end of input, or when amd-smi fails."""
    import select

    fd = sys.stdin.fileno()  # raw reads: no buffered line may hide the next one
    bdf = None
    while True:
        got = os.read(fd, 64)
        if not got:
            return 0
        if bdf is None:
            bdf = {}
            for g in smi_json("list") or []:
                if isinstance(g, dict) and "gpu" in g:
                    bdf[str(g["gpu"])] = str(g.get("bdf", "")).lower()
        samples = []
        ended = False
        while True:
            d = smi_json("metric", "-c", "-p")
            for g in (d or {}).get("gpu_data", []) if isinstance(d, dict) else []:
                try:
                    clks = [v["clk"]["value"] for k, v in g["clock"].items()
                            if k.startswith("gfx_") and isinstance(v.get("clk"), dict)]
                    samples.append([str(g["gpu"]), sum(clks) / len(clks),
                                    float(g["power"]["socket_power"]["value"])])
                except (KeyError, TypeError, ValueError, ZeroDivisionError, AttributeError):
                    pass
            if d is None:
                ended = True
                break
            if select.select([fd], [], [], 0)[0]:
                ended = not os.read(fd, 64)
                break
        print(json.dumps({"bdf": bdf, "samples": samples}), flush=True)
        if ended:
            return 0


def start_sampler():
    """A sampler child (this file run as a script); call it before the
    calling process first touches the GPU.  None when amd-smi or a GPU
    device node is missing."""
    if not os.path.exists("/dev/kfd") or smi_command() is None:
        return None
    return subprocess.Popen([sys.executable, os.path.abspath(__file__)], stdin=subprocess.PIPE,
                            stdout=subprocess.PIPE, text=True)


def stop_sampler(sampler) -> None:
    """End a sampler child that no window used."""
    if sampler is not None and sampler.poll() is None:
        sampler.stdin.close()  # end of input: the sampler exits
        try:
            sampler.wait(timeout=60)
        except subprocess.TimeoutExpired:
            sampler.kill()


def samples_of(got, domain, bus):
    """The (MHz, W) samples of the GPU at PCI domain:bus in the sampler's
    output; all of them when amd-smi lists a single GPU."""
    want = "%04x:%02x:" % (domain, bus)
    ids = [k for k, v in got.get("bdf", {}).items() if v.startswith(want)]
    if not ids and len(got.get("bdf", {})) == 1:
        ids = list(got["bdf"])
    return [(c, w) for g, c, w in got.get("samples", []) if ids and g == ids[0]]


def tell(sampler, line):
    """One line to the sampler; it may already have ended (amd-smi failing)."""
    try:
        sampler.stdin.write(line + "\n")
        sampler.stdin.flush()
    except OSError:
        pass


def read_window(sampler, keep: bool, timeout: float = 60.0) -> str:
    """The sampler's report of the window just stopped: with keep, one line
    read while the child waits for the next window; else its whole output
    once its input is closed (the child then exits)."""
    if not keep:
        return sampler.communicate(timeout=timeout)[0]
    import select
    if not select.select([sampler.stdout], [], [], timeout)[0]:
        raise subprocess.TimeoutExpired("amd-smi sampler", timeout)
    return sampler.stdout.readline()


def clock_window(sampler, seconds, step, stream, flops, props, peak_tflops, label="bench", keep=False):
    """Back-to-back calls of step() for `seconds` while the sampler child
    polls amd-smi: the rate (flops per call over the event-timed window on
    `stream`), the engine clock and board power under that load, and the
    rate as a share of peak_tflops scaled to the median clock (peak_tflops
    is quoted at 2.4 GHz).  None when amd-smi gave no samples.  With keep
    the sampler stays up for another window."""
    import torch

    s0 = torch.cuda.Event(enable_timing=True)
    e0 = torch.cuda.Event(enable_timing=True)
    for _ in range(5):  # reach load before the first sample
        step()
    torch.cuda.synchronize()
    s0.record(stream)
    tell(sampler, "start")
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step()
        n += 20
        torch.cuda.synchronize()
    e0.record(stream)
    tell(sampler, "stop")
    torch.cuda.synchronize()
    try:
        got = json.loads(read_window(sampler, keep).strip().splitlines()[-1])
    except (ValueError, IndexError, OSError, subprocess.SubprocessError):
        log("%s: amd-smi gave no samples; no clock window" % label)
        return None
    mine = samples_of(got, props.pci_domain_id, props.pci_bus_id)
    if not mine:
        log("%s: amd-smi gave no samples for this GPU; no clock window" % label)
        return None
    ms = s0.elapsed_time(e0) / n
    tflops = flops / (ms * 1e-3) / 1e12
    clk = [c for c, _ in mine]
    pw = [w for _, w in mine]
    # the median: the first sample may still see the clock of the ramp-up
    mhz = statistics.median(clk)
    rec = {"seconds": seconds, "launches": n, "ms_per_launch": ms, "tflops": tflops,
           "samples": len(mine), "sclk_mhz_median": mhz, "sclk_mhz_mean": statistics.mean(clk),
           "sclk_mhz_range": [min(clk), max(clk)], "power_w_mean": statistics.mean(pw), "power_w_max": max(pw),
           "pct_of_peak_at_sclk": 100 * tflops / (peak_tflops * mhz / 2400.0),
           "source": "amd-smi metric -c -p (engine clock averaged over the XCDs)"}
    log("%s: %.1f s of launches: %.1f TFLOP/s at %.0f MHz median engine clock, %.0f W; %.1f%% of the peak "
        "at that clock" % (label, seconds, tflops, mhz, rec["power_w_mean"], rec["pct_of_peak_at_sclk"]))
    return rec


if __name__ == "__main__":
    sys.exit(smi_sampler())
