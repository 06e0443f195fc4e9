"""Host logic of bench.py (no GPU): the one-GPU guard, argument checks and
the fresh-process repeat that reports the median run, and the amd-smi clock
sampler (run against a stand-in amd-smi script), both as bench.py starts it
and as the package's clock module does."""
from __future__ import annotations

import json
import subprocess
import sys
import types

import pytest

import bench
from dense_fp16_gemm_04_amd import clock


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err


def test_bad_counts_are_refused():
    assert bench.main(["--steps", "0"]) == 2
    assert bench.main(["--repeat", "0"]) == 2


def test_repeat_reports_the_median_run(monkeypatch, capsys):
    values = iter([1300.0, 1340.0, 1320.0])
    seen = []

    def fake_run(cmd, stdout=None, text=None):
        seen.append(cmd)
        rec = {"metric": "m", "value": next(values), "unit": "TFLOP/s"}
        return types.SimpleNamespace(returncode=0, stdout="bench noise\n" + json.dumps(rec) + "\n")

    monkeypatch.setattr(subprocess, "run", fake_run)
    assert bench.main(["--repeat", "3", "--cpu-rows", "0", "--steps", "5"]) == 0
    out = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert out["value"] == 1320.0
    assert out["repeat"]["values"] == [1300.0, 1340.0, 1320.0]
    assert out["repeat"]["range"] == [1300.0, 1340.0]
    assert len(seen) == 3
    for cmd in seen:
        # each child runs once, on the same arguments, without the CPU baseline
        assert cmd[0] == sys.executable and cmd[1].endswith("bench.py")
        assert cmd.count("--repeat") == 1 and cmd[cmd.index("--repeat") + 1] == "1"
        assert cmd[cmd.index("--cpu-rows") + 1] == "0"
        assert "--steps" in cmd and cmd[cmd.index("--steps") + 1] == "5"


FAKE_SMI = r'''
import json, sys
if sys.argv[1] == "list":
    print("noise before the document")
    print(json.dumps([{"gpu": 0, "bdf": "0000:75:00.0"}, {"gpu": 1, "bdf": "0000:05:00.0"}]))
else:
    clock = lambda mhz: {"clk": {"value": mhz, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"}}
    gpu = lambda i, base, w: {"gpu": i, "power": {"socket_power": {"value": w, "unit": "W"}},
                              "clock": {"gfx_0": clock(base), "gfx_1": clock(base + 20), "mem_0": clock(2000),
                                        "fclk_0": {"clk": "N/A"}}}
    print(json.dumps({"gpu_data": [gpu(0, 1500, 1300), gpu(1, 100, 200)]}))
'''


# the sampler child as bench.py starts it, and as clock.start_sampler() does
SAMPLER_COMMANDS = {"bench": [sys.executable, bench.__file__, "--smi-sampler"],
                    "clock": [sys.executable, clock.__file__]}


@pytest.mark.parametrize("entry", sorted(SAMPLER_COMMANDS))
def test_clock_sampler_protocol(tmp_path, entry):
    """The sampler waits for a first line, queries until a second one, and
    reports every GPU's mean engine clock over the XCDs and its power;
    samples_of picks the GPU by PCI address."""
    script = tmp_path / "amdsmi_cli.py"
    script.write_text(FAKE_SMI)
    script.chmod(0o755)
    (tmp_path / "amd-smi").symlink_to(script)
    env = dict(__import__("os").environ, PATH="%s:%s" % (tmp_path, __import__("os").environ.get("PATH", "")))
    proc = subprocess.Popen(SAMPLER_COMMANDS[entry], stdin=subprocess.PIPE,
                            stdout=subprocess.PIPE, text=True, env=env)
    proc.stdin.write("start\n")
    proc.stdin.flush()
    import time
    time.sleep(1.0)
    proc.stdin.write("stop\n")
    proc.stdin.flush()
    got = json.loads(proc.communicate(timeout=60)[0].strip().splitlines()[-1])
    assert proc.returncode == 0
    assert got["bdf"] == {"0": "0000:75:00.0", "1": "0000:05:00.0"}
    assert len(got["samples"]) >= 2
    mine = bench.samples_of(got, 0, 0x75)
    assert mine and all(m == (1510.0, 1300.0) for m in mine)
    assert all(m == (110.0, 200.0) for m in bench.samples_of(got, 0, 0x05))
    assert bench.samples_of(got, 0, 0x99) == []


def test_one_sampler_serves_window_after_window(tmp_path):
    """After a window's report the sampler waits for the next start line;
    read_window(keep=True) takes one report and leaves the child running."""
    import time

    script = tmp_path / "amdsmi_cli.py"
    script.write_text(FAKE_SMI)
    script.chmod(0o755)
    (tmp_path / "amd-smi").symlink_to(script)
    env = dict(__import__("os").environ, PATH="%s:%s" % (tmp_path, __import__("os").environ.get("PATH", "")))
    proc = subprocess.Popen(SAMPLER_COMMANDS["clock"], stdin=subprocess.PIPE, stdout=subprocess.PIPE, text=True,
                            env=env)
    reports = []
    for _ in range(2):
        clock.tell(proc, "start")
        time.sleep(0.5)
        clock.tell(proc, "stop")
        reports.append(json.loads(clock.read_window(proc, keep=True, timeout=60)))
        assert proc.poll() is None
    clock.stop_sampler(proc)
    assert proc.returncode == 0
    for got in reports:
        assert got["samples"] and clock.samples_of(got, 0, 0x75)[0] == (1510.0, 1300.0)


@pytest.mark.parametrize("entry", sorted(SAMPLER_COMMANDS))
def test_clock_sampler_without_a_start_line_exits(entry):
    proc = subprocess.run(SAMPLER_COMMANDS[entry], input="", stdout=subprocess.PIPE, text=True, timeout=60)
    assert proc.returncode == 0 and proc.stdout == ""


def test_profiler_runs_skip_the_clock_window(monkeypatch):
    monkeypatch.delenv("ROCPROF_OUTPUT_PATH", raising=False)
    base = bench.under_profiler()
    monkeypatch.setenv("ROCPROF_OUTPUT_PATH", "/tmp/x")
    assert bench.under_profiler() and not base


def test_cpu_configs_table(monkeypatch):
    """The oracle timing table: every configuration on the host's threads,
    the small ones on one thread too, with the CPU named."""
    from dense_fp16_gemm_04_amd import workloads

    small = tuple(workloads.Workload("w%d" % i, m, n, k, 100 + i)
                  for i, (m, n, k) in enumerate([(16, 8, 8), (24, 16, 32), (40, 8, 16)]))
    monkeypatch.setattr(workloads, "WORKLOADS", small)
    t = bench.cpu_configs()
    assert t["threads"] >= 1 and t["nproc"] >= 1 and isinstance(t["cpu_model"], str)
    assert [(r["workload"], r["threads"]) for r in t["runs"]] == [
        (w.name, th) for w in small for th in ([t["threads"], 1])]
    assert all(r["seconds"] > 0 and r["gflops"] > 0 for r in t["runs"])


def test_traffic_record_follows_the_kernel_code_not_its_comments(tmp_path, monkeypatch):
    """bench.py reports the measured traffic only for the kernel code it was
    measured on: the digest ignores comments and whitespace, and changes with
    any code."""
    import bench

    src = tmp_path / "k.hip"
    src.write_text("// a comment\nint f(int x) { return x + 1; }  /* more */\n")
    monkeypatch.setattr(bench, "SOURCE", str(src))
    d0 = bench.source_digest()
    src.write_text("// another comment\nint f(int x)\n{\n    return x + 1;\n}\n")
    assert bench.source_digest() == d0
    src.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_digest() != d0
    assert len(d0) == 16
