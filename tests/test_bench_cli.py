"""Host logic of bench.py (no GPU): the one-GPU guard, argument checks and
the fresh-process repeat that reports the median run."""
from __future__ import annotations

import json
import subprocess
import sys
import types

import bench


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
