import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950)")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run where no GPU is visible; say so instead of failing.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    # the error distribution of every Gaussian workload compared in full
    try:
        import _errstats
    except ImportError:  # pragma: no cover
        return
    if not _errstats.RECORDS:
        return
    tr = terminalreporter
    tr.write_sep("-", "error of the GPU result against the oracle's binary64 sum")
    tr.write_line("%-26s %6s %10s %10s %10s %10s %10s %9s %10s %10s" % (
        "workload", "K", "outputs", "mean", "p99", "max", "signed", "bit-eq", "rne mean", "rne max"))
    for r in _errstats.RECORDS:
        tr.write_line("%-26s %6d %10d %10.4g %10.4g %10.4g %10.3g %9.5f %10.4g %10.4g" % (
            r["workload"], r["K"], r["outputs"], r["mean"], r["p99"], r["max"], r["signed_mean"],
            r["bit_equal_to_rne_c64"], r["rne_floor_mean"], r["rne_floor_max"]))
    path = os.environ.get("GEMM_ERROR_REPORT")
    if path:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "w") as f:
            json.dump(_errstats.RECORDS, f, indent=1)
