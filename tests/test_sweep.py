"""The shape sweep: its candidate list matches the library's variants and
its table is built from a run's JSON line (host logic, no GPU); autotune
picks a way of running a shape whose result matches the oracle (GPU)."""
from __future__ import annotations

import json

import numpy as np
import pytest

from dense_fp16_gemm_04_amd import binding, sweep, workloads


def test_candidates_are_variants():
    names = binding.variants()
    for n in sweep.CANDIDATES:
        assert n in names
    for s in sweep.DEFAULT_SHAPES:
        M, N, K = (int(t) for t in s.split("x"))
        # every default shape takes the MFMA path (K % 8 == 0, aligned rows)
        v, rows, rest = binding.gemm_nt_f16_plan(M, N, K)
        assert names[v] in sweep.CANDIDATES
        assert rows == M or names[rest] in sweep.CANDIDATES


def test_table_from_json(tmp_path, capsys):
    t = {n: 100.0 + i for i, n in enumerate(sweep.CANDIDATES)}
    t.update({"selected": 101.0, "hipBLASLt": 50.0})
    row = {"shape": "64x64x64", "selected": sweep.CANDIDATES[1], "tflops": t}
    split = dict(row, shape="128x64x64", split={"rows": 64, "rest": sweep.CANDIDATES[2]})
    p = tmp_path / "sweep.json"
    p.write_text("noise\n" + json.dumps({"launches": 5, "rows": [row, split]}) + "\n")
    assert sweep.table(str(p)) == 0
    out = capsys.readouterr().out.splitlines()
    assert out[0].startswith("| shape | selected |")
    cells = [c.strip() for c in out[2].strip("|").split("|")]
    assert cells[0] == "64x64x64"
    assert cells[2] == "101"
    best = 100.0 + len(sweep.CANDIDATES) - 1
    assert cells[-3] == "%.2f" % (best / 101.0)
    assert cells[-1] == "%.2f" % (101.0 / 50.0)
    assert "(rows < 64)" in out[3]


@pytest.mark.gpu
def test_autotune_choice_is_correct():
    import torch

    import oracle

    M, N, K = 1000, 520, 264
    variant, ms = sweep.autotune(M, N, K, launches=5, repeats=2)
    names = binding.variants()
    assert set(ms) == {"plan", *sweep.CANDIDATES} and all(t > 0 for t in ms.values())
    assert variant == -1 or names[variant] in sweep.CANDIDATES
    assert ms["plan" if variant < 0 else names[variant]] == min(ms.values())
    a, b = workloads.small_integers(M, N, K, seed=31)
    _, c16 = oracle.gemm_nt(a, b)
    ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    c = binding.gemm_nt_f16(ta, tb) if variant < 0 else binding.gemm_nt_f16_ex(ta, tb, variant=variant)
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy().view(np.uint16), c16.view(np.uint16))
