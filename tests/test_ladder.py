"""The ablation ladder's host logic (no GPU): its rows, the row filter, and
the counter summary, on synthetic rocprofv3 output."""
from __future__ import annotations

import csv
import os

import pytest

from dense_fp16_gemm_04_amd import binding, ladder

COLUMNS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
           "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
           "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
           "End_Timestamp"]


def test_every_row_is_a_variant_of_the_library():
    names = set(binding.variants())
    rows = ladder.rows()
    assert [r for _, r, _ in rows[:9]] == ["R%d" % i for i in range(9)]
    for v, _, _ in rows:
        assert v in names, v
    assert len({v for v, _, _ in rows}) == len(rows)


def test_only_keeps_table_order_and_rejects_unknown_rows():
    picked = ladder.rows(["mfma16_256x256x64_w4_r5_persistent_lean", "mfma16_256x256x64_w8_r5_l4_persistent"])
    assert [r for _, r, _ in picked] == ["R7", "R8"]
    with pytest.raises(SystemExit):
        ladder.rows(["no_such_variant"])


def _write_run(d, dispatches):
    """dispatches: list of (kernel name, ns, {counter: value})."""
    os.makedirs(d)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(COLUMNS)
        t = 1000
        for i, (name, ns, counters) in enumerate(dispatches, start=1):
            for c, val in counters.items():
                w.writerow([i, i, "Agent 1", 1, 1, 1, 0, 1, name, 256, 0, 0, 0, 0, 0, c, val, t, t + ns])
            t += ns + 10


def test_summary_takes_busy_cycles_and_cycle_count_from_the_same_run(tmp_path, capsys):
    """MFMA busy divides the matrix-core cycles by the GRBM cycles of the
    run that counted them, not by those of a later counter run."""
    only = ["mfma16_256x256x64_w8_r5_l4_persistent", "mfma16_256x256x64_w4_r5_persistent_lean"]
    cyc = 1_000_000  # per XCD
    run1, run2 = [], []
    for busy in (0.90, 0.88):
        for _ in range(3):  # 1 warm-up + 2 counted
            run1.append(("gemm_nt_f16_kernel", 700_000, {
                "GRBM_GUI_ACTIVE": 8 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": busy * cyc * 1024,
                "SQ_WAVE_CYCLES": 100.0, "SQ_WAIT_ANY": 5.0, "SQ_INSTS_LDS": 1.0, "SQ_INSTS_SALU": 1.0,
                "SQ_LDS_BANK_CONFLICT": 1.0, "SQ_LDS_IDX_ACTIVE": 100.0}))
            # a second run whose dispatches took twice the cycles
            run2.append(("gemm_nt_f16_kernel", 700_000, {"GRBM_GUI_ACTIVE": 16 * cyc, "TCC_HIT_sum": 8.0,
                                                         "TCC_REQ_sum": 10.0}))
    _write_run(str(tmp_path / "a"), run1)
    _write_run(str(tmp_path / "b"), run2)
    assert ladder.summarize([str(tmp_path / "a"), str(tmp_path / "b")], 1, 2, only=only) == 0
    out = capsys.readouterr().out
    lines = [l for l in out.splitlines() if l.startswith("| R7") or l.startswith("| R8")]
    assert "| 90.0% |" in lines[0] and "| 88.0% |" in lines[1], out
    assert "| 80.0% |" in lines[0]  # the L2 hit rate from the second run
