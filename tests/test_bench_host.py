"""Host logic of bench.py (no GPU): attribution of counter-run dispatches to workloads and
kernels, and the clock / matrix-core utilisation arithmetic, on a synthetic rocprofv3 CSV."""
import csv
import json

import pytest

import bench
import fa_inputs as FI

NAMES = {"fwd": "void fa::fwd_kernel<fa::BF16, 128, 64, 4, true, false>(int)",
         "fwd_pingpong": "void fa::fwd_kernel<fa::BF16, 128, 64, 8, true, false>(int)",
         "bwd_dkv": "void fa::bwd_dkv_kernel<fa::BF16, 128, 4, true>(int)",
         "bwd_dq_delta": "void fa::bwd_dq_kernel<fa::BF16, 128, 64, 4, true>(int)"}


def _write_csv(path, order, ns=1_000_000, gui=None, busy=None, extra_first=True, counters=None, copy=None):
    """One row per (dispatch, counter); a foreign kernel (a copy) interleaved first."""
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    rows, d = [], 1
    if extra_first:
        rows.append([d, "__amd_rocclr_copyBuffer", "GRBM_GUI_ACTIVE", 5.0, 0, 10])
        d += 1
    for i, stage in enumerate(order):
        start = 1000 + i * 10 * ns
        g = gui(i) if gui else 8 * 1.5e9 * ns * 1e-9          # 1.5 GHz on every XCD
        b = busy(i) if busy else 0.5 * 1024 * (g / 8)          # 50% of 1024 SIMDs
        vals = counters(stage) if counters else (("GRBM_GUI_ACTIVE", g), ("SQ_VALU_MFMA_BUSY_CYCLES", b),
                                                 ("SQ_INSTS_MFMA", 1000.0))
        for name, val in vals:
            rows.append([d, NAMES[stage], name, val, start, start + ns])
        d += 1
    if copy is not None:
        rows.append([d, "__amd_rocclr_copyBuffer", copy[0], copy[1], 0, 10])
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(fields)
        w.writerows(rows)


def _plan():
    return [st for _ in bench.config_list(FI) for st in bench.STAGES for _ in range(bench.COUNTER_REPEATS)]


def test_ingest_sq_attributes_by_launch_order(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "SQ_FILE", str(tmp_path / "sq.json"))
    path = tmp_path / "c.csv"
    _write_csv(path, _plan())
    table = bench.ingest_sq(str(path))
    assert len(table) == len(bench.config_list(FI)) * len(bench.STAGES)
    for key, causal in bench.config_list(FI):
        for st in bench.STAGES:
            rec = table[f"{key}|{int(causal)}|{st}"]
            assert rec["dispatches"] == bench.COUNTER_REPEATS
            assert rec["clock_ghz"] == pytest.approx(1.5)
            assert rec["mfma_busy"] == pytest.approx(0.5)
            assert rec["us"] == pytest.approx(1000.0)
    with open(tmp_path / "sq.json") as f:
        assert json.load(f).keys() == table.keys()
    # the committed-table lookup sees the current sources
    rec = bench.counters_for("fwd", "llm_layer", True)
    assert rec is not None and rec["clock_ghz"] == pytest.approx(1.5)


def test_ingest_sq_refuses_a_wrong_order(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "SQ_FILE", str(tmp_path / "sq.json"))
    plan = _plan()
    plan[0], plan[-1] = plan[-1], plan[0]
    path = tmp_path / "c.csv"
    _write_csv(path, plan)
    with pytest.raises(SystemExit):
        bench.ingest_sq(str(path))
    _write_csv(path, _plan()[:-1])
    with pytest.raises(SystemExit):
        bench.ingest_sq(str(path))


def test_kernel_work_counts():
    w = FI.WORKLOADS["llm_layer"]
    F = 4.0 * 4 * 32 * 4096 * 4096 * 128 * 0.5
    assert bench.kernel_work("fwd", w, True)[1] == pytest.approx(F / 1e12)
    assert bench.kernel_work("bwd_dkv", w, True)[1] == pytest.approx(2 * F / 1e12)
    assert bench.kernel_work("bwd_dq_delta", w, True)[1] == pytest.approx(0.5 * F / 1e12)
    t, rows = 4 * 32 * 4096 * 128 * 2, 4 * 32 * 4096 * 4
    assert bench.algorithmic_bytes("bwd_dq_delta", w) == 6 * t + 2 * rows


def test_ingest_traffic_scales_by_the_copy(tmp_path, monkeypatch):
    """FETCH_SIZE / WRITE_SIZE per dispatch (KiB) scaled by what the same counter read for the
    copy of known size: a copy of 256 MiB that reads as 64 MiB fetched (factor 4) and 256 MiB
    written (factor 1)."""
    monkeypatch.setattr(bench, "SQ_FILE", str(tmp_path / "c.json"))
    sq, fe, wr = tmp_path / "sq.csv", tmp_path / "f.csv", tmp_path / "w.csv"
    _write_csv(sq, _plan())
    kib = {"fwd": 1000.0, "fwd_pingpong": 1100.0, "bwd_dkv": 3000.0, "bwd_dq_delta": 4000.0}
    _write_csv(fe, _plan(), counters=lambda st: (("FETCH_SIZE", kib[st]),), copy=("FETCH_SIZE", 64 * 1024.0))
    _write_csv(wr, _plan(), counters=lambda st: (("WRITE_SIZE", kib[st] / 2),), copy=("WRITE_SIZE", 256 * 1024.0))
    table = bench.ingest_traffic(str(fe), str(wr), 256, bench.ingest_sq(str(sq), write=False))
    rec = table["llm_layer|1|bwd_dkv"]
    assert rec["fetch_bytes"] == 4 * 3000 * 1024 and rec["write_bytes"] == 1500 * 1024
    assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert rec["clock_ghz"] == pytest.approx(1.5)
    assert table["_calibration"]["fetch_factor"] == pytest.approx(4.0)


def test_source_hash_ignores_comments_only():
    """The counter table is tied to a kernel's code: comments and layout may change, code may
    not. A changed comment or blank line keeps the text that is hashed; a changed token does not."""
    src = "int f(int x) {  // a comment\n  return x + 1;  // another\n}\n"
    assert bench.code_text(src) == bench.code_text("int f(int x) {\n\n  // reworded\n  return x + 1;\n}\n")
    assert bench.code_text(src) != bench.code_text(src.replace("x + 1", "x + 2"))
    assert "comment" not in bench.code_text(src)
    assert len(bench.source_sha("fwd")) == 16
