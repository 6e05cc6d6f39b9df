"""Host-side checks of the bench's profile bookkeeping (no GPU): the counter
summary scales each stage's FETCH_SIZE and WRITE_SIZE by what the same counters
read for a plain copy of known size, both summaries cover only the last layer
calls of a run (cut at the anchor kernel launched once per call), a stage's
figure is the sum of its kernels per call, and a recorded figure is used only
while the stage's kernel sources are unchanged."""
import csv
import json
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

ATTN = "void srp::attn_bf16_kernel<128>(srp::AttnArgs)"
GEMM = "void srp::gemm_bf16_kernel<0, srp::GemmCfg<256, 256, 2, 4, 2, 64> >(srp::GemmArgs)"
FIX = "void srp::gemm_fixup_kernel<0, srp::GemmCfg<256, 256, 2, 4, 2, 64> >(srp::GemmArgs)"
META = "srp::row_meta_kernel(srp::SelectArgs, srp::Workspace)"


def _counter_csv(path, rows):
    """rocprofv3 counter_collection.csv layout: one row per (dispatch, counter)."""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for d, name, counter, value in rows:
            wr.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


@pytest.fixture
def pmc_dirs(tmp_path):
    # three layer calls (K/V GEMM, fix-up, attention: the counter runs record only
    # the MFMA stages and cut at the K/V GEMM); the first is a warm-up that the
    # summary of the last two leaves out; counters split over two rows (per-XCD
    # instances) add up
    fetch, write = [], []
    for c, (fa, fg, ff) in enumerate([(9999.0, 9999.0, 9999.0), (400.0, 1000.0, 40.0), (600.0, 3000.0, 60.0)]):
        d = 10 * c
        fetch += [(d + 1, GEMM, "FETCH_SIZE", fg / 2), (d + 1, GEMM, "FETCH_SIZE", fg / 2),
                  (d + 2, FIX, "FETCH_SIZE", ff), (d + 3, ATTN, "FETCH_SIZE", fa)]
        write += [(d + 1, GEMM, "WRITE_SIZE", 100.0), (d + 2, FIX, "WRITE_SIZE", 20.0),
                  (d + 3, ATTN, "WRITE_SIZE", 100.0)]
    _counter_csv(tmp_path / "fetch", fetch)
    _counter_csv(tmp_path / "write", write)
    # a 1 MiB copy: FETCH_SIZE reads half the bytes, WRITE_SIZE all of them
    _counter_csv(tmp_path / "cfetch", [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0)])
    _counter_csv(tmp_path / "cwrite", [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0)])
    return tmp_path


def _record(md):
    return json.loads(md.split("```json", 1)[1].split("```", 1)[0])


def _pmc(pmc_dirs, calls=2):
    return bench.summarize_pmc(str(pmc_dirs / "fetch"), str(pmc_dirs / "write"), str(pmc_dirs / "cfetch"),
                               str(pmc_dirs / "cwrite"), 1, calls)


def test_traffic_summary_scales_by_the_copy_calibration(pmc_dirs):
    rec = _record(_pmc(pmc_dirs))
    assert rec["fetch_factor"] == pytest.approx(2.0) and rec["write_factor"] == pytest.approx(1.0)
    attn = rec["stages"]["attention"]
    # last two calls: fetch (400 + 600) / 2 = 500 KiB x 2, write 100 KiB x 1
    assert attn["bytes_per_call"] == pytest.approx((500 * 2 + 100) * 1024)
    # the K/V stage adds its fix-up kernel: fetch (1040 + 3060) / 2, write 120
    kv = rec["stages"]["kv_proj"]
    assert kv["bytes_per_call"] == pytest.approx((2050 * 2 + 120) * 1024)
    assert "q_proj" not in rec["stages"] and "select" not in rec["stages"]  # no dispatches of them
    assert attn["source_hash"] == bench.source_hash(bench.STAGE_KERNELS["attention"][1])
    with pytest.raises(SystemExit):
        _pmc(pmc_dirs, calls=4)  # more calls than the record holds


def test_trace_summary_per_layer_call(tmp_path):
    rows, t = [], 0
    for c, (kv, fx, at) in enumerate([(900, 90, 900), (300, 20, 500), (340, 40, 700)]):
        for name, dur in [(META, 5), (GEMM, kv), (FIX, fx), (ATTN, at)]:
            rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur * 1000})
            t += dur * 1000 + 10
    path = tmp_path / "kernel_trace.csv"
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        wr.writerows(rows)
    rec = _record(bench.summarize_trace(str(path), 2))
    assert rec["stages"]["kv_proj"]["avg_ms"] == pytest.approx((300 + 20 + 340 + 40) / 2 / 1000)
    assert rec["stages"]["attention"]["avg_ms"] == pytest.approx(0.6)
    assert rec["kernel_ms_per_call"] == pytest.approx((5 + 300 + 20 + 500 + 5 + 340 + 40 + 700) / 2 / 1000)


def test_trace_window_counts_calls_opened_by_either_prepare_kernel(tmp_path):
    # a stack: the first layer call opens with the row metadata kernel, later ones
    # (candidate lists) with the one-group prepare kernel; both mark a call
    prep = "srp::prepare_one_group_kernel(srp::SelectArgs, srp::Workspace)"
    rows, t = [], 0
    for c, opener in enumerate([META, prep, prep, META, prep, prep]):
        for name, dur in [(opener, 5), (GEMM, 100 + c), (ATTN, 200)]:
            rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur * 1000})
            t += dur * 1000 + 10
    path = tmp_path / "kernel_trace.csv"
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        wr.writerows(rows)
    rec = _record(bench.summarize_trace(str(path), 3))  # the last three calls
    assert rec["stages"]["kv_proj"]["avg_ms"] == pytest.approx((103 + 104 + 105) / 3 / 1000)
    assert rec["stages"]["prepare"]["avg_ms"] == pytest.approx(0.005)
    with pytest.raises(SystemExit):
        bench.summarize_trace(str(path), 7)


def test_recorded_figures_only_for_unchanged_sources(pmc_dirs, tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    md = _pmc(pmc_dirs)
    (tmp_path / "hbm_traffic_demo.md").write_text("# traffic\n\n" + md)
    assert bench.recorded_stage("demo", "traffic", "attention") == pytest.approx((500 * 2 + 100) * 1024)
    # the record of a stage whose sources changed since is not used
    rec = _record(md)
    rec["stages"]["attention"]["source_hash"] = "0" * 16
    (tmp_path / "hbm_traffic_demo.md").write_text("```json\n" + json.dumps(rec) + "\n```\n")
    assert bench.recorded_stage("demo", "traffic", "attention") is None
    assert bench.recorded_stage("demo", "traffic", "kv_proj") == pytest.approx((2050 * 2 + 120) * 1024)
    # no record at all
    assert bench.recorded_stage("missing", "trace", "attention") is None
