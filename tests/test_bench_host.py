"""Host-side checks of the bench's HBM-traffic bookkeeping (no GPU): the counter
summary scales each kernel's FETCH_SIZE and WRITE_SIZE by what the same counters
read for a plain copy of known size, and a recorded figure is used only while the
kernel's sources are unchanged."""
import csv
import json
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


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
    attn = "void srp::attn_bf16_kernel<128>(srp::AttnArgs)"
    gemm = "void srp::gemm_bf16_kernel<0, srp::GemmCfg<256, 256, 2, 4, 2, 64> >(srp::GemmArgs)"
    # two launches each; counters split over two rows (per-XCD instances) that add up
    _counter_csv(tmp_path / "fetch", [
        (1, attn, "FETCH_SIZE", 300.0), (1, attn, "FETCH_SIZE", 100.0),
        (2, gemm, "FETCH_SIZE", 1000.0),
        (3, attn, "FETCH_SIZE", 600.0),
        (4, gemm, "FETCH_SIZE", 3000.0)])
    _counter_csv(tmp_path / "write", [
        (1, attn, "WRITE_SIZE", 50.0), (2, gemm, "WRITE_SIZE", 70.0),
        (3, attn, "WRITE_SIZE", 150.0), (4, gemm, "WRITE_SIZE", 130.0)])
    # a 1 MiB copy: FETCH_SIZE reads half the bytes, WRITE_SIZE all of them
    _counter_csv(tmp_path / "cfetch", [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0)])
    _counter_csv(tmp_path / "cwrite", [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0)])
    return tmp_path


def _record(md):
    return json.loads(md.split("```json", 1)[1].split("```", 1)[0])


def test_summary_scales_by_the_copy_calibration(pmc_dirs):
    md = bench.summarize_pmc(str(pmc_dirs / "fetch"), str(pmc_dirs / "write"), str(pmc_dirs / "cfetch"),
                             str(pmc_dirs / "cwrite"), 1)
    rec = _record(md)
    assert rec["fetch_factor"] == pytest.approx(2.0) and rec["write_factor"] == pytest.approx(1.0)
    attn = rec["kernels"]["attn_bf16_kernel<128>"]
    # mean fetch (400 + 600) / 2 = 500 KiB x 2, mean write (50 + 150) / 2 = 100 KiB x 1
    assert attn["launches"] == 2
    assert attn["bytes_per_launch"] == pytest.approx((500 * 2 + 100) * 1024)
    kv = rec["kernels"]["gemm_bf16_kernel<EPI_KV>"]
    assert kv["bytes_per_launch"] == pytest.approx((2000 * 2 + 100) * 1024)
    # a kernel with no dispatches in the counter files is left out
    assert "gemm_bf16_kernel<EPI_Q>" not in rec["kernels"]
    assert attn["source_hash"] == bench.source_hash(bench.TRAFFIC_KERNELS["attn_bf16_kernel<128>"][1])


def test_recorded_traffic_only_for_unchanged_sources(pmc_dirs, tmp_path, monkeypatch):
    md = bench.summarize_pmc(str(pmc_dirs / "fetch"), str(pmc_dirs / "write"), str(pmc_dirs / "cfetch"),
                             str(pmc_dirs / "cwrite"), 1)
    f = tmp_path / "traffic.md"
    f.write_text("# traffic\n\n" + md)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic("attn_bf16_kernel<128>") == pytest.approx((500 * 2 + 100) * 1024)
    # the record of a kernel whose sources changed since is not used
    rec = _record(md)
    rec["kernels"]["attn_bf16_kernel<128>"]["source_hash"] = "0" * 16
    f.write_text("```json\n" + json.dumps(rec) + "\n```\n")
    assert bench.recorded_traffic("attn_bf16_kernel<128>") is None
    assert bench.recorded_traffic("gemm_bf16_kernel<EPI_KV>") == pytest.approx((2000 * 2 + 100) * 1024)
    # no record at all
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.recorded_traffic("attn_bf16_kernel<128>") is None

