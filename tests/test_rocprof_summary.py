"""Host-side checks of the rocprofv3 summary tool that feeds bench.py's
roofline traffic: counter averaging per kernel, the copy calibration, the
source-hash gate, and the kernel-trace table."""

import csv
import json

from block_sparse_attention_32_amd import rocprof_summary as R

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, name, counter, value in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_traffic_scales_by_copy_calibration(tmp_path):
    kern = "void qsa::attn_mfma_kernel<128, false, false>(qsa::AttnArgs)"
    copy = "__amd_rocclr_copyBuffer"
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    # the 256 MiB copy reads half its size on FETCH_SIZE (factor 2) and the
    # full size on WRITE_SIZE (factor 1); a small copy must be ignored
    _counters(fetch, [(1, copy, "FETCH_SIZE", 131072.0), (2, copy, "FETCH_SIZE", 10.0),
                      (3, kern, "FETCH_SIZE", 1000.0), (4, kern, "FETCH_SIZE", 3000.0),
                      (4, kern, "WRITE_SIZE", 5.0)])
    _counters(write, [(1, copy, "WRITE_SIZE", 262144.0), (3, kern, "WRITE_SIZE", 100.0),
                      (4, kern, "WRITE_SIZE", 300.0)])
    d = R.traffic_summary(str(fetch), str(write), "attn_mfma_kernel", "wl",
                          ["attention_mfma.hip"], "cmd-f", "cmd-w")
    assert d["fetch_kib_per_dispatch_raw"] == 2000.0
    assert d["copy_calibration"]["fetch_factor"] == 2.0
    assert d["copy_calibration"]["write_factor"] == 1.0
    assert d["fetch_bytes_per_launch"] == 2000 * 1024 * 2
    assert d["write_bytes_per_launch"] == 200 * 1024
    assert d["hbm_bytes_per_launch"] == 2000 * 1024 * 2 + 200 * 1024
    assert d["dispatches"] == {"fetch_run": 2, "write_run": 2}
    assert d["source_hash"] == R.source_hash("attention_mfma.hip")


def test_traffic_gated_by_source_hash(tmp_path, monkeypatch):
    monkeypatch.setattr(R, "PROFILES", str(tmp_path))
    h = R.source_hash("attention_mfma.hip", "attention.hpp")
    (tmp_path / "k_wl_traffic.json").write_text(json.dumps(
        {"source_hash": h, "hbm_bytes_per_launch": 1234}))
    assert R.traffic_for("k", "wl", h) == 1234
    assert R.traffic_for("k", "wl", "0" * 16) is None       # kernel changed since
    assert R.traffic_for("other", "wl", h) is None           # no summary


def test_trace_summary_table(tmp_path):
    stats = tmp_path / "s.csv"
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                          "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writeheader()
        w.writerow({"Name": "void qsa::pool_kernel<unsigned short, 64>(qsa::PoolArgs)",
                    "Calls": 4, "TotalDurationNs": 8000, "AverageNs": 2000, "Percentage": 100,
                    "MinNs": 1500, "MaxNs": 2500, "StdDev": 1})
    text = R.trace_summary(str(stats), "wl", "the command")
    assert "# command: the command" in text
    line = text.strip().splitlines()[-1].split()
    assert line[0] == "4" and line[1] == "0.008" and line[2] == "2.00"
    assert text.rstrip().endswith("qsa::pool_kernel<unsigned short, 64>")
