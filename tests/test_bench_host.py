"""Host logic of bench.py (no GPU): the one-GPU guard and the rocprofv3 counter summary that
turns FETCH_SIZE / WRITE_SIZE runs into bytes per launch."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus above 1 is not supported" in r.stderr


def write_counters(path, counter, rows):
    """rows: (dispatch id, kernel id, kernel name, value in KiB)."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for d, k, n, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Id": k, "Kernel_Name": n, "Counter_Name": counter,
                        "Counter_Value": v})


def test_counter_means_split_same_names_and_stop_at_the_mixer(tmp_path):
    p = tmp_path / "c.csv"
    rows = [(1, 7, "vectorized_elementwise_kernel", 524288.0),       # the calibration copy
            (2, 10, "ssd_scan64_kernel", 100.0), (3, 10, "ssd_scan64_kernel", 300.0),
            (4, 11, "ssd_scan64_kernel", 50.0),                         # a second instance
            (5, 12, "conv1d_kernel", 8.0),
            (6, 30, "Cijk_Alik_Bljk_gemm", 1e6),                        # the mixer starts here
            (7, 10, "ssd_scan64_kernel", 9e9)]                          # not counted
    write_counters(p, "FETCH_SIZE", rows)
    means, calib = bench._counter_means(str(p), "FETCH_SIZE")
    assert calib == 524288.0
    assert means["ssd_scan64_kernel#0"] == 200.0      # first dispatched instance
    assert means["ssd_scan64_kernel#1"] == 50.0
    assert means["conv1d_kernel"] == 8.0
    assert not any("Cijk" in k for k in means)


def test_summarize_scales_by_the_calibration(tmp_path, monkeypatch):
    """The fetch counter reads half the copy's 1 GiB, the write counter all of it: fetch
    counts are doubled, write counts kept; a kernel's bytes are KiB * 1024 * factor."""
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    names = [(3, 1, "ssd_prep_kernelIDF16bLi64ELb1ELb0E"), (4, 2, "ssd_scan64_kernel"),
             (5, 3, "ssd_prep_kernelIDF16bLi64ELb0ELb0E"), (6, 4, "ssd_scan64_kernel"),
             (7, 5, "conv1d_kernel"), (8, 6, "state_update_kernel"), (9, 8, "group_rmsnorm_kernel")]
    write_counters(fetch, "FETCH_SIZE", [(1, 9, "vectorized_elementwise_kernel", 524288.0)] +
                   [(d, k, n, 1000.0 * k) for d, k, n in names])
    write_counters(write, "WRITE_SIZE", [(1, 9, "vectorized_elementwise_kernel", 1048576.0)] +
                   [(d, k, n, 10.0 * k) for d, k, n in names])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    out = bench.summarize_counters(str(fetch), str(write), 64)
    cal = out["_calibration"]
    assert cal["fetch_factor"] == pytest.approx(2.0) and cal["write_factor"] == pytest.approx(1.0)
    one_call = out["conv_ssd_prefill"]                   # prep (kernel 1) + first scan (kernel 2)
    assert one_call["fetch_bytes"] == pytest.approx((1000 + 2000) * 1024 * 2.0)
    assert one_call["write_bytes"] == pytest.approx((10 + 20) * 1024)
    two_call = out["ssd_prefill"]                        # prep (kernel 3) + second scan (kernel 4)
    assert two_call["fetch_bytes"] == pytest.approx((3000 + 4000) * 1024 * 2.0)
    assert out["state_update"]["bytes_per_launch"] == pytest.approx(6000 * 1024 * 2.0 + 60 * 1024)
    assert json.load(open(tmp_path / "traffic.json"))["conv1d"]["source_hash"] == bench.kernel_source_hash("conv1d")
