"""Host-side logic of bench.py, on the CPU: the one-GPU refusal and the
arithmetic that turns rocprofv3 FETCH_SIZE / WRITE_SIZE counters into HBM
bytes per launch (the roofline's traffic figure)."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_counters(directory, counter, rows):
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows, start=1):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_counter_scaling(tmp_path):
    # The calibration copy moves COPY_BYTES each way.  FETCH_SIZE reads half
    # of that (scale 2), WRITE_SIZE all of it (scale 1); the kernel's own
    # KiB per dispatch are scaled the same way.
    kern = "void topk::(anonymous namespace)::topk_col_kernel<topk::Bf16, 4>(topk::ColArgs)"
    copy = "__amd_rocclr_copyBuffer"
    half, full = bench.COPY_BYTES / 2048.0, bench.COPY_BYTES / 1024.0
    fetch = [(kern, 1800.0), (kern, 1810.0), (kern, 1790.0)] + [(copy, half)] * 5
    write = [(kern, 25.0), (kern, 25.0), (kern, 26.0)] + [(copy, full)] * 5
    write_counters(tmp_path / "fetch", "FETCH_SIZE", fetch)
    write_counters(tmp_path / "write", "WRITE_SIZE", write)
    out = bench.summarize_counters(str(tmp_path / "fetch"), str(tmp_path / "write"), 2,
                                   out_path=str(tmp_path / "traffic.json"))
    assert out["counters"]["FETCH_SIZE"]["scale"] == pytest.approx(2.0)
    assert out["counters"]["WRITE_SIZE"]["scale"] == pytest.approx(1.0)
    # medians: 1800 KiB fetched x 2, 25 KiB written x 1
    assert out["hbm_bytes_per_launch"] == 1800 * 1024 * 2 + 25 * 1024
    assert out["algorithmic_bytes"] == 248046 * 7 * 2 + 7 * 8 * (2 + 4)
    assert os.path.exists(tmp_path / "traffic.json")


def test_missing_calibration_is_an_error(tmp_path):
    kern = "topk_col_kernel<topk::Bf16, 4>"
    write_counters(tmp_path / "fetch", "FETCH_SIZE", [(kern, 1800.0)])
    write_counters(tmp_path / "write", "WRITE_SIZE", [(kern, 25.0)])
    with pytest.raises(SystemExit):
        bench.summarize_counters(str(tmp_path / "fetch"), str(tmp_path / "write"), 2,
                                 out_path=str(tmp_path / "traffic.json"))
