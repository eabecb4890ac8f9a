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


def test_rotation_order_never_rereads_a_warm_copy():
    # warm-up, timed and per-call calls read one sequence over the copies
    R, warmup, steps, per_call = 5, 7, 4, 3
    w, t, p = bench.rotation_order(R, warmup, steps, per_call)
    assert w == [0, 1, 2, 3, 4, 0, 1]
    assert t == [2, 3, 4, 0]
    assert p == [1, 2, 3]
    seq = w + t + p
    for i in range(len(seq)):
        # a copy comes back only after all R copies have been read
        later = seq[i + 1:i + R]
        assert seq[i] not in later


TRACE_FIELDS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id",
                "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size",
                "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X",
                "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]


def test_trace_summary(tmp_path):
    d = tmp_path / "ktrace"
    os.makedirs(d)
    kern = "void topk::(anonymous namespace)::topk_col_kernel<topk::Bf16, 4>(topk::ColArgs)"
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=TRACE_FIELDS)
        wr.writeheader()
        t = 1_000_000
        for i, dur in enumerate([1000, 2000, 3000, 4000, 5000] + [777]):
            name = kern if i < 5 else "__amd_rocclr_copyBuffer"
            wr.writerow({"Kind": "KERNEL_DISPATCH", "Dispatch_Id": i + 1, "Kernel_Name": name,
                         "Start_Timestamp": t, "End_Timestamp": t + dur, "LDS_Block_Size": 23328,
                         "Scratch_Size": 0, "VGPR_Count": 40, "Accum_VGPR_Count": 0, "SGPR_Count": 112,
                         "Workgroup_Size_X": 256, "Grid_Size_X": 259 * 256})
            t += 10_000
    out = bench.summarize_trace(str(d), 2, out_dir=str(tmp_path))
    (name, k), = out["kernels"].items()
    assert name == "topk_col_kernel<topk::Bf16, 4>"
    assert k["calls"] == 5 and k["mean_us"] == pytest.approx(3.0) and k["median_us"] == pytest.approx(3.0)
    assert k["min_us"] == pytest.approx(1.0) and k["max_us"] == pytest.approx(5.0)
    assert out["kernel_sources_digest"] == bench.kernel_sources_digest("col")
    md = open(tmp_path / "topk_col_kernel_cfg2_ktrace.md").read()
    assert "| 5 | 3.000 | 3.000 |" in md and "259 x 256" in md


def test_read_request_bytes(tmp_path):
    kern = "topk_col_kernel<topk::Bf16, 4>"
    copy = "__amd_rocclr_copyBuffer"
    d = tmp_path / "rdreq"
    os.makedirs(d)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=FIELDS)
        wr.writeheader()
        n = 0
        for name, counts in ((kern, (110, 0, 10, 100)), (kern, (110, 0, 10, 100)),
                             (copy, (bench.COPY_BYTES // 128, 0, 0, bench.COPY_BYTES // 128))):
            n += 1
            for counter, v in zip(bench.READREQ_COUNTERS.split(), counts):
                wr.writerow({"Correlation_Id": n, "Dispatch_Id": n, "Kernel_Name": name, "Counter_Name": counter,
                             "Counter_Value": v})
    out = bench.summarize_readreq(str(d), 2, out_path=str(tmp_path / "rr.md"))
    assert out[kern]["bytes"] == 10 * 64 + 100 * 128
    assert out["copy"]["bytes"] == bench.COPY_BYTES


def test_sq_summary_per_wave(tmp_path):
    kern = "topk_col_kernel<topk::Bf16, 4>"
    d1, d2 = tmp_path / "sq1", tmp_path / "sq2"
    write_counters(d1, "SQ_WAVES", [(kern, 1036.0)] * 3)
    write_counters(d2, "SQ_INSTS_VALU", [(kern, 1036.0 * 300)] * 3)
    bench.summarize_sq([str(d1), str(d2)], 2, out_path=str(tmp_path / "sq.md"))
    md = open(tmp_path / "sq.md").read()
    assert "| SQ_INSTS_VALU | 310,800 | 300 |" in md
