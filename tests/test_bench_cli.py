"""Host-side checks of the benchmark script: the one-GPU contract and the HBM traffic
figure it derives from rocprofv3 counter files (synthetic files here)."""
import csv
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

DEC = "void nvfp4::(anonymous namespace)::decode_ring_kernel<128, 128, true>(nvfp4::AttnArgs)"
COPY = "__amd_rocclr_copyBuffer"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


def _counter_dir(tmp, name, counter, rows):
    d = tmp / name / "host"
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value", "Start_Timestamp", "End_Timestamp",
                                          "Grid_Size"])
        w.writeheader()
        for i, (kernel, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": kernel, "Counter_Name": counter,
                        "Counter_Value": value, "Start_Timestamp": 0, "End_Timestamp": 1000,
                        "Grid_Size": 256})
    return str(tmp / name)


def test_traffic_is_scaled_by_the_calibration_copy(tmp_path):
    """The copy of CALIB_BYTES calibrates each counter: a FETCH_SIZE that reads half the
    copied KiB doubles the kernel's reading, a WRITE_SIZE that reads all of it keeps it."""
    kib = bench.CALIB_BYTES / 1024
    fetch = _counter_dir(tmp_path, "f", "FETCH_SIZE",
                         [(COPY, kib / 2)] * 3 + [(DEC, 1000.0), (DEC, 1002.0)])
    write = _counter_dir(tmp_path, "w", "WRITE_SIZE", [(COPY, kib)] * 3 + [(DEC, 10.0)] * 2)
    out = tmp_path / "summary.txt"
    args = types.SimpleNamespace(summarize_pmc=[fetch, write], workload="batch_decode",
                                 command="synthetic", out=str(out))
    bench.summarize_pmc(args)
    text = out.read_text()
    rec = __import__("json").loads(text.strip().splitlines()[-1])
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["bytes_per_launch"] == round((1001.0 * 2 + 10.0) * 1024)
    assert rec["kernel"].startswith("decode_ring_kernel<128, 128, true>")
