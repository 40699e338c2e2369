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


def test_counter_summary_derivations(tmp_path):
    """Derived figures of the SQ counter summary on synthetic passes: a kernel of 1 ms
    (2.4 M cycles at the nominal clock) on 1024 SIMDs whose MFMAs keep the matrix
    units busy 25 % of the time."""
    cyc = 1e-3 * bench.CLOCK_GHZ * 1e9
    mfma = 1000.0
    counters = {"SQ_VALU_MFMA_BUSY_CYCLES": 0.25 * bench.SIMDS * cyc, "SQ_INSTS_MFMA": mfma,
                "SQ_INSTS_VALU": 4 * mfma, "SQ_INSTS_SALU": 2 * mfma,
                "SQ_WAVE_CYCLES": 18 * mfma}
    d = tmp_path / "p" / "host"
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value", "Start_Timestamp", "End_Timestamp",
                                          "Grid_Size"])
        w.writeheader()
        for c, v in counters.items():
            w.writerow({"Dispatch_Id": 1, "Kernel_Name": "prefill_coop_kernel<128, 128>",
                        "Counter_Name": c, "Counter_Value": v, "Start_Timestamp": 0,
                        "End_Timestamp": 1_000_000, "Grid_Size": 64 * 10})
    out = tmp_path / "s.txt"
    args = types.SimpleNamespace(summarize_counters=[str(tmp_path / "p")], kernel="prefill_coop_kernel",
                                 workload="w", command="synthetic", out=str(out))
    bench.summarize_counters(args)
    der = __import__("json").loads(out.read_text().strip().splitlines()[-1])["derived"]
    assert der["mfma_busy_share"] == pytest.approx(0.25, rel=1e-4)
    assert der["mfma_per_wave"] == pytest.approx(mfma / 10)
    assert der["other_valu_per_mfma"] == pytest.approx(3.0)
    assert der["sq_insts_salu_per_mfma"] == pytest.approx(2.0)
    # wave cycles count in units of four cycles
    assert der["sq_wave_cycles_cycles_per_mfma"] == pytest.approx(72.0)


def test_counter_summary_measures_the_clock(tmp_path):
    """With GRBM_GUI_ACTIVE in a pass (summed over 8 XCCs) the summary derives the engine
    clock from it instead of assuming 2.4 GHz: a 1 ms kernel at 2.1 GHz whose MFMAs keep
    the matrix units busy 40 % of the measured cycles."""
    clock = 2.1e9
    cyc = 1e-3 * clock
    counters = {"SQ_VALU_MFMA_BUSY_CYCLES": 0.4 * bench.SIMDS * cyc, "SQ_INSTS_MFMA": 100.0,
                "GRBM_GUI_ACTIVE": bench.XCCS * cyc, "MfmaUtil": 40.0}
    d = tmp_path / "p" / "host"
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value", "Start_Timestamp", "End_Timestamp",
                                          "Grid_Size"])
        w.writeheader()
        for c, v in counters.items():
            w.writerow({"Dispatch_Id": 1, "Kernel_Name": "prefill_coop_kernel<128, 128>",
                        "Counter_Name": c, "Counter_Value": v, "Start_Timestamp": 0,
                        "End_Timestamp": 1_000_000, "Grid_Size": 64 * 10})
    out = tmp_path / "s.txt"
    args = types.SimpleNamespace(summarize_counters=[str(tmp_path / "p")], kernel="prefill_coop_kernel",
                                 workload="w", command="synthetic", out=str(out))
    bench.summarize_counters(args)
    rec = __import__("json").loads(out.read_text().strip().splitlines()[-1])
    assert rec["clock"] == "measured"
    assert rec["derived"]["clock_ghz"] == pytest.approx(2.1, rel=1e-4)
    assert rec["derived"]["mfma_busy_share"] == pytest.approx(0.4, rel=1e-4)
    assert rec["derived"]["rocprof_mfma_util_share"] == pytest.approx(0.4)


def test_variant_traffic_record_names_the_plain_kernel(tmp_path):
    """A --variant counter run has no append launch: the record takes the plain decode
    kernel and prices it against the variant's own algorithmic bytes."""
    kib = bench.CALIB_BYTES / 1024
    plain = "decode_ring_kernel<128, 128, false, 0>(nvfp4::AttnArgs)"
    fetch = _counter_dir(tmp_path, "f", "FETCH_SIZE", [(COPY, kib)] * 3 + [(plain, 500.0)] * 2)
    write = _counter_dir(tmp_path, "w", "WRITE_SIZE", [(COPY, kib)] * 3 + [(plain, 8.0)] * 2)
    out = tmp_path / "summary.txt"
    args = types.SimpleNamespace(summarize_pmc=[fetch, write], workload="batch_decode",
                                 command="synthetic", out=str(out), variant="NHD_page16")
    bench.summarize_pmc(args)
    rec = __import__("json").loads(out.read_text().strip().splitlines()[-1])
    assert rec["variant"] == "NHD_page16" and rec["kernel"].startswith("decode_ring_kernel")
    w = bench.variant_workload(bench.synth_module(), "batch_decode", "NHD_page16")[0]
    kv, qo = bench.decode_bytes(w)
    assert rec["algorithmic_bytes"] == kv + qo
    assert rec["traffic_over_algorithmic"] == pytest.approx(508.0 * 1024 / (kv + qo), abs=1e-4)
