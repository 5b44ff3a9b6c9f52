"""Host logic of bench.py, on the CPU: the one-GPU refusal, the HBM-traffic
figure from rocprofv3 counter tables (each counter scaled by what it reads
for a copy of known size), the check that counter readings belong to the
current kernel sources, the per-call distribution summary, the clock-reading
window and the plausibility check on the driver's clock reading."""
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
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def write_counter_csv(folder, counter, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_from_counters_scales_by_the_copy(tmp_path):
    gemm = "void rtl::(anonymous namespace)::sparse_gemm_kernel<0, true, 4, false>(...)"
    copy = "__amd_rocclr_copyBuffer"
    # The copy of 256 MiB reads as 250 MiB fetched and 260 MiB written; the
    # small uploads through the same kernel are left out (below 3/4 of the
    # largest); medians over the three launches of each kernel.
    mib = 1024.0
    write_counter_csv(tmp_path / "f", "FETCH_SIZE",
                      [(gemm, 100000.0), (gemm, 100002.0), (gemm, 99990.0),
                       (copy, 250 * mib), (copy, 250 * mib), (copy, 250 * mib), (copy, 12.0)])
    write_counter_csv(tmp_path / "w", "WRITE_SIZE",
                      [(gemm, 98000.0), (gemm, 98000.0), (gemm, 98000.0),
                       (copy, 260 * mib), (copy, 260 * mib), (copy, 260 * mib), (copy, 3.0)])
    t = bench.traffic_from_counters(str(tmp_path / "f"), str(tmp_path / "w"), "mlp_up")
    copy_bytes = float(256 << 20)
    want = 100000.0 * 1024 * copy_bytes / (250 * mib * 1024) + 98000.0 * 1024 * copy_bytes / (260 * mib * 1024)
    assert t["hbm_bytes_per_launch"] == round(want)
    assert t["fetch_size_kib"] == 100000.0 and t["write_size_kib"] == 98000.0
    assert t["copy_fetch_size_kib"] == 250 * mib and t["copy_write_size_kib"] == 260 * mib
    assert t["kernel_source_hash"] == bench.kernel_source_hash()


def test_traffic_needs_both_kernels(tmp_path):
    write_counter_csv(tmp_path / "f", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 5.0)])
    write_counter_csv(tmp_path / "w", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 5.0)])
    with pytest.raises(SystemExit):
        bench.traffic_from_counters(str(tmp_path / "f"), str(tmp_path / "w"), "mlp_up")


def test_traffic_of_other_sources_is_not_reported(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.load_traffic("mlp_up") is None                  # no file
    rec = {"hbm_bytes_per_launch": 123, "kernel_source_hash": bench.kernel_source_hash()}
    (tmp_path / "traffic_sparse_gemm_mlp_up.json").write_text(json.dumps(rec))
    assert bench.load_traffic("mlp_up")["hbm_bytes_per_launch"] == 123
    rec["kernel_source_hash"] = "0" * 16
    (tmp_path / "traffic_sparse_gemm_mlp_up.json").write_text(json.dumps(rec))
    assert bench.load_traffic("mlp_up") is None


def test_kernel_source_hash_follows_the_sources(tmp_path, monkeypatch):
    h0 = bench.kernel_source_hash()
    for f in bench.GEMM_SOURCES:
        (tmp_path / f).write_bytes(open(os.path.join(bench.CSRC, f), "rb").read())
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    assert bench.kernel_source_hash() == h0
    with open(tmp_path / bench.GEMM_SOURCES[0], "ab") as fh:
        fh.write(b"\n")
    assert bench.kernel_source_hash() != h0


def test_dist_summary():
    d = bench.dist([0.004, 0.001, 0.003, 0.002, 0.010])          # ms
    assert d == {"median": 3.0, "min": 1.0, "p90": 10.0, "mean": 4.0}   # us


def test_clock_window_picks_the_loop():
    c = object.__new__(bench.ClockSampler)
    c.samples = [(0.5, 2400.0), (1.0, 1800.0), (1.5, 1900.0), (2.0, 2000.0), (3.0, 100.0)]
    assert c.window(1.0, 2.0) == {"median": 1900.0, "min": 1800.0, "max": 2000.0, "readings": 3}
    assert c.window(4.0, 5.0) is None


def test_clock_reading_below_the_measured_rates_is_not_used():
    # 1900 MHz: peak 1992.3 TFLOP/s, above every measured dense-rate figure
    peak, note = bench.peak_at_clock(1900.0, (1017.3, 1268.2, 1450.4))
    assert note is None and abs(peak - bench.PEAK_BF16_DENSE_TFLOPS * 1900 / 2400) < 1e-9
    # 767.5 MHz: peak 804.8, below what hipBLASLt measurably did
    peak, note = bench.peak_at_clock(767.5, (1017.3, 1268.2, 1450.4))
    assert peak is None and "767.5 MHz" in note and "1383 MHz" in note
    assert bench.peak_at_clock(None, (1.0,)) == (None, None)
