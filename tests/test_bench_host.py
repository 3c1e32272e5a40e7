"""Host logic of bench.py (no GPU): the single-GPU guard, and the reduction of
rocprofv3 FETCH_SIZE / WRITE_SIZE records to the per-launch HBM bytes that
the bench reports as roofline.traffic.  The counter records here are
synthetic CSV files in rocprofv3's column layout."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test",
                                                  os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def write_counters(d, counter, rows):
    """rows: (kernel name, grid size, value in KiB) per dispatch."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "cnt_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        for i, (name, grid, kib) in enumerate(rows):
            w.writerow([i, name, grid, counter, kib])


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single-GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("op,kernel", [("decode", "decode_split_kernel<1, 128, 16, false, false>"),
                                       ("prefill", "prefill_kernel<1, 128, 2, 2, false>")])
def test_counter_summary_scales_by_the_copy(tmp_path, op, kernel):
    """FETCH_SIZE reads half of a copy's bytes on this ROCm and WRITE_SIZE all
    of them: each counter is scaled by copy bytes / what it read for the copy,
    and the kernel's figure is the mean over its dispatches."""
    b = bench_module()
    kib_copy = b.COPY_BYTES / 1024
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    name = f"void pa::(anonymous namespace)::{kernel}(int*)"
    small_copy = ("__amd_rocclr_copyBuffer", 512, 7.0)  # a small copy: not the calibration
    write_counters(fetch, "FETCH_SIZE", [(name, 65536, 100.0), (name, 65536, 140.0),
                                         ("__amd_rocclr_copyBuffer", 1 << 20, kib_copy / 2),
                                         small_copy])
    write_counters(write, "WRITE_SIZE", [(name, 65536, 3.0), (name, 65536, 5.0),
                                         ("__amd_rocclr_copyBuffer", 1 << 20, kib_copy),
                                         small_copy])
    rec = b.summarize_counters(fetch, write, "llama8b", False, op=op)
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes"] == pytest.approx(120.0 * 1024 * 2.0)
    assert rec["write_bytes"] == pytest.approx(4.0 * 1024)
    assert rec["traffic_bytes"] == pytest.approx(120.0 * 1024 * 2.0 + 4.0 * 1024)
    assert rec["source_sha256"] == b.kernel_source_hash(op)
    json.dumps(rec)  # the record is plain JSON


def test_counter_summary_needs_the_calibration_copy(tmp_path):
    b = bench_module()
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    name = "void pa::(anonymous namespace)::decode_split_kernel<1, 128, 16, false, false>(int*)"
    write_counters(fetch, "FETCH_SIZE", [(name, 65536, 100.0)])
    write_counters(write, "WRITE_SIZE", [(name, 65536, 3.0)])
    with pytest.raises(SystemExit):
        b.summarize_counters(fetch, write, "llama8b", False)


def test_recorded_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    """A counters record counts only for the workload it names and only while
    the kernel source hashes as recorded; otherwise traffic is null."""
    b = bench_module()
    path = tmp_path / "rec.txt"
    monkeypatch.setattr(b, "counters_path", lambda tag, op="decode": str(path))
    rec = {"workload": "llama8b", "source_sha256": b.kernel_source_hash("decode"),
           "traffic_bytes": 123.0}
    path.write_text(json.dumps(rec))
    assert b.recorded_traffic("llama8b") == 123.0
    assert b.recorded_traffic("long") is None
    path.write_text(json.dumps(dict(rec, source_sha256="0" * 64)))
    assert b.recorded_traffic("llama8b") is None
    path.write_text("not json")
    assert b.recorded_traffic("llama8b") is None
