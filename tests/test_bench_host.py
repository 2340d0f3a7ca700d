"""bench.py's host-side parts on the CPU: the one-GPU guard, the traffic
record written from rocprofv3 counter files, and the rule that retires that
record when the kernel source changes."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

DECODE_KERNEL = "void tv::(anonymous namespace)::paged_decode_seq_kernel<true>(tv::DecodeArgs)"
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def _counter_csv(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_record_from_counter_files(tmp_path):
    """Copy calibration: a 1 GiB copy reads FETCH_SIZE = 512 Ki KiB (half the
    bytes) and WRITE_SIZE = 1 Gi / 1 KiB, so the scales are 2 and 1; the
    kernel's means are scaled by them."""
    gib_kib = bench.COPY_CALIBRATION_BYTES / 1024
    _counter_csv(tmp_path / "fetch", "FETCH_SIZE",
                 [(DECODE_KERNEL, 100.0), (DECODE_KERNEL, 200.0), ("other", 7.0)])
    _counter_csv(tmp_path / "write", "WRITE_SIZE", [(DECODE_KERNEL, 10.0), (DECODE_KERNEL, 30.0)])
    _counter_csv(tmp_path / "copy_fetch", "FETCH_SIZE",
                 [(COPY_KERNEL, gib_kib / 2)] * 5 + [(COPY_KERNEL, 3.0)])
    _counter_csv(tmp_path / "copy_write", "WRITE_SIZE", [(COPY_KERNEL, gib_kib)] * 5)
    out = tmp_path / "record.json"
    rec = bench.write_traffic_record(str(tmp_path), 1, 512, out_path=str(out))
    assert rec["kernel"] == "paged_decode_seq_kernel<append>"
    assert rec["copy_calibration"]["fetch_scale"] == 2.0
    assert rec["copy_calibration"]["write_scale"] == 1.0
    (name, w), = rec["workloads"].items()
    assert name == "decode-b1-ctx37"
    assert w["hbm_read_bytes_per_launch"] == 150 * 1024 * 2
    assert w["hbm_write_bytes_per_launch"] == 20 * 1024
    assert w["hbm_bytes_per_launch"] == 150 * 2048 + 20 * 1024
    assert json.loads(out.read_text()) == rec
    # The record is read back only for its kernel, its workload and an
    # unchanged kernel source.
    kernel = "paged_decode_seq_kernel<append>"
    assert bench.measured_traffic(name, kernel, path=str(out)) == w["hbm_bytes_per_launch"]
    assert bench.measured_traffic(name, "paged_decode_kernel<append>", path=str(out)) is None
    assert bench.measured_traffic("decode-b64-ctx512-4096", kernel, path=str(out)) is None
    rec["kernel_source_sha256"] = "0" * 64
    out.write_text(json.dumps(rec))
    assert bench.measured_traffic(name, kernel, path=str(out)) is None


def test_source_digest_ignores_comments_and_blank_space(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f() {\n  return 1; // one\n}\n")
    b.write_text("/* header */\nint f() { return 1; }\n\n")
    c.write_text("int f() { return 2; }\n")
    assert bench.source_digest(str(a)) == bench.source_digest(str(b))
    assert bench.source_digest(str(a)) != bench.source_digest(str(c))


def test_missing_counter_files_are_an_error(tmp_path):
    with pytest.raises(FileNotFoundError):
        bench.write_traffic_record(str(tmp_path), 1, 512, out_path=str(tmp_path / "r.json"))
