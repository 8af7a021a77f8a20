"""Host-side parts of bench.py, on the CPU: the one-GPU refusal, the counter ingestion that
turns two rocprofv3 --pmc runs into HBM bytes per forward launch, and the keying of those
counters on the kernel code (a comment edit keeps them, a code change voids them)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for i, (kernel, value) in enumerate(rows):
            w.writerow(dict(Dispatch_Id=i, Kernel_Name=kernel, Counter_Name=counter,
                            Counter_Value=value))


def test_ingest_pmc_scales_each_counter_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    fwd, copy = "void llp::k_fwd<0, 8>(llp::FwdArgs)", "__amd_rocclr_copyBuffer"
    gib_kib = (1 << 30) / 1024
    # The copy of 1 GiB reads half its bytes in FETCH_SIZE and all of them in WRITE_SIZE; a
    # small copy and another kernel are in the runs too and must be ignored.
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                 [(copy, gib_kib / 2), (copy, 12.0), (fwd, 4.0e6), (fwd, 6.0e6),
                  ("void llp::k_combine(llp::CombineArgs)", 9.0e4)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                 [(copy, gib_kib), (copy, 4.0), (fwd, 3.0e4), (fwd, 3.0e4)])
    bench.ingest_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    d = json.load(open(tmp_path / "traffic.json"))
    assert d["kernel"] == fwd
    assert d["fetch_scale"] == pytest.approx(2.0) and d["write_scale"] == pytest.approx(1.0)
    assert d["fetch_kib_per_dispatch"] == pytest.approx(5.0e6)
    assert d["bytes_per_launch"] == pytest.approx((5.0e6 * 2.0 + 3.0e4) * 1024)
    assert d["kernel_source_hash"] == bench.kernel_source_hash()
    assert bench.measured_traffic() == pytest.approx(d["bytes_per_launch"])


def test_measured_traffic_is_void_for_other_kernel_code(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    path.write_text(json.dumps({"kernel_source_hash": "0" * 16, "bytes_per_launch": 1.0}))
    assert bench.measured_traffic() is None
    path.write_text(json.dumps({"kernel_source_hash": bench.kernel_source_hash(),
                                "bytes_per_launch": 1.0}))
    assert bench.measured_traffic() == 1.0
    path.write_text("not json")
    assert bench.measured_traffic() is None


def test_kernel_source_hash_ignores_comments_and_layout_only(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src)])
    src.write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    h0 = bench.kernel_source_hash()
    src.write_text("/* a block\n comment */ int f(int x)   {\n\n return x + 1;\n}  // other\n")
    assert bench.kernel_source_hash() == h0
    src.write_text("int f(int x) {\n  return x + 2;  // one\n}\n")
    assert bench.kernel_source_hash() != h0
