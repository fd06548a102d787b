"""Host-side logic of bench.py (CPU only): the one-GPU guard, kernel-name
parsing of profiler rows, per-dispatch counter grouping and the copy-scaled
HBM byte totals."""
import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_short_kernel_names():
    assert bench._short_name("retopk::k_step(retopk::Dims, retopk::Bufs const*, int)") == "k_step"
    assert bench._short_name("retopk::(anonymous namespace)::k_dense(retopk::Dims, int)") == "k_dense"
    assert bench._short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def _rows(counter, spec):
    """spec: (dispatch id, kernel, grid, value KiB) tuples -> profiler-like rows."""
    return [{"Counter_Name": counter, "Kernel_Name": k, "Dispatch_Id": str(i), "Grid_Size": str(g),
             "Counter_Value": str(v)} for i, k, g, v in spec]


def test_per_dispatch_keeps_the_last_calls_per_grid():
    k = "retopk::k_step(int)"
    spec = [(1, k, 100, 9.0), (2, k, 100, 1.0), (3, k, 200, 2.0), (4, k, 100, 3.0), (5, k, 200, 4.0)]
    got = bench._per_dispatch(_rows("FETCH_SIZE", spec), "FETCH_SIZE", last=2)
    # the last 2 calls of a kernel launched with two grids are its last 4 dispatches
    assert got[("k_step", 100)] == [1.0, 3.0]
    assert got[("k_step", 200)] == [2.0, 4.0]
    assert bench._per_dispatch(_rows("WRITE_SIZE", spec), "FETCH_SIZE") == {}


def _write_counters(d, counter, spec):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Counter_Name", "Kernel_Name", "Dispatch_Id", "Grid_Size",
                                          "Counter_Value"])
        w.writeheader()
        w.writerows(_rows(counter, spec))


def test_traffic_scaled_by_the_copy(tmp_path, monkeypatch):
    # the copy's counters read half (fetch) and all (write) of its bytes
    copy_kib = bench.COPY_BYTES / 1024
    for c, frac in (("FETCH_SIZE", 0.5), ("WRITE_SIZE", 1.0)):
        _write_counters(tmp_path / f"copy_{c}", c, [(i, "__amd_rocclr_copyBuffer", 64, copy_kib * frac)
                                                    for i in range(1, 4)])
    k = "retopk::k_step(int)"
    _write_counters(tmp_path / "exact_FETCH_SIZE", "FETCH_SIZE", [(i, k, 1000, 100.0) for i in range(1, 5)])
    _write_counters(tmp_path / "exact_WRITE_SIZE", "WRITE_SIZE", [(i, k, 1000, 10.0) for i in range(1, 5)])
    out = tmp_path / "repo"
    (out / "profiles").mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(out))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h")
    bench.summarize_traffic(str(tmp_path), 4, "w")
    doc = json.load(open(out / "profiles" / "traffic.json"))
    (row,) = doc["rows"]
    assert row["kernel"] == "k_step" and row["leg"] == "exact" and row["dispatches"] == 4
    assert row["fetch_bytes_per_launch"] == 2 * 100 * 1024
    assert row["write_bytes_per_launch"] == 10 * 1024
    assert bench.load_traffic("k_step", "w", "exact") == 210 * 1024
    assert bench.load_traffic("k_step", "w", "natural") is None
