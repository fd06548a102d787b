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
    assert bench._short_name("void retopk::k_step<true>(retopk::Dims, retopk::Bufs const*, int)") == "k_step"


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
    # the counter run's own result line: its timed window and algorithmic bytes
    (tmp_path / "exact_FETCH_SIZE.json").write_text(json.dumps(
        {"steps": 4, "warmup": 2, "config": {"rotated_layers": 3},
         "roofline_exact": {"algorithmic_bytes_per_call": 200000}}))
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
    win = {"steps": 4, "warmup": 2, "layers": 3}
    assert row["window"] == win and row["algorithmic_bytes_per_launch"] == 200000
    # traffic only for a run over the same window; else the other window's row beside it
    assert bench.load_traffic("k_step", "w", "exact", win) == (210 * 1024, None)
    t, other = bench.load_traffic("k_step", "w", "exact", {**win, "steps": 20})
    assert t is None and other == {"window": win, "hbm_bytes_per_launch": 210 * 1024,
                                   "algorithmic_bytes_per_launch": 200000}
    assert bench.load_traffic("k_step", "w", "natural", win) == (None, None)
    # a later summary over another window keeps this row
    (tmp_path / "exact_FETCH_SIZE.json").write_text(json.dumps(
        {"steps": 20, "warmup": 5, "config": {"rotated_layers": 3},
         "roofline_exact": {"algorithmic_bytes_per_call": 200001}}))
    bench.summarize_traffic(str(tmp_path), 4, "w")
    doc = json.load(open(out / "profiles" / "traffic.json"))
    assert sorted(r["window"]["steps"] for r in doc["rows"]) == [4, 20]


def test_layer_offsets_spread_over_the_decode():
    # 25 layer-steps over 4 layers: layer 0 runs 7 positions, the others 6
    counts = [len(range(l, 25, 4)) for l in range(4)]
    offs = bench.layer_offsets(counts, 512)
    assert offs[0] == 0 and offs[-1] + counts[-1] == 512 and offs == sorted(offs)
    assert bench.layer_offsets([516] * 4, 516) == [0, 0, 0, 0]
    assert bench.layer_offsets([7], 512) == [0]
    offs = bench.layer_offsets([3] * 32, 256)
    assert offs[0] == 0 and offs[-1] + 3 == 256 and offs == sorted(offs)
