"""Host logic of bench.py, on the CPU: the HBM-traffic record built from rocprofv3
counter CSVs, the guard that drops counters taken on other GEMM sources, the flop
counts behind the roofline, and the refusal of more than one GPU."""
import csv
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

APPLY = "k_ns_gemm<2, muon::GemmCfg<256, 256, true, 32, 4>, true>"


def write_counters(path, rows):
    """rows: (dispatch id, kernel name, counter, value); two dimension rows per value,
    as the profiler reports one row per hardware instance."""
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, k, c, v in rows:
            for half in (0.25 * v, 0.75 * v):
                w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": half})


def test_summarize_traffic_scales_by_the_copy_calibration(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    gemm = f"void muon::{APPLY}(muon::NsArgs)"
    write_counters(tmp_path / "cf.csv", [(1, copy, "FETCH_SIZE", 524288.0)])     # 1 GiB read seen as 0.5 GiB
    write_counters(tmp_path / "cw.csv", [(1, copy, "WRITE_SIZE", 1048576.0)])    # 1 GiB written seen as 1 GiB
    write_counters(tmp_path / "rf.csv", [(7, gemm, "FETCH_SIZE", 1000.0), (9, gemm, "FETCH_SIZE", 3000.0),
                                         (8, "some_torch_kernel", "FETCH_SIZE", 5.0)])
    write_counters(tmp_path / "rw.csv", [(7, gemm, "WRITE_SIZE", 500.0), (9, gemm, "WRITE_SIZE", 700.0)])
    out = tmp_path / "rec.json"
    rec = bench.summarize_traffic(str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), str(tmp_path / "rf.csv"),
                                  str(tmp_path / "rw.csv"), str(out))
    assert rec["calibration"]["fetch_factor"] == 2.0 and rec["calibration"]["write_factor"] == 1.0
    assert list(rec["kernels"]) == [APPLY]  # torch kernels and the copy are left out
    k = rec["kernels"][APPLY]
    assert k["fetch_kib_per_dispatch"] == 2000 and k["write_kib_per_dispatch"] == 600
    # means over the two dispatches, KiB -> bytes, fetch doubled by the calibration
    assert k["hbm_bytes_per_dispatch"] == (2000 * 2.0 + 600 * 1.0) * 1024
    assert json.load(open(out)) == rec


def test_measured_traffic_is_dropped_for_other_sources_or_workloads(tmp_path, monkeypatch):
    assert bench.measured_traffic(APPLY, "bucket2048") is None
    committed = bench.measured_traffic(APPLY, "15b")
    if committed is None:
        pytest.skip("the committed counters belong to other GEMM sources")
    rec = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic_15b_h5120.json")))
    assert committed == rec["kernels"][APPLY]["hbm_bytes_per_dispatch"]
    # a copy of the tree whose GEMM sources differ by one byte: the counters say nothing
    fake = tmp_path / "root"
    csrc = fake / "matrix_orthogonalising_optimizer_02_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "matrix_orthogonalising_optimizer_02_amd", "csrc"), csrc)
    shutil.copytree(os.path.join(ROOT, "profiles"), fake / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(fake))
    assert bench.measured_traffic(APPLY, "15b") == committed
    with open(csrc / bench.GEMM_SOURCES[0], "a") as fh:
        fh.write("\n")
    assert bench.measured_traffic(APPLY, "15b") is None


def test_flop_counts():
    m, n = 5120, 15360
    assert bench.apply_flops(m, n) == 2.0 * m * m * n
    # per iteration: X X^T and B X count m^2 n and 2 m^2 n, A A counts m^3 (symmetric halves)
    assert bench.ns5_flops_sym(m, n, steps=1) == 3.0 * m * m * n + m ** 3
    assert bench.ns5_flops_sym(m, n) == 5 * bench.ns5_flops_sym(m, n, steps=1)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and "exactly one GPU" in r.stderr
