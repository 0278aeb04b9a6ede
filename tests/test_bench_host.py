"""Host logic of bench.py (CPU): the one-GPU guard, the HBM-traffic summary
from rocprofv3 counter files, and the rule that a summary taken on other
kernel sources is not reported."""
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
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kernel, counter, value in rows:
            w.writerow({"Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


@pytest.fixture
def traffic_env(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(tmp_path / "profiles")
    run = tmp_path / "run"
    k = "void opr::attn_dkdv_kernel<128>(opr::AttnParams, float*, float*)"
    # two dispatches per counter: the summary averages them
    _counter_csv(run / "fetch", [(k, "FETCH_SIZE", 1000.0), (k, "FETCH_SIZE", 3000.0),
                                 ("void other_kernel()", "FETCH_SIZE", 9e9)])
    _counter_csv(run / "write", [(k, "WRITE_SIZE", 500.0), (k, "WRITE_SIZE", 500.0)])
    # the probe copies 1 GiB: FETCH_SIZE counts half of it, WRITE_SIZE all of it (in KiB)
    _counter_csv(run / "copy_fetch", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0),
                                      ("__amd_rocclr_fillBufferAligned", "FETCH_SIZE", 1.0)])
    _counter_csv(run / "copy_write", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0)])
    return run


def test_traffic_summary_scales_by_the_copy_probe(traffic_env):
    bench.summarize_traffic(str(traffic_env), "attn_dkdv")
    d = json.load(open(bench.traffic_file("attn_dkdv")))
    assert d["fetch_kib_per_dispatch"] == 2000.0 and d["write_kib_per_dispatch"] == 500.0
    assert d["fetch_bytes_per_kib"] == 2048.0 and d["write_bytes_per_kib"] == 1024.0
    assert d["bytes_per_launch"] == 2000 * 2048 + 500 * 1024
    assert bench.load_traffic("attn_dkdv") == d["bytes_per_launch"]


def test_traffic_of_other_sources_is_not_reported(traffic_env):
    bench.summarize_traffic(str(traffic_env), "attn_dkdv")
    path = bench.traffic_file("attn_dkdv")
    d = json.load(open(path))
    d["source_sha"] = "0" * 16
    json.dump(d, open(path, "w"))
    assert bench.load_traffic("attn_dkdv") is None
    os.remove(path)
    assert bench.load_traffic("attn_dkdv") is None


def test_layout_traffic_sums_its_kernels(tmp_path, monkeypatch):
    # one opr_build_layout call is four dispatches: the summary adds the
    # per-dispatch average of each kernel
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(tmp_path / "profiles")
    run = tmp_path / "run"
    ks = ["opr::(anonymous namespace)::layout_prep(int, int, int, opr::LayoutWs)",
          "opr::(anonymous namespace)::layout_fill(int, int, opr::LayoutWs, opr_layout)",
          "void opr::(anonymous namespace)::layout_classify_attention<128, 128>(int, int, int, int, opr_layout)",
          "opr::(anonymous namespace)::layout_compact(int, int, int, opr_layout)"]
    _counter_csv(run / "fetch", [(k, "FETCH_SIZE", v) for k in ks for v in (10.0, 30.0)]
                 + [("void opr::attn_fwd_kernel<128>()", "FETCH_SIZE", 9e9)])
    _counter_csv(run / "write", [(k, "WRITE_SIZE", 100.0 * (i + 1)) for i, k in enumerate(ks)])
    _counter_csv(run / "copy_fetch", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0)])
    _counter_csv(run / "copy_write", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0)])
    bench.summarize_traffic(str(run), "layout")
    d = json.load(open(bench.traffic_file("layout")))
    assert bench.traffic_file("layout").endswith("layout_batch_traffic.json")
    assert d["workload"] == "layout_batch"
    assert d["fetch_kib_per_dispatch"] == 4 * 20.0 and d["write_kib_per_dispatch"] == 1000.0
    assert d["bytes_per_launch"] == 80 * 2048 + 1000 * 1024
    assert bench.load_traffic("layout") == d["bytes_per_launch"]
