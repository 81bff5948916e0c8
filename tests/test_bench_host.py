"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the copy-calibrated scaling
of the fabric-byte counters, and the source check that keeps stale counters off the line."""
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
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (kernel, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_scaling_and_source_check(tmp_path, monkeypatch):
    """The copy reads and writes 1 GiB per launch; its FETCH_SIZE reads half of that (KiB per
    dispatch), WRITE_SIZE all of it, so kernel counts scale by 2 and 1.  The file is used only
    while its source hash and workload match."""
    gib_kib = (1 << 30) / 1024.0
    copy = "__amd_rocclr_copyBuffer(void*, void*)"
    kern = "void dsa3d::k_dq_qs<128, 3, 3>(unsigned short const*)"
    f, w, cf, cw = (str(tmp_path / n) for n in ("f.csv", "w.csv", "cf.csv", "cw.csv"))
    _counter_csv(f, "FETCH_SIZE", [(kern, 1000.0), (kern, 3000.0)])      # mean 2000 KiB per dispatch
    _counter_csv(w, "WRITE_SIZE", [(kern, 500.0)])
    _counter_csv(cf, "FETCH_SIZE", [(copy, gib_kib / 2)] * 3 + [("other_small", 1.0)])
    _counter_csv(cw, "WRITE_SIZE", [(copy, gib_kib)] * 3)
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda: "abc")
    out = bench.write_traffic(f, w, cf, cw, "C5-256f")
    assert out["fetch_scale"] == pytest.approx(2.0)
    assert out["write_scale"] == pytest.approx(1.0)
    e = out["kernels"]["k_dq_qs"]
    assert e["read_bytes"] == pytest.approx(2000 * 1024 * 2.0)
    assert e["write_bytes"] == pytest.approx(500 * 1024)
    assert e["hbm_bytes_per_launch"] == pytest.approx(e["read_bytes"] + e["write_bytes"])
    assert json.load(open(tmp_path / "profiles" / "traffic.json"))["source_hash"] == "abc"
    assert bench.measured_traffic("k_dq_qs", "C5-256f") == pytest.approx(e["hbm_bytes_per_launch"])
    assert bench.measured_traffic("k_dq_qs", "C3") is None        # another workload
    assert bench.measured_traffic("k_forward_qs", "C5-256f") is None  # not counted
    monkeypatch.setattr(bench, "source_hash", lambda: "changed")
    assert bench.measured_traffic("k_dq_qs", "C5-256f") is None   # kernels changed since


def test_committed_traffic_matches_the_sources():
    """profiles/traffic.json was taken on the kernel sources in the tree."""
    d = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert d["source_hash"] == bench.source_hash()
    assert bench.measured_traffic("k_dq_qs", d["workload"]) is not None
