"""bench.py's host-side contract (no GPU): it refuses more than one GPU with
a message, and it reports the counter-based HBM traffic only for the
workload and the kernel source the committed counter summary was taken on."""

import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_traffic_reported_for_its_workload_and_source_only(tmp_path, monkeypatch):
    rec = bench.recorded_traffic("518x378")
    assert rec is not None and rec > 3e8     # the committed summary matches the source
    assert bench.recorded_traffic("224x224") is None
    # the same summary against another kernel source: not reported
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0000000000000000")
    assert bench.recorded_traffic("518x378") is None
    # a missing or malformed summary: not reported
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.txt"))
    assert bench.recorded_traffic("518x378") is None
    bad = tmp_path / "bad.txt"
    bad.write_text("workload: 518x378\nkernel_source_sha256_16: 0000000000000000\n"
                   "hbm_bytes_per_launch: many\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(bad))
    assert bench.recorded_traffic("518x378") is None
