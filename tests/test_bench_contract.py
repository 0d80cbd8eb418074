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


def _summary(path, workload="518x378", sha=None, nk=72441, nbytes="393488234"):
    path.write_text(f"# counters\nworkload: {workload}\n"
                    f"kernel_source_sha256_16: {sha or bench.kernel_hash()}\n"
                    f"visible_tokens: {nk}\nhbm_bytes_per_launch: {nbytes}\n")
    return str(path)


def test_traffic_reported_for_its_workload_source_and_window_only(tmp_path, monkeypatch):
    good = tmp_path / "good.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _summary(good))
    assert bench.recorded_traffic("518x378", 72441) == 393488234.0
    assert bench.recorded_traffic("518x378", 70000) == 393488234.0     # within 5%
    assert bench.recorded_traffic("224x224", 72441) is None             # other workload
    assert bench.recorded_traffic("518x378", 18600) is None             # other window
    # the same summary against another kernel source: not reported
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0000000000000000")
    assert bench.recorded_traffic("518x378", 72441) is None
    monkeypatch.undo()
    # a missing or malformed summary: not reported
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.txt"))
    assert bench.recorded_traffic("518x378", 72441) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _summary(tmp_path / "bad.txt", nbytes="many"))
    assert bench.recorded_traffic("518x378", 72441) is None


def test_committed_traffic_summary_names_its_window():
    kv = {}
    for line in open(bench.TRAFFIC_FILE):
        if ":" in line and not line.startswith(("#", "|")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    assert kv["workload"] == "518x378"
    assert 60000 < float(kv["visible_tokens"]) < 80000     # steady state
    assert float(kv["hbm_bytes_per_launch"]) > 3e8


def test_untimed_frames_fill_the_window():
    import synth
    # 8 scale + 64 window keyframes at interval 2: the 72nd keyframe is frame 142
    assert bench.fill_frames(synth.WORKLOADS["518x378"]) == 143
    assert bench.fill_frames(synth.WORKLOADS["224x224"]) == 72
    # the dynamic stream commits only accepted frames: 128 of them
    wl = synth.WORKLOADS["dynamic"]
    n = bench.fill_frames(wl)
    assert sum(synth.accept_decisions(wl, n)) == 128
    assert sum(synth.accept_decisions(wl, n - 1)) == 127
