"""The boundary from plain C: tests/c_abi_client.c includes include/spkv.h,
is built with gcc as C99 with warnings as errors, links libspkv.so and
drives a host-only handle (no GPU).  Its per-frame plans, free lists and
stats must equal the tiny worked example in tests/golden (derived by hand
from the pages' rules), and the codes of its other calls must be the ones
the header's contract fixes."""

import json
import os
import shutil
import subprocess

import pytest

from conftest import ROOT
import streaming_paged_kv_amd as spkv

SRC = os.path.join(ROOT, "tests", "c_abi_client.c")


@pytest.fixture(scope="module")
def client(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    spkv.load_library()                       # raises if libspkv.so is missing
    out = str(tmp_path_factory.mktemp("cclient") / "c_abi_client")
    libdir = os.path.dirname(spkv.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), SRC, "-o", out,
                    "-L", libdir, "-l:libspkv.so", f"-Wl,-rpath,{libdir}"],
                   check=True, capture_output=True)
    return out


def test_c_client_runs_the_worked_example(client, golden_dir):
    g = json.load(open(os.path.join(golden_dir, "tiny_stream_conventions.json")))
    cfg = g["config"]
    args = [cfg[k] for k in ("num_blocks", "num_heads", "head_dim", "page_size",
                             "patch_tokens", "num_special_tokens", "scale_frames",
                             "sliding_window", "headroom", "max_total_frames")]
    res = subprocess.run([client] + [str(a) for a in args] + [str(len(g["frames"]))],
                         capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    lines = res.stdout.splitlines()
    kv = dict(l.split(" ", 1) for l in lines if not l.startswith("frame "))
    frames = [l for l in lines if l.startswith("frame ")]
    assert len(frames) == len(g["frames"])
    for line, row in zip(frames, g["frames"]):
        words = line.split()
        table = [int(x) for x in words[words.index("table") + 1:words.index("lpl")]]
        lpl = int(words[words.index("lpl") + 1])
        free = [int(x) for x in words[words.index("free") + 1:words.index("stats")]]
        stats = [int(x) for x in words[words.index("stats") + 1:]]
        assert table == row["table"], line
        assert lpl == row["last_page_len"], line
        assert free == row["free"], line
        assert stats == row["stats"], line
    codes = {v: k for k, v in spkv.ERROR_NAMES.items()}
    mnp, pool, _, _ = spkv.query_sizes(**cfg)
    assert kv["query_sizes"] == f"0 {mnp} {pool}"
    assert kv["query_workspace"] == "0 1 1"
    assert int(kv["query_workspace_bad"]) == codes["INVALID_ARG"]
    assert int(kv["create"]) == 0
    assert int(kv["run_before_plan"]) == codes["NOT_PLANNED"]
    assert int(kv["plan_empty"]) == codes["EMPTY"]
    assert int(kv["run"]) == codes["UNSUPPORTED"]          # host-only, checks passed
    assert int(kv["bad_block"]) == codes["BAD_BLOCK"]
    assert int(kv["run_batch"]) == codes["UNSUPPORTED"]
    assert int(kv["run_batch_same_handle"]) == codes["INVALID_ARG"]
    assert int(kv["run_batch_empty"]) == codes["INVALID_ARG"]
    assert int(kv["rollback_after_evictions"]) == codes["NOTHING_TO_ROLLBACK"]
    assert int(kv["reset"]) == 0
    assert int(kv["run_after_reset"]) == codes["NOT_PLANNED"]
    assert kv["destroy"] == "0 0"
    assert kv["error_string"] == "block state differs from the plan"


def _plan_line(line):
    """'p 0 table .. lpl N pspec .. bspec .. free ..' -> dict of int lists."""
    words = line.split()
    keys = ["table", "lpl", "pspec", "bspec", "free"]
    pos = [words.index(k) for k in keys] + [len(words)]
    out = {k: [int(x) for x in words[pos[i] + 1:pos[i + 1]]] for i, k in enumerate(keys)}
    out["code"] = int(words[1])
    return out


def _runs(flat):
    return [flat[i:i + 3] for i in range(0, len(flat), 3)]


def test_c_client_replays_the_eviction_flags_example(client, golden_dir):
    """The hand-derived eviction-flag example (tests/golden), driven from C:
    frames admitted alternately by append_frame_in_run and append_frame,
    evicted with each scenario's flags, planned; the plan's table,
    last_page_len and visible special runs, and the block's own runs, as the
    example gives them; then the deferred step (set_defer_eviction,
    execute_deferred_eviction with the flags of the last evict_frames) and
    the codes of run, run_own and run_noalloc on a host-only handle, of
    set_num_splits and of a rollback after pages moved."""
    g = json.load(open(os.path.join(golden_dir, "eviction_flags_tiny.json")))
    cfg = g["config"]
    args = [cfg[k] for k in ("num_blocks", "num_heads", "head_dim", "page_size",
                             "patch_tokens", "num_special_tokens", "scale_frames",
                             "sliding_window", "headroom", "max_total_frames")]
    codes = {v: k for k, v in spkv.ERROR_NAMES.items()}
    for sc in g["scenarios"]:
        flags, n = sc["flags"]
        sched = [tuple(flags)] * n + [tuple(x) for x in sc.get("then", [])]
        cmds = []
        for t, (cf, cam) in enumerate(sched):
            cmds += ["a" if t % 2 == 0 else "A", f"e {cf} {cam}", "p"]
        cmds += ["c", "r"]
        d = sc.get("deferred")
        if d:
            cmds += ["d 1", "a", "e 0 0", "x", "d 0", "p"]
        res = subprocess.run([client, "script"] + [str(a) for a in args],
                             input="\n".join(cmds) + "\n", capture_output=True, text=True,
                             timeout=60)
        assert res.returncode == 0, res.stdout + res.stderr
        lines = res.stdout.splitlines()
        assert lines[0] == "create 0" and lines[-1] == "destroy 0", sc["name"]
        plans = [_plan_line(l) for l in lines if l.startswith("p ")]
        other = [l for l in lines[1:-1] if not l.startswith("p ")]
        assert all(p["code"] == 0 for p in plans), sc["name"]
        checks = {row["t"]: row for row in sc["checks"]}
        for t, row in checks.items():
            p = plans[t]
            assert p["table"] == row["table"], (sc["name"], t)
            assert p["lpl"] == [row["last_page_len"]], (sc["name"], t)
            assert _runs(p["pspec"]) == row["specials"], (sc["name"], t)
            assert _runs(p["bspec"]) == row["specials"], (sc["name"], t)
        c_line = next(l for l in other if l.startswith("c "))
        assert [int(x) for x in c_line.split()[1:]] == [
            codes["UNSUPPORTED"], codes["UNSUPPORTED"], codes["UNSUPPORTED"], 0,
            codes["INVALID_ARG"]], sc["name"]
        r_line = next(l for l in other if l.startswith("r "))
        # the last append took a free page; the free list kept its length iff
        # that frame's eviction returned one, after which rollback is refused
        last, prev = plans[len(sched) - 1]["free"], plans[len(sched) - 2]["free"]
        moved = len(last) == len(prev)
        assert moved, sc["name"]          # every scenario ends in the full window
        assert int(r_line.split()[1]) == codes["NOTHING_TO_ROLLBACK"], sc["name"]
        if d:
            p = plans[-1]
            assert p["table"] == d["table"] and p["lpl"] == [d["last_page_len"]], sc["name"]
            assert _runs(p["pspec"]) == d["specials"], sc["name"]
            assert p["free"] == d["free"], sc["name"]
        assert all(int(l.split()[-1]) == 0 for l in other
                   if l.split()[0] in ("a", "A", "e", "d", "x")), sc["name"]
