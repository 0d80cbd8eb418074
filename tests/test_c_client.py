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
