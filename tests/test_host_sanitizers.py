"""The host page-pool allocator (streaming_paged_kv_amd/csrc/pool.cpp) under
AddressSanitizer and UndefinedBehaviorSanitizer.

tests/host_sanitize_driver.cpp drives seeded random sequences of every pool
operation (append, undo, evict with valid and invalid arguments and every
pair of special-token flags, deferred eviction, rollback, reset, plan,
check_run, stats, block_state) over six geometries, and checks the pool's
invariants after each step: the scale list, live window and free list
partition the patch pages, a failed call changes nothing, the plan equals
scale then live then the special pages that still show a token, with the
last-page length the special stream implies, and the visible special tokens
follow the driver's own per-frame model of what eviction kept.  The two-stream layout these
invariants restate is the one of the pages' sections on patch and special
pages and on the physical page layout.

It is built with g++ only (pool.cpp has no HIP dependency), so it runs on any
host.  A sanitizer report, a broken invariant or a digest that differs from
an unsanitized -O2 build fails the test."""

import os
import re
import shutil
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "streaming_paged_kv_amd", "csrc")
SOURCES = [os.path.join(CSRC, "pool.cpp"),
           os.path.join(ROOT, "tests", "host_sanitize_driver.cpp")]
OUTCOMES = ("append_ok", "pool_exhausted", "special_overflow", "undo_append",
            "evict_moved", "evict_deferred", "bad_block", "specials_thinned", "invalid_arg",
            "rollback_ok", "nothing_to_rollback", "plan_ok", "plan_empty", "run_ok",
            "stale_plan", "not_planned", "block_state_small_cap")


def _build(tmp_path, name, flags):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path / name)
    res = subprocess.run([gxx, "-std=c++17", "-Wall", "-Wextra", "-Wno-sign-compare",
                          "-Werror", *flags, "-I", CSRC, *SOURCES, "-o", out],
                         capture_output=True, text=True)
    if res.returncode != 0 and "sanitize" in res.stderr and "cannot find" in res.stderr:
        pytest.skip("sanitizer runtime not installed: " + res.stderr.strip()[-200:])
    assert res.returncode == 0, res.stderr
    return out


def _run(exe):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([exe, "40", "400"], capture_output=True, text=True,
                         timeout=300, env=env)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "runtime error" not in res.stderr, res.stderr[-4000:]
    m = re.search(r"^ok .* digest ([0-9a-f]{16})$", res.stdout, re.M)
    assert m, res.stdout[-2000:]
    counts = dict(l.split(" ", 1) for l in res.stdout.splitlines() if not l.startswith("ok "))
    return m.group(1), {k: int(v) for k, v in counts.items()}


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    tmp = tmp_path_factory.mktemp("sanitize")
    san = _build(tmp, "drv_san", ["-O1", "-g", "-fno-omit-frame-pointer",
                                  "-fsanitize=address,undefined",
                                  "-fno-sanitize-recover=all"])
    plain = _build(tmp, "drv_o2", ["-O2"])
    return san, plain


def test_allocator_clean_under_asan_ubsan(builds):
    digest, counts = _run(builds[0])
    # Every outcome, error paths included, was reached at least once.
    for k in OUTCOMES:
        assert counts.get(k, 0) > 0, (k, counts)


def test_sanitized_and_optimised_builds_agree(builds):
    d_san, c_san = _run(builds[0])
    d_o2, c_o2 = _run(builds[1])
    assert d_san == d_o2
    assert c_san == c_o2
