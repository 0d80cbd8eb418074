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
an unsanitized -O2 build fails the test.

The C ABI layer above it (api.cpp) is checked the same way through the plain
C client on host-only handles: seeded random command scripts reach every
call of the ABI that a host-only handle serves, error paths included, under
both sanitizers, and the -O2 build must print the same transcript."""

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


# ---------------------------------------------------------------------------
# The C ABI layer (streaming_paged_kv_amd/csrc/api.cpp) with the allocator,
# driven through plain C (tests/c_abi_client.c) on host-only handles.  It is
# built with g++/gcc against tests/hip_host_stub, a stand-in for the HIP
# runtime header whose functions abort: host-only handles make no HIP call.

ABI_SOURCES = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "pool.cpp"),
               os.path.join(ROOT, "tests", "hip_host_stub", "launch_stubs.cpp")]
STUB = os.path.join(ROOT, "tests", "hip_host_stub")
CLIENT = os.path.join(ROOT, "tests", "c_abi_client.c")
# (NB H D PS P NS S W R MTF): the tiny stream, odd page sizes, no scale
# frames with a one-page window, a special stream of four frames, the
# 518x378 pool, padded pages
ABI_GEOMETRIES = [(1, 4, 64, 16, 16, 6, 2, 4, 2, 32), (2, 2, 64, 13, 11, 4, 1, 3, 1, 40),
                  (1, 3, 64, 6, 5, 6, 0, 1, 1, 30), (1, 2, 64, 12, 10, 6, 1, 2, 1, 4),
                  (1, 16, 64, 999, 999, 6, 8, 64, 16, 2048),
                  (1, 16, 64, 1024, 999, 6, 8, 64, 16, 2048)]


def _build_abi(tmp_path, name, flags):
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    if gxx is None or gcc is None:
        pytest.skip("g++/gcc not available")
    objs = []
    for src in ABI_SOURCES + [CLIENT]:
        obj = str(tmp_path / (name + "_" + os.path.basename(src) + ".o"))
        if src.endswith(".c"):
            cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", *flags,
                   "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
        else:
            cmd = [gxx, "-std=c++17", "-Wall", "-Wextra", "-Werror", *flags, "-I", STUB,
                   "-I", CSRC, "-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
        objs.append(obj)
    out = str(tmp_path / name)
    res = subprocess.run([gxx, *flags, *objs, "-o", out], capture_output=True, text=True)
    if res.returncode != 0 and "sanitize" in res.stderr and "cannot find" in res.stderr:
        pytest.skip("sanitizer runtime not installed: " + res.stderr.strip()[-200:])
    assert res.returncode == 0, res.stderr
    return out


@pytest.fixture(scope="module")
def abi_builds(tmp_path_factory):
    tmp = tmp_path_factory.mktemp("sanitize_abi")
    san = _build_abi(tmp, "abi_san", ["-O1", "-g", "-fno-omit-frame-pointer",
                                      "-fsanitize=address,undefined",
                                      "-fno-sanitize-recover=all"])
    plain = _build_abi(tmp, "abi_o2", ["-O2"])
    return san, plain


def _script(rng, n):
    """A seeded random command script for the client's script mode, with
    invalid flag and defer values now and then."""
    out = []
    for _ in range(n):
        r = rng.random()
        if r < 0.22:
            out.append("a")
        elif r < 0.34:
            out.append("A")
        elif r < 0.56:
            if rng.random() < 0.05:
                out.append(f"e {int(rng.integers(-1, 3))} {int(rng.integers(-1, 3))}")
            else:
                out.append(f"e {int(rng.integers(0, 2))} {int(rng.integers(0, 2))}")
        elif r < 0.62:
            out.append(f"d {int(rng.integers(0, 2)) if rng.random() > 0.1 else 2}")
        elif r < 0.68:
            out.append("x")
        elif r < 0.76:
            out.append("r")
        elif r < 0.90:
            out.append("p")
        elif r < 0.94:
            out.append("c")
        elif r < 0.97:
            out.append("s")
        else:
            out.append("R")
    return out


def _run_client(exe, args, stdin=None):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([exe, *map(str, args)], input=stdin, capture_output=True,
                         text=True, timeout=120, env=env)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "runtime error" not in res.stderr, res.stderr[-4000:]
    return res.stdout


def test_abi_layer_clean_under_asan_ubsan(abi_builds):
    """Seeded random scripts over six geometries (every call of the script
    mode, error paths included), and the client's fixed sequence, on the
    sanitized build; the -O2 build prints the same transcript."""
    import numpy as np
    san, plain = abi_builds
    seen = set()
    for gi, geo in enumerate(ABI_GEOMETRIES):
        for seed in range(6):
            rng = np.random.default_rng(1000 * gi + seed)
            text = "\n".join(_script(rng, 400)) + "\n"
            out_san = _run_client(san, ["script", *geo], text)
            assert out_san == _run_client(plain, ["script", *geo], text), (geo, seed)
            for line in out_san.splitlines():
                w = line.split()
                if w[0] in "aAedxrpRs" and len(w) > 1:
                    seen.add((w[0], int(w[1])))
        frames = min(3 * (geo[6] + geo[7] + geo[8]), geo[9])   # within the special stream
        out_san = _run_client(san, [*geo, frames])
        assert out_san == _run_client(plain, [*geo, frames]), geo
    codes = {v: k for k, v in __import__("streaming_paged_kv_amd").ERROR_NAMES.items()}
    for want in [("a", 0), ("A", 0), ("a", codes["POOL_EXHAUSTED"]),
                 ("a", codes["SPECIAL_OVERFLOW"]), ("e", 0), ("e", codes["INVALID_ARG"]),
                 ("d", codes["INVALID_ARG"]), ("x", 0), ("r", 0),
                 ("r", codes["NOTHING_TO_ROLLBACK"]), ("p", 0), ("p", codes["EMPTY"]),
                 ("R", 0), ("s", 0)]:
        assert want in seen, want
