"""The C-ABI library loads without a GPU and exports every symbol that
include/spkv.h declares; sizes it reports match the configuration arithmetic
the pages fix.  No compute calls here."""

import ctypes
import os
import re

import pytest

from conftest import ROOT
import streaming_paged_kv_amd as spkv

HEADER = os.path.join(ROOT, "include", "spkv.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SPKV_API\s+[\w\s\*]+?\b(spkv_\w+)\s*\(", text)))


def test_header_declares_the_binding_set():
    assert declared_symbols() == sorted(spkv.EXPORTED)


def test_library_loads_and_exports_all_symbols():
    lib = ctypes.CDLL(spkv.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_error_strings():
    lib = spkv.load_library()
    for code in spkv.ERROR_NAMES:
        assert lib.spkv_error_string(code)
    assert lib.spkv_error_string(12345) == b"unknown status"


def test_query_sizes_224_config():
    mnp, pool, wmin, wfull = spkv.query_sizes(
        num_blocks=24, num_heads=16, head_dim=64, page_size=256, patch_tokens=256,
        num_special_tokens=6, scale_frames=8, sliding_window=64, headroom=16,
        max_total_frames=2048)
    assert mnp == 88 + 49
    assert pool == 137 * 2 * 256 * 16 * 64 * 2
    assert 0 < wmin < wfull


def test_query_sizes_518_exact_and_padded():
    kw = dict(num_blocks=24, num_heads=16, head_dim=64, patch_tokens=999,
              num_special_tokens=6, scale_frames=8, sliding_window=64, headroom=16,
              max_total_frames=2048)
    mnp, pool, _, _ = spkv.query_sizes(page_size=999, **kw)
    assert mnp == 88 + 13          # 166 frames per special page
    mnp2, pool2, wmin, wfull = spkv.query_sizes(page_size=1024, **kw)
    assert mnp2 == 88 + 13         # 170 frames per special page
    assert pool2 > pool
    # the pages' 128 MiB workspace holds at least 16 key splits here
    per_split = (wfull - wmin) // 32
    assert (128 * 2 ** 20 - wmin) // per_split >= 16
    # one split of one frame: bf16 normalised O and fp32 (m, l) for 1005
    # rows x 16 heads
    w1 = spkv.query_workspace(1005, 1, page_size=999, **kw)
    assert w1 - spkv.query_sizes(page_size=999, **kw)[2] == 1005 * 16 * 64 * 2 + 1005 * 16 * 8 + 128   # 256-byte rounding
    for nq, sp in ((0, 1), (1, 0), (1, 33), ((1 << 20) + 1, 1)):
        with pytest.raises(spkv.SpkvError):
            spkv.query_workspace(nq, sp, page_size=999, **kw)


@pytest.mark.parametrize("bad", [
    dict(head_dim=128), dict(page_size=5), dict(patch_tokens=0),
    dict(patch_tokens=17), dict(sliding_window=0), dict(num_blocks=0),
    dict(max_total_frames=0), dict(scale_frames=-1)])
def test_query_sizes_rejects(bad):
    kw = dict(num_blocks=1, num_heads=4, head_dim=64, page_size=16, patch_tokens=16,
              num_special_tokens=6, scale_frames=2, sliding_window=4, headroom=2,
              max_total_frames=32)
    kw.update(bad)
    with pytest.raises(spkv.SpkvError) as ei:
        spkv.query_sizes(**kw)
    assert ei.value.name in ("INVALID_ARG", "UNSUPPORTED")


def test_create_rejects_half_device_arguments():
    lib = spkv.load_library()
    c = spkv.make_config(num_blocks=1, num_heads=4, head_dim=64, page_size=16,
                         patch_tokens=16, num_special_tokens=6, scale_frames=2,
                         sliding_window=4, headroom=2, max_total_frames=32)
    h = ctypes.c_void_p()
    ptrs = (ctypes.c_void_p * 1)(ctypes.c_void_p(256))
    # pools without a workspace (or the reverse) is invalid; checked before any
    # device call
    assert lib.spkv_create(ctypes.byref(c), ptrs, None, 0, ctypes.byref(h)) == -1
    assert lib.spkv_create(ctypes.byref(c), None, ctypes.c_void_p(256), 4096,
                           ctypes.byref(h)) == -1
    assert lib.spkv_create(ctypes.byref(c), None, None, 0, None) == -1
    assert lib.spkv_destroy(None) == 0
