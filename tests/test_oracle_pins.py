"""Pins of the oracle's page-pool state machine (Part 1) to what the pages
print, to closed forms that follow from their rules, to invariants, and to a
hand-derived worked example.  CPU only."""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle.pagepool as pp
from oracle import OracleConfig, OracleError, PagePoolOracle
from oracle.pagepool import visible_tokens_closed_form, window_mode_frames


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def cfg_224():
    return OracleConfig(num_blocks=2, num_heads=1, head_dim=1, page_size=256,
                        patch_tokens=256, num_special_tokens=6, scale_frames=8,
                        sliding_window=64, headroom=16, max_total_frames=2048)


# --------------------------------------------------------------- page numbers
def test_patch_pool_is_88_pages(golden_dir):
    g = load(golden_dir, "pages_constants.json")["patch_pool_pages"]
    c = OracleConfig(1, 1, 1, 256, 256, 6, g["scale"], g["window"], g["headroom"], 2048)
    assert c.num_patch_pages == g["total"] == 88


def test_42_frames_per_special_page_at_256(golden_dir):
    g = load(golden_dir, "pages_constants.json")
    sp = g["special_page_packing"]
    c = OracleConfig(1, 1, 1, sp["page_size"], 256,
                     g["special_tokens_per_frame"]["value"], 8, 64, 16,
                     sp["max_total_frames_default"])
    assert c.frames_per_special_page == sp["frames_per_page"] == 42
    # 2048 frames need ceil(2048 / 42) = 49 special pages.
    assert c.num_special_pages == 49
    assert c.max_num_pages == 88 + 49


def test_window_mode_1568_frames_by_slot_count(golden_dir):
    """8 + 120 x 13 = 1568: with the first 8 frames stored as scale frames and
    then one frame in 13 stored as a keyframe, the window's 128 slots are all
    taken (8 scale + 120 live pages) and the first frame that would need a
    129th slot is frame 1568, where the next window starts."""
    g = load(golden_dir, "pages_constants.json")["window_mode"]
    s, kf, iv = g["scale_slots"], g["keyframe_slots"], g["keyframe_interval"]
    assert window_mode_frames(g["window_size"], s, iv) == g["frames_per_window"]
    c = OracleConfig(1, 1, 1, 999, 999, 6, s, kf, 16, 2048)
    o = PagePoolOracle(c)
    i, first_overflow = 0, None
    while first_overflow is None:
        stored = i < s or (i - s) % iv == 0
        if stored:
            fc, sc, lv, fr, sp = o.get_cache_stats(0)
            if sc + lv == g["window_size"]:
                first_overflow = i
                break
            o.append_frame(0)
            o.evict_frames(0, c.scale_frames, c.sliding_window)
        i += 1
    assert first_overflow == g["frames_per_window"] == 1568
    fc, sc, lv, fr, sp = o.get_cache_stats(0)
    assert (sc, lv, fc) == (s, kf, g["window_size"])


def test_healthy_stats_224_stream(golden_dir):
    """Healthy values: scale_pg = 8, live_pg <= 64, free varies, special +6 per
    frame; at steady state the 16 headroom pages idle in the free list."""
    g = load(golden_dir, "pages_constants.json")
    hs = g["healthy_stats"]
    c = cfg_224()
    o = PagePoolOracle(c)
    for f in range(200):
        o.append_frame(0)
        o.evict_frames(0, 8, 64)
        fc, sc, lv, fr, sp = o.get_cache_stats(0)
        assert fc == f + 1
        assert sp == hs["special_tokens_per_frame"] * (f + 1)
        assert sc == min(f + 1, hs["scale_pages"])
        assert lv <= hs["live_pages_max"]
        if f + 1 >= 8 + 64:
            assert (sc, lv, fr) == (8, 64, g["headroom_idles_in_free_list"]["free_pages_steady"])


def test_special_tokens_land_in_order_after_patch_pages(golden_dir):
    """The frame's first 6 tokens [camera, register x4, scale] go to the
    special stream in order, its patch tokens to a patch page, K at index 0 and
    V at index 1; special frames pack back to back, floor(ps/6) per page."""
    g = load(golden_dir, "pages_constants.json")
    ns = g["special_tokens_per_frame"]["value"]
    kv = g["kv_index"]
    c = OracleConfig(1, 2, 3, 16, 10, ns, 2, 4, 2, 32)
    o = PagePoolOracle(c, track_pool=[0])
    rng = np.random.default_rng(0)
    frames = []
    for f in range(5):
        k = rng.integers(1, 60000, size=(16, 2, 3)).astype(np.uint16)
        v = rng.integers(1, 60000, size=(16, 2, 3)).astype(np.uint16)
        frames.append((k, v))
        p, sp, slot = o.append_frame(0, k, v)
        pool = o.pools[0]
        fpp = 16 // ns
        assert sp == c.num_patch_pages + f // fpp
        assert slot == ns * (f % fpp)
        for name_i, row in enumerate(range(ns)):
            assert np.array_equal(pool[sp, kv["key"], slot + row], k[row])
            assert np.array_equal(pool[sp, kv["value"], slot + row], v[row])
        assert np.array_equal(pool[p, kv["key"], 0:10], k[ns:])
        assert np.array_equal(pool[p, kv["value"], 0:10], v[ns:])
        # padded tail of the patch page untouched (still zero)
        assert not pool[p, :, 10:].any()


# ------------------------------------------------------------- worked example
def test_tiny_stream_worked_example(golden_dir):
    g = load(golden_dir, "tiny_stream_conventions.json")
    c = OracleConfig(**g["config"])
    o = PagePoolOracle(c)
    for row in g["frames"]:
        o.append_frame(0)
        o.evict_frames(0, c.scale_frames, c.sliding_window)
        pl = o.plan()
        assert pl.table == row["table"], row["t"]
        assert pl.last_page_len == row["last_page_len"]
        assert pl.num_visible_tokens(c) == row["nk"]
        assert o.block_state(0)[2] == row["free"]
        assert list(o.get_cache_stats(0)) == row["stats"]
    rp = g["rollback_probe"]
    o.set_defer_eviction(True)
    o.append_frame(0)
    o.evict_frames(0, c.scale_frames, c.sliding_window)
    pl = o.plan()
    assert pl.table == rp["pending_table"]
    assert pl.last_page_len == rp["pending_last_page_len"]
    assert o.block_state(0)[2] == rp["pending_free"]
    o.rollback_last_frame(0)
    scale, live, free, nsf = o.block_state(0)
    assert free == rp["after_free"] and live == rp["after_live"] and nsf == rp["after_nsf"]


def _flag_schedule(sc):
    """Per-frame eviction flags of a scenario: the first entry's flags for
    its count of frames, then one frame each for the entries of `then`."""
    flags, n = sc["flags"]
    return [tuple(flags)] * n + [tuple(f) for f in sc.get("then", [])]


def test_eviction_flags_worked_example(golden_dir):
    """Hand-derived tables, special runs and visible counts under each pair of
    eviction flags, a change of flags mid-stream and a deferred eviction that
    takes the flags of the deferred call (reading R13)."""
    g = load(golden_dir, "eviction_flags_tiny.json")
    c = OracleConfig(**g["config"])
    for sc in g["scenarios"]:
        o = PagePoolOracle(c)
        checks = {row["t"]: row for row in sc["checks"]}
        for t, flags in enumerate(_flag_schedule(sc)):
            o.append_frame(0)
            o.evict_frames(0, c.scale_frames, c.sliding_window, *flags)
            pl = o.plan()
            assert o.special_visibility(0) == pp.special_runs(pl.spec_vis)
            if t in checks:
                row = checks[t]
                assert pl.table == row["table"], (sc["name"], t)
                assert pl.last_page_len == row["last_page_len"]
                assert o.special_visibility(0) == row["specials"], (sc["name"], t)
                assert pl.num_visible_tokens(c) == row["nk"], (sc["name"], t)
        d = sc.get("deferred")
        if d:
            o.set_defer_eviction(True)
            o.append_frame(0)
            assert o.evict_frames(0, c.scale_frames, c.sliding_window, 0, 0) == 0
            assert o.execute_deferred_eviction(0, c.scale_frames, c.sliding_window) == 1
            o.set_defer_eviction(False)
            pl = o.plan()
            assert pl.table == d["table"]
            assert pl.last_page_len == d["last_page_len"]
            assert o.special_visibility(0) == d["specials"]
            assert pl.num_visible_tokens(c) == d["nk"]
            assert o.block_state(0)[2] == d["free"]
            o.reset()                      # a reset restores the default flags
            assert o.blocks[0].flags == (1, 0)


@settings(max_examples=100, deadline=None)
@given(cfg=st.builds(
    lambda ns, s, w, r: OracleConfig(1, 1, 1, 2 * ns + 1, 2 * ns, ns, s, w, r, 60),
    ns=st.integers(1, 6), s=st.integers(0, 3), w=st.integers(1, 5), r=st.integers(1, 2)),
    n=st.integers(1, 40), cross=st.integers(0, 1), camera=st.integers(0, 1))
def test_closed_form_visible_tokens_under_eviction_flags(cfg, n, cross, camera):
    """Nk = (P + 6) x held frames + kept x evicted frames, kept = 6, 1 or 0
    for the flags; the special runs say the same frame by frame."""
    o = PagePoolOracle(cfg)
    kept = pp.special_tokens_kept(cfg, cross, camera)
    assert kept == (0 if not cross else 1 if camera else cfg.num_special_tokens)
    for k in range(1, n + 1):
        o.append_frame(0)
        o.evict_frames(0, cfg.scale_frames, cfg.sliding_window, cross, camera)
        pl = o.plan()
        assert pl.num_visible_tokens(cfg) == pp.visible_tokens_closed_form(cfg, k, kept=kept)
        held = min(k, cfg.scale_frames) + min(max(k - cfg.scale_frames, 0), cfg.sliding_window)
        evicted = k - held
        assert sum(r[1] * r[2] for r in o.special_visibility(0)) == \
            cfg.num_special_tokens * held + kept * evicted
        # stats keep counting the stored specials: the stream's bytes stay
        assert o.get_cache_stats(0)[4] == cfg.num_special_tokens * k


# ------------------------------------------------------------- closed forms
small_cfgs = st.builds(
    lambda ns, ps_extra, pt_cut, s, w, r, mtf: OracleConfig(
        2, 1, 1, ns + ps_extra, max(1, ns + ps_extra - pt_cut), ns, s, w, r, mtf),
    ns=st.integers(1, 6), ps_extra=st.integers(0, 12), pt_cut=st.integers(0, 3),
    s=st.integers(0, 3), w=st.integers(1, 5), r=st.integers(1, 3),
    mtf=st.integers(8, 60))


@settings(max_examples=150, deadline=None)
@given(cfg=small_cfgs, n=st.integers(1, 40))
def test_closed_forms_keyframe_stream(cfg, n):
    o = PagePoolOracle(cfg)
    fpp = cfg.frames_per_special_page
    n = min(n, cfg.special_capacity_frames)
    for k in range(1, n + 1):
        o.append_frame(0)
        o.evict_frames(0, cfg.scale_frames, cfg.sliding_window)
        pl = o.plan()
        n_sp = -(-k // fpp)
        assert pl.table[pl.n_patch:] == [cfg.num_patch_pages + i for i in range(n_sp)]
        assert pl.last_page_len == cfg.num_special_tokens * (k - fpp * (n_sp - 1))
        assert cfg.num_special_tokens <= pl.last_page_len <= cfg.num_special_tokens * fpp
        assert pl.num_visible_tokens(cfg) == visible_tokens_closed_form(cfg, k)
        assert pl.n_patch == min(k, cfg.scale_frames) + min(max(k - cfg.scale_frames, 0), cfg.sliding_window)


# -------------------------------------------------------------- invariants
OPS = st.lists(st.sampled_from(
    ["append", "evict", "defer_on", "defer_off", "execute", "rollback", "plan", "reset"]),
    min_size=1, max_size=60)


def _check_invariants(o):
    c = o.cfg
    for b in range(c.num_blocks):
        scale, live, free, nsf = o.block_state(b)
        allp = scale + live + free
        assert sorted(allp) == list(range(c.num_patch_pages))
        assert len(scale) <= c.scale_frames
        fc, sc, lv, fr, sp = o.get_cache_stats(b)
        assert sp == c.num_special_tokens * fc
        assert sc + lv + fr == c.num_patch_pages
        if not o.defer:
            # without deferral the window never exceeds W after evict; with a
            # pending frame it may hold more
            pass
    # all blocks follow the same op sequence here, so they are identical
    s0 = o.block_state(0)
    for b in range(1, c.num_blocks):
        assert o.block_state(b) == s0


def _apply(o, op):
    c = o.cfg
    try:
        if op == "append":
            for b in range(c.num_blocks):
                o.append_frame(b)
        elif op == "evict":
            for b in range(c.num_blocks):
                o.evict_frames(b, c.scale_frames, c.sliding_window)
        elif op == "defer_on":
            o.set_defer_eviction(True)
        elif op == "defer_off":
            o.set_defer_eviction(False)
        elif op == "execute":
            for b in range(c.num_blocks):
                o.execute_deferred_eviction(b, c.scale_frames, c.sliding_window)
        elif op == "rollback":
            for b in range(c.num_blocks):
                o.rollback_last_frame(b)
        elif op == "plan":
            pl = o.plan()
            assert len(set(pl.table)) == len(pl.table)
            for b in range(c.num_blocks):
                o.check_run(b)
        elif op == "reset":
            o.reset()
        return None
    except OracleError as e:
        return e.name


@settings(max_examples=300, deadline=None)
@given(cfg=small_cfgs, ops=OPS)
def test_invariants_under_random_ops(cfg, ops):
    o = PagePoolOracle(cfg)
    for op in ops:
        before = [o.block_state(b) for b in range(cfg.num_blocks)]
        err = _apply(o, op)
        if err is not None:
            # strong guarantee: an error leaves every block unchanged (blocks
            # fail on the first one, before any change, since all are equal)
            assert [o.block_state(b) for b in range(cfg.num_blocks)] == before
        _check_invariants(o)


@settings(max_examples=200, deadline=None)
@given(cfg=small_cfgs, ops=OPS, defer=st.booleans())
def test_append_then_rollback_is_identity(cfg, ops, defer):
    o = PagePoolOracle(cfg)
    for op in ops:
        _apply(o, op)
    o.set_defer_eviction(defer)
    before = o.block_state(0)
    try:
        o.append_frame(0)
    except OracleError:
        return
    if defer:
        o.evict_frames(0, cfg.scale_frames, cfg.sliding_window)  # no-op
    o.rollback_last_frame(0)
    assert o.block_state(0) == before
    with pytest.raises(OracleError) as ei:
        o.rollback_last_frame(0)
    assert ei.value.name == "NOTHING_TO_ROLLBACK"


@settings(max_examples=150, deadline=None)
@given(cfg=small_cfgs, n=st.integers(0, 30))
def test_execute_after_deferred_equals_immediate_evict(cfg, n):
    a, b = PagePoolOracle(cfg), PagePoolOracle(cfg)
    b.set_defer_eviction(True)
    for _ in range(min(n, cfg.special_capacity_frames)):
        for o in (a, b):
            try:
                o.append_frame(0)
            except OracleError:
                return
        a.evict_frames(0, cfg.scale_frames, cfg.sliding_window)
        b.evict_frames(0, cfg.scale_frames, cfg.sliding_window)   # deferred: no-op
        b.execute_deferred_eviction(0, cfg.scale_frames, cfg.sliding_window)
        assert a.block_state(0) == b.block_state(0)


# ------------------------------------------------------------- error cases
def test_errors_and_strong_guarantee():
    c = OracleConfig(2, 1, 1, 6, 6, 6, 1, 1, 0, 2)   # M = 2, fpp = 1, NS = 2
    o = PagePoolOracle(c)
    with pytest.raises(OracleError, match="EMPTY"):
        o.plan()
    with pytest.raises(OracleError, match="NOT_PLANNED"):
        o.check_run(0)
    with pytest.raises(OracleError, match="BAD_BLOCK"):
        o.append_frame(2)
    with pytest.raises(OracleError, match="NOTHING_TO_ROLLBACK"):
        o.rollback_last_frame(0)
    with pytest.raises(OracleError, match="INVALID_ARG"):
        o.evict_frames(0, 1, 1, cross_frame_special=2)
    with pytest.raises(OracleError, match="INVALID_ARG"):
        o.evict_frames(0, 1, 1, camera_only=-1)
    with pytest.raises(OracleError, match="INVALID_ARG"):
        o.evict_frames(0, 1, 2, cross_frame_special=0)   # flags recorded only if valid
    assert o.blocks[0].flags == (1, 0)
    with pytest.raises(OracleError, match="INVALID_ARG"):
        o.evict_frames(0, 2, 1)
    with pytest.raises(OracleError, match="INVALID_ARG"):
        o.evict_frames(0, 1, 2)      # W' > M - S
    o.set_defer_eviction(True)
    o.append_frame(0)
    o.append_frame(0)                # scale [0], live [1]
    st0 = o.block_state(0)
    with pytest.raises(OracleError, match="POOL_EXHAUSTED"):
        o.append_frame(0)
    assert o.block_state(0) == st0
    o.plan()
    with pytest.raises(OracleError, match="STALE_PLAN"):
        o.check_run(1)               # block 1 never appended
    o.check_run(0)
    # special overflow before pool exhaustion
    c2 = OracleConfig(1, 1, 1, 6, 6, 6, 0, 4, 4, 2)  # NS*fpp = 2, M = 8
    o2 = PagePoolOracle(c2)
    o2.append_frame(0)
    o2.append_frame(0)
    with pytest.raises(OracleError, match="SPECIAL_OVERFLOW"):
        o2.append_frame(0)
    o.reset()
    with pytest.raises(OracleError, match="NOT_PLANNED"):
        o.check_run(0)
    assert o.defer is False
