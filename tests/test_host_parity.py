"""The C++ page-pool allocator (through the C ABI, host-only handles, no GPU)
against the oracle's state machine: bit-exact block state, plans, stats and
error codes on fixed and random operation sequences."""

import pytest
from hypothesis import given, settings, strategies as st

import streaming_paged_kv_amd as spkv
from oracle import OracleConfig, OracleError, PagePoolOracle
from oracle.pagepool import special_runs
import synth


def make_pair(**cfg):
    o = PagePoolOracle(OracleConfig(**cfg))
    c = spkv.PagedKVCache(host_only=True, **cfg)
    return o, c


def code_of(fn, *a):
    try:
        fn(*a)
        return "OK"
    except OracleError as e:
        return e.name
    except spkv.SpkvError as e:
        return e.name


def assert_same(o, c):
    cfg = o.cfg
    for b in range(cfg.num_blocks):
        assert list(o.block_state(b)) == list(c.get_block_state(b)), b
        assert tuple(o.get_cache_stats(b)) == c.get_cache_stats(b), b
        assert o.special_visibility(b) == c.get_block_specials(b), b
    if o.plan_state is None:
        assert code_of(c.get_plan) == "NOT_PLANNED"
        assert code_of(c.get_plan_specials) == "NOT_PLANNED"
    else:
        pl = o.plan_state
        assert c.get_plan() == (pl.table, pl.n_patch, pl.last_page_len)
        assert c.get_plan_specials() == special_runs(pl.spec_vis)


def step(o, c, op, block, arg):
    cfg = o.cfg
    if op == "append":
        r = (code_of(o.append_frame, block), code_of(c.append_frame, block))
    elif op == "evict":
        w = arg if arg else cfg.sliding_window
        r = (code_of(o.evict_frames, block, cfg.scale_frames, w),
             code_of(c.evict_frames, block, cfg.scale_frames, w))
    elif op == "evict_badS":
        r = (code_of(o.evict_frames, block, cfg.scale_frames + 1, cfg.sliding_window),
             code_of(c.evict_frames, block, cfg.scale_frames + 1, cfg.sliding_window))
    elif op == "evict_flags":
        # arg picks the flags: every valid pair and two invalid ones
        cfs, cam = [(0, 0), (0, 1), (1, 1), (1, 0), (2, 0), (1, -1), (0, 0)][arg]
        w = 1 + (arg + block) % (cfg.num_patch_pages - cfg.scale_frames)
        r = (code_of(o.evict_frames, block, cfg.scale_frames, w, cfs, cam),
             code_of(c.evict_frames, block, cfg.scale_frames, w, cfs, cam))
    elif op == "defer":
        r = (code_of(o.set_defer_eviction, bool(arg)),
             code_of(c.set_defer_eviction, bool(arg)))
    elif op == "execute":
        w = arg if arg else cfg.sliding_window
        r = (code_of(o.execute_deferred_eviction, block, cfg.scale_frames, w),
             code_of(c.execute_deferred_eviction, block, cfg.scale_frames, w))
    elif op == "rollback":
        r = (code_of(o.rollback_last_frame, block), code_of(c.rollback_last_frame, block))
    elif op == "reset":
        r = (code_of(o.reset), code_of(c.reset))
    elif op == "plan":
        r = (code_of(o.plan), code_of(c.plan))
    elif op in ("run", "run_own"):
        ro = code_of(o.check_run, block)
        rc = code_of(c.run if op == "run" else c.run_own, block)
        # a host-only handle reports UNSUPPORTED once the checks pass
        r = (ro, "OK" if rc == "UNSUPPORTED" else rc)
    else:
        raise AssertionError(op)
    assert r[0] == r[1], (op, block, arg, r)


CFGS = [
    dict(num_blocks=2, num_heads=4, head_dim=64, page_size=16, patch_tokens=16,
         num_special_tokens=6, scale_frames=2, sliding_window=4, headroom=2,
         max_total_frames=32),
    dict(num_blocks=3, num_heads=1, head_dim=64, page_size=13, patch_tokens=11,
         num_special_tokens=4, scale_frames=1, sliding_window=2, headroom=1,
         max_total_frames=9),
    dict(num_blocks=1, num_heads=2, head_dim=64, page_size=6, patch_tokens=6,
         num_special_tokens=6, scale_frames=0, sliding_window=3, headroom=0,
         max_total_frames=5),
]

op_strategy = st.tuples(
    st.sampled_from(["append", "append", "append", "evict", "evict", "defer",
                     "execute", "rollback", "plan", "plan", "run", "run_own", "reset",
                     "evict_badS", "evict_flags", "evict_flags"]),
    st.integers(-1, 3), st.integers(0, 6))


@pytest.mark.parametrize("ci", range(len(CFGS)))
@settings(max_examples=120, deadline=None)
@given(ops=st.lists(op_strategy, min_size=1, max_size=80))
def test_random_ops_match_oracle(ci, ops):
    o, c = make_pair(**CFGS[ci])
    try:
        for op, block, arg in ops:
            step(o, c, op, block, arg)
            assert_same(o, c)
    finally:
        c.close()


def test_tiny_stream_worked_example_through_abi(golden_dir):
    import json, os
    g = json.load(open(os.path.join(golden_dir, "tiny_stream_conventions.json")))
    cfg = g["config"]
    c = spkv.PagedKVCache(host_only=True, **cfg)
    for row in g["frames"]:
        c.append_frame(0)
        c.evict_frames(0, cfg["scale_frames"], cfg["sliding_window"])
        c.plan()
        assert c.get_plan()[0] == row["table"]
        assert c.get_plan()[2] == row["last_page_len"]
        assert c.get_block_state(0)[2] == row["free"]
        assert list(c.get_cache_stats(0)) == row["stats"]
    c.close()


def test_append_in_run_admits_like_append():
    """On a host-only handle append_frame_in_run is append_frame: the same
    state, plans and errors over a stream with evictions, deferral, rollback
    and the special stream filling up."""
    cfg = CFGS[0]
    a = spkv.PagedKVCache(host_only=True, **cfg)
    b = spkv.PagedKVCache(host_only=True, **cfg)
    S, W = cfg["scale_frames"], cfg["sliding_window"]
    for f in range(40):
        defer = f % 5 == 3
        for c in (a, b):
            c.set_defer_eviction(defer)
        r = (code_of(a.append_frame, 0), code_of(b.append_frame_in_run, 0))
        assert r[0] == r[1], (f, r)
        a.evict_frames(0, S, W, 1, f % 3 == 0)
        b.evict_frames(0, S, W, 1, f % 3 == 0)
        if defer:
            assert code_of(a.rollback_last_frame, 0) == code_of(b.rollback_last_frame, 0)
        assert a.get_block_state(0) == b.get_block_state(0)
        assert a.get_block_specials(0) == b.get_block_specials(0)
        if a.get_cache_stats(0)[0]:
            a.plan(); b.plan()
            assert a.get_plan() == b.get_plan()
    assert code_of(b.append_frame_in_run, 5) == "BAD_BLOCK"
    a.close(); b.close()


def test_eviction_flags_worked_example_through_abi(golden_dir):
    """The hand-derived eviction-flag example, replayed on the C++ allocator."""
    import json, os
    g = json.load(open(os.path.join(golden_dir, "eviction_flags_tiny.json")))
    cfg = g["config"]
    S, W = cfg["scale_frames"], cfg["sliding_window"]
    for sc in g["scenarios"]:
        c = spkv.PagedKVCache(host_only=True, **cfg)
        checks = {row["t"]: row for row in sc["checks"]}
        flags, n = sc["flags"]
        sched = [tuple(flags)] * n + [tuple(x) for x in sc.get("then", [])]
        for t, fl in enumerate(sched):
            c.append_frame(0)
            c.evict_frames(0, S, W, *fl)
            c.plan()
            if t in checks:
                row = checks[t]
                assert c.get_plan()[0] == row["table"], (sc["name"], t)
                assert c.get_plan()[2] == row["last_page_len"]
                assert c.get_plan_specials() == row["specials"], (sc["name"], t)
                assert c.get_block_specials(0) == row["specials"]
        d = sc.get("deferred")
        if d:
            c.set_defer_eviction(True)
            c.append_frame(0)
            c.evict_frames(0, S, W, 0, 0)
            c.execute_deferred_eviction(0, S, W)
            c.set_defer_eviction(False)
            c.plan()
            assert c.get_plan()[0] == d["table"]
            assert c.get_plan()[2] == d["last_page_len"]
            assert c.get_plan_specials() == d["specials"]
            assert c.get_block_state(0)[2] == d["free"]
        c.close()


@pytest.mark.parametrize("name,flags", [
    ("224x224", (1, 0)), ("518x378", (1, 0)), ("518x378-padded", (1, 0)), ("dynamic", (1, 0)),
    ("518x378", (1, 1)), ("dynamic", (0, 0)), ("224x224", (0, 1))])
def test_full_stream_schedules_match_oracle(name, flags):
    """The whole frame schedule of each workload (all blocks, every frame),
    bit-exact on every block's state and on every plan, with the pages'
    default eviction flags and with the variants that thin or drop the
    specials of evicted frames."""
    wl = synth.WORKLOADS[name]
    cfg = wl.cfg_kwargs()
    o, c = make_pair(**cfg)
    S, W = wl.scale_frames, wl.sliding_window
    decisions = synth.accept_decisions(wl) if wl.dynamic else None
    nb = wl.num_blocks
    frames = wl.frames
    if wl.dynamic:
        o.set_defer_eviction(True)
        c.set_defer_eviction(True)
    for f in range(frames):
        if wl.reset_every and f > 0 and f % wl.reset_every == 0:
            o.reset(); c.reset()
            if wl.dynamic:
                o.set_defer_eviction(True); c.set_defer_eviction(True)
        key = synth.is_keyframe(wl, f)
        transient = not wl.dynamic and not key
        if transient:
            o.set_defer_eviction(True); c.set_defer_eviction(True)
        for b in range(nb):
            o.append_frame(b); c.append_frame(b)
            o.evict_frames(b, S, W, *flags); c.evict_frames(b, S, W, *flags)
            if b == 0:
                o.plan(); c.plan()
                pl = o.plan_state
                assert c.get_plan() == (pl.table, pl.n_patch, pl.last_page_len), f
                assert c.get_plan_specials() == special_runs(pl.spec_vis), f
            o.check_run(b)
            assert code_of(c.run, b) == "UNSUPPORTED"
        for b in range(nb):
            if transient or (wl.dynamic and not decisions[f]):
                o.rollback_last_frame(b); c.rollback_last_frame(b)
            elif wl.dynamic:
                o.execute_deferred_eviction(b, S, W)
                c.execute_deferred_eviction(b, S, W)
        if transient:
            o.set_defer_eviction(False); c.set_defer_eviction(False)
        if f % 50 == 0 or f == frames - 1:
            assert_same(o, c)
    c.close()


def test_run_accepts_several_frames_of_queries():
    """The batch mode of the first frames runs all their queries at once:
    run() checks nq against its own bound, not against one frame."""
    import streaming_paged_kv_amd as spkv
    c = spkv.PagedKVCache(num_blocks=1, num_heads=4, head_dim=64, page_size=16,
                          patch_tokens=16, num_special_tokens=6, scale_frames=2,
                          sliding_window=4, headroom=2, max_total_frames=32, host_only=True)
    for _ in range(2):
        c.append_frame(0)
        c.evict_frames(0, 2, 4)
    c.plan()
    for nq in (1, 22, 44, 1 << 20):
        assert code_of(lambda: c.run(0, nq=nq)) == "UNSUPPORTED", nq   # checks passed
    for nq in (0, (1 << 20) + 1):
        assert code_of(lambda: c.run(0, nq=nq)) == "INVALID_ARG", nq
    c.close()


def test_run_batch_checks_every_request_first():
    """run_batch (several streams in one launch) applies run()'s checks to
    every request before anything is enqueued: the first failing request's
    code comes back, and host-only handles report UNSUPPORTED only once all
    requests pass."""
    cfg = CFGS[0]
    caches = [spkv.PagedKVCache(host_only=True, **cfg) for _ in range(3)]
    oracles = [PagePoolOracle(OracleConfig(**cfg)) for _ in range(3)]
    req = lambda i, **kw: dict(cache=caches[i], block=kw.pop("block", 0), **kw)
    batch = lambda *rs: code_of(lambda: spkv.run_batch(list(rs)))
    # nothing planned yet: the first request's NOT_PLANNED
    assert batch(req(0), req(1)) == "NOT_PLANNED"
    for o, c in zip(oracles, caches):
        for _ in range(3):
            o.append_frame(0); c.append_frame(0)
            o.evict_frames(0, cfg["scale_frames"], cfg["sliding_window"])
            c.evict_frames(0, cfg["scale_frames"], cfg["sliding_window"])
    oracles[0].plan(); caches[0].plan()
    oracles[2].plan(); caches[2].plan()
    assert batch(req(0), req(1)) == "NOT_PLANNED"        # request 1 unplanned
    oracles[1].plan(); caches[1].plan()
    assert batch(req(0), req(1), req(2)) == "UNSUPPORTED"  # every check passed
    assert batch(req(0), req(2, nq=44)) == "UNSUPPORTED"
    assert batch(req(1, block=2), req(0)) == "BAD_BLOCK"
    assert batch(req(0), req(1, nq=0)) == "INVALID_ARG"
    assert batch(req(0), req(1, sm_scale=float("nan"))) == "INVALID_ARG"
    assert batch(req(0), req(0)) == "INVALID_ARG"          # a handle twice
    assert code_of(lambda: spkv.run_batch([req(0)] * 0)) != "OK"
    many = [spkv.PagedKVCache(host_only=True, **cfg) for _ in range(spkv.MAX_BATCH + 1)]
    for c in many:
        c.append_frame(0); c.plan()
    assert code_of(lambda: spkv.run_batch(
        [dict(cache=c, block=0) for c in many[:spkv.MAX_BATCH]])) == "UNSUPPORTED"
    assert code_of(lambda: spkv.run_batch(
        [dict(cache=c, block=0) for c in many])) == "INVALID_ARG"
    # STALE_PLAN: block 1 of stream 2 changes after its plan
    caches[2].append_frame(1)
    oracles[2].append_frame(1)
    assert code_of(oracles[2].check_run, 1) == "STALE_PLAN"
    assert batch(req(0), req(2, block=1)) == "STALE_PLAN"
    # the state of every handle is what the oracle holds
    for o, c in zip(oracles, caches):
        assert_same(o, c)
    for c in caches + many:
        c.close()


def test_separate_handles_from_concurrent_threads():
    """Handles share no state: eight threads, each driving its own host-only
    handle (the C calls run without the interpreter lock) through a seeded
    random operation sequence, each checked step by step against its own
    oracle."""
    import random
    import threading
    ops = ["append", "append", "append", "evict", "evict", "defer", "execute",
           "rollback", "plan", "plan", "run", "run_own", "reset", "evict_badS",
           "evict_flags"]
    errors = []

    def worker(t):
        rng = random.Random(1000 + t)
        o, c = make_pair(**CFGS[t % len(CFGS)])
        try:
            for _ in range(400):
                step(o, c, rng.choice(ops), rng.randint(-1, 3), rng.randint(0, 6))
                assert_same(o, c)
        except Exception as e:      # reported by the main thread
            errors.append((t, repr(e)))
        finally:
            c.close()

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
