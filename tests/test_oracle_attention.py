"""Pins of the oracle's attention (Part 2) and of Parts 1+2 together against
the page-free brute-force model (Part 3), closed-form special cases of
softmax attention, and a library cross-check.  CPU only."""

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle.attention as att
from oracle import (BruteForceStream, OracleConfig, OracleError, PagePoolOracle,
                    bf16_bits_to_f64, f64_to_bf16_bits)


# Called through the module so that planted mistakes (test_oracle_mutants)
# reach every pin.
def dense_attention(*a, **kw):
    return att.dense_attention(*a, **kw)


def gather_visible(*a, **kw):
    return att.gather_visible(*a, **kw)


def paged_attention(*a, **kw):
    return att.paged_attention(*a, **kw)


def rand_bits(rng, shape, scale=1.0):
    return f64_to_bf16_bits(rng.standard_normal(shape) * scale)


def run_stream(cfg, schedule, seed, sm_scale=0.125, flags=(1, 0)):
    """Drive the page-pool oracle and the brute-force model side by side.

    schedule: list of 'key' (append + evict, committed), 'transient' (defer,
    append, attend, rollback), 'accept'/'reject' (append under deferral,
    attend, then execute / rollback), 'reset'.  Every evict_frames call
    passes `flags` (cross_frame_special, camera_only); the brute-force model
    keeps as many specials of a frame past the window as those flags say.
    Returns the number of attention comparisons made.
    """
    rng = np.random.default_rng(seed)
    o = PagePoolOracle(cfg, track_pool=[0])
    kept = 0 if not flags[0] else 1 if flags[1] else cfg.num_special_tokens
    bf = BruteForceStream(cfg.scale_frames, cfg.sliding_window, cfg.num_special_tokens,
                          kept=kept)
    t, h, d = cfg.tokens_per_frame, cfg.num_heads, cfg.head_dim
    n_cmp = 0
    for ev in schedule:
        if ev == "reset":
            o.reset()
            bf.reset()
            continue
        q = rand_bits(rng, (t, h, d))
        k = rand_bits(rng, (t, h, d), 0.7)
        v = rand_bits(rng, (t, h, d))
        if ev == "key":
            try:
                o.append_frame(0, k, v)
            except OracleError:
                return n_cmp
            o.evict_frames(0, cfg.scale_frames, cfg.sliding_window, *flags)
            bf.commit(bf16_bits_to_f64(k), bf16_bits_to_f64(v))
            own = (None, None)
        else:
            # run_own's definition over the committed cache must give the same
            # attention as the transient append (same tokens, other order)
            try:
                pl0 = o.plan()
            except OracleError:
                pl0 = None
            with_own = None
            if pl0 is not None:
                with_own = att.paged_attention_with_own(o.pools[0], pl0, cfg, q, k, v,
                                                        sm_scale)
            o.set_defer_eviction(True)
            try:
                o.append_frame(0, k, v)
            except OracleError:
                o.set_defer_eviction(False)
                return n_cmp
            o.evict_frames(0, cfg.scale_frames, cfg.sliding_window, *flags)  # no-op
            own = (bf16_bits_to_f64(k), bf16_bits_to_f64(v))
        pl = o.plan()
        o.check_run(0)
        got = paged_attention(o.pools[0], pl, cfg, q, sm_scale)
        want, nk = bf.attend(bf16_bits_to_f64(q), sm_scale, *own)
        assert pl.num_visible_tokens(cfg) == nk
        # same tokens in the same order through the same float64 code path
        assert np.array_equal(got, want)
        if ev != "key" and with_own is not None:
            np.testing.assert_allclose(with_own, got, rtol=1e-10, atol=1e-12)
        n_cmp += 1
        if ev in ("transient", "reject"):
            o.rollback_last_frame(0)
        elif ev == "accept":
            o.execute_deferred_eviction(0, cfg.scale_frames, cfg.sliding_window)
            bf.commit(*own)
        if ev != "key":
            o.set_defer_eviction(False)
    return n_cmp


TINY = OracleConfig(1, 2, 8, 16, 16, 6, 2, 4, 2, 32)


def test_brute_force_tiny_keyframes():
    assert run_stream(TINY, ["key"] * 12, 1) == 12


def test_brute_force_interval_two():
    assert run_stream(TINY, ["key", "transient"] * 8, 2) == 16


def test_brute_force_dynamic_accept_reject():
    rng = np.random.default_rng(3)
    sched = ["accept" if rng.random() < 0.4 else "reject" for _ in range(30)]
    assert run_stream(TINY, sched, 3) == 30


def test_brute_force_reset_mid_stream():
    sched = ["key"] * 7 + ["reset"] + ["key", "transient"] * 5 + ["reset", "key"]
    assert run_stream(TINY, sched, 4) == 18


def test_brute_force_padded_pages_and_odd_sizes():
    # 13 patch tokens in 16-token pages (pad never read); 2 frames per special page
    c = OracleConfig(1, 3, 4, 16, 13, 6, 2, 3, 2, 20)
    assert run_stream(c, ["key", "transient", "accept", "reject"] * 6, 5) == 24
    # special pages packing 3 frames of 4 special tokens in 13-slot pages
    c2 = OracleConfig(1, 2, 4, 13, 11, 4, 1, 2, 1, 20)
    assert run_stream(c2, ["key"] * 9 + ["transient", "accept"] * 4, 6) == 17


@settings(max_examples=60, deadline=None)
@given(sched=st.lists(st.sampled_from(["key", "transient", "accept", "reject", "reset"]),
                      min_size=1, max_size=25),
       s=st.integers(0, 3), w=st.integers(1, 4), seed=st.integers(0, 1000),
       flags=st.sampled_from([(1, 0), (1, 1), (0, 0), (0, 1)]))
def test_brute_force_random_schedules(sched, s, w, seed, flags):
    c = OracleConfig(1, 2, 4, 9, 7, 3, s, w, 2, 40)
    run_stream(c, sched, seed, flags=flags)


EVICTION_FLAGS = [(1, 1), (0, 0), (0, 1)]


@pytest.mark.parametrize("flags", EVICTION_FLAGS)
def test_brute_force_eviction_flags(flags):
    """Parts 1+2 against the page-free model when evicted frames keep only
    their camera token or none of their specials (reading R13): keyframes,
    interval two, accept/reject under deferral (execute_deferred_eviction
    takes the flags of the deferred evict_frames call) and resets."""
    assert run_stream(TINY, ["key"] * 12, 11, flags=flags) == 12
    assert run_stream(TINY, ["key", "transient"] * 8, 12, flags=flags) == 16
    rng = np.random.default_rng(13)
    sched = ["accept" if rng.random() < 0.4 else "reject" for _ in range(30)]
    assert run_stream(TINY, sched, 13, flags=flags) == 30
    sched = ["key"] * 9 + ["reset"] + ["key", "transient"] * 6
    assert run_stream(TINY, sched, 14, flags=flags) == 21
    c2 = OracleConfig(1, 2, 4, 13, 11, 4, 1, 2, 1, 20)
    assert run_stream(c2, ["key"] * 9 + ["transient", "accept"] * 4, 15, flags=flags) == 17


# --------------------------------------------------- attention special cases
def test_constant_v_gives_that_constant():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((7, 3, 16))
    k = rng.standard_normal((50, 3, 16)) * 3
    c = rng.standard_normal((3, 16))
    v = np.broadcast_to(c, (50, 3, 16))
    out = dense_attention(q, k, v, 0.125)
    assert np.allclose(out, np.broadcast_to(c, out.shape), rtol=0, atol=1e-13)


def test_equal_keys_give_mean_of_v():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((5, 2, 8))
    k = np.broadcast_to(rng.standard_normal((1, 2, 8)), (40, 2, 8))
    v = rng.standard_normal((40, 2, 8))
    out = dense_attention(q, k, v, 0.3)
    assert np.allclose(out, np.broadcast_to(v.mean(axis=0), out.shape), atol=1e-13)


def test_planted_key_dominates():
    rng = np.random.default_rng(12)
    d = 16
    q = rng.standard_normal((4, 1, d))
    k = rng.standard_normal((100, 1, d)) * 0.01
    v = rng.standard_normal((100, 1, d))
    j = 37
    # make token j's logit 40 above every other one for every query
    k[j, 0] = q.mean(axis=0)[0]
    out = dense_attention(q * 0 + q.mean(axis=0, keepdims=True), k, v,
                          40.0 / float(q.mean(axis=0)[0] @ q.mean(axis=0)[0]))
    assert np.allclose(out[:, 0], np.broadcast_to(v[j, 0], (4, d)), atol=1e-9)


def test_two_tokens_closed_form():
    """Two keys: the weight of the first is the logistic function of the logit
    difference."""
    q = np.array([[[1.0, 2.0]]])
    k = np.array([[[0.5, -1.0]], [[2.0, 0.25]]])
    v = np.array([[[3.0, 0.0]], [[-1.0, 4.0]]])
    s = 0.7
    a = s * (q[0, 0] @ k[0, 0])
    b = s * (q[0, 0] @ k[1, 0])
    w0 = 1.0 / (1.0 + np.exp(b - a))
    want = w0 * v[0, 0] + (1 - w0) * v[1, 0]
    assert np.allclose(dense_attention(q, k, v, s)[0, 0], want, rtol=0, atol=1e-15)


def test_matches_torch_sdpa_float64():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((33, 4, 64))
    k = rng.standard_normal((300, 4, 64))
    v = rng.standard_normal((300, 4, 64))
    got = dense_attention(q, k, v, 0.125)
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).permute(1, 0, 2)
    tv = torch.from_numpy(v).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.125)
    assert np.allclose(got, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_row_subset_equals_rows_of_full_result():
    rng = np.random.default_rng(14)
    c = TINY
    o = PagePoolOracle(c, track_pool=[0])
    t = c.tokens_per_frame
    for _ in range(5):
        o.append_frame(0, rand_bits(rng, (t, 2, 8)), rand_bits(rng, (t, 2, 8)))
        o.evict_frames(0, 2, 4)
    pl = o.plan()
    q = rand_bits(rng, (t, 2, 8))
    full = paged_attention(o.pools[0], pl, c, q, 0.125)
    rows = [0, 5, 21]
    assert np.array_equal(paged_attention(o.pools[0], pl, c, q, 0.125, rows=rows), full[rows])


def test_exact_and_padded_layouts_agree():
    """Same stream, page_size 13 (exact) vs 16 (padded): identical outputs."""
    rng = np.random.default_rng(15)
    ce = OracleConfig(1, 2, 8, 13, 13, 6, 2, 3, 2, 12)
    cp = OracleConfig(1, 2, 8, 16, 13, 6, 2, 3, 2, 12)
    oe, op = PagePoolOracle(ce, track_pool=[0]), PagePoolOracle(cp, track_pool=[0])
    for f in range(9):
        k, v, q = (rand_bits(rng, (19, 2, 8)) for _ in range(3))
        for o in (oe, op):
            o.append_frame(0, k, v)
            o.evict_frames(0, 2, 3)
        a = paged_attention(oe.pools[0], oe.plan(), ce, q, 0.125)
        b = paged_attention(op.pools[0], op.plan(), cp, q, 0.125)
        assert np.array_equal(a, b)


def test_gather_reads_only_valid_slots():
    """Garbage in the pad and in unused special slots never reaches the
    gathered sequence."""
    rng = np.random.default_rng(16)
    c = OracleConfig(1, 1, 2, 16, 13, 6, 1, 2, 1, 8)
    o = PagePoolOracle(c, track_pool=[0])
    o.pools[0][:] = 0x7FC0   # NaN everywhere before any write
    for _ in range(3):
        o.append_frame(0, rand_bits(rng, (19, 1, 2)), rand_bits(rng, (19, 1, 2)))
        o.evict_frames(0, 1, 2)
    k, v = gather_visible(o.pools[0], o.plan(), c)
    assert k.shape[0] == 3 * 13 + 18
    assert np.isfinite(k).all() and np.isfinite(v).all()
