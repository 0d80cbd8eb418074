"""Parity of the HIP path (through the C ABI) with the oracle on the GPU.

Bar: page tables, last_page_len, stats and allocator state bit-exact at every
frame; pool bytes bit-exact (whole pool on small streams; the visible patch
pages and every special page at chosen frames on full-size streams);
attention within max-abs 2e-2 and mean-abs 2e-3 of the float64 oracle, with
relative L2 error <= 1e-2 as an extra guard."""

import numpy as np
import pytest
import torch

import synth
import harness as H
from oracle import OracleConfig, PagePoolOracle
from oracle.attention import paged_attention
from oracle.pagepool import special_runs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def new_cache(wl, **kw):
    import streaming_paged_kv_amd as spkv
    return spkv.PagedKVCache(**wl.cfg_kwargs(), **kw)


def log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------ small streams
def full_parity(wl, frames=None, splits=0, flags=(1, 0), in_run=False):
    """Every frame: whole-pool bytes, plan (with its visible special runs),
    stats, state bit-exact; attention on every row of every block.  Every
    evict_frames call passes the eviction flags."""
    need_gpu()
    cache = new_cache(wl)
    if splits:
        cache.set_num_splits(splits)
    cfg = OracleConfig(**wl.cfg_kwargs())
    o = PagePoolOracle(cfg, track_pool=range(wl.num_blocks))
    kinds = H.frame_kinds(wl, frames)
    sm = wl.head_dim ** -0.5
    worst = 0.0
    for f, (kind, reset) in enumerate(kinds):
        qkv = H.gen_frame(wl, f, wl.num_blocks, DEV)
        bits = [[synth.bf16_bits(t) for t in x] for x in qkv]
        outs = [torch.empty_like(x[0]) for x in qkv]
        # oracle first so that its attention uses the state of this frame
        ref = {}
        S, W = wl.scale_frames, wl.sliding_window
        if reset:
            o.reset()
        if wl.dynamic or kind == "transient":
            o.set_defer_eviction(True)
        for b in range(wl.num_blocks):
            o.append_frame(b, bits[b][1], bits[b][2])
            o.evict_frames(b, S, W, *flags)
            if b == 0:
                o.plan()
            pl = o.check_run(b)
            ref[b] = paged_attention(o.pools[b], pl, cfg, bits[b][0], sm)
        plan_ref = (list(o.plan_state.table), o.plan_state.n_patch,
                    o.plan_state.last_page_len)
        specials_ref = special_runs(o.plan_state.spec_vis)
        for b in range(wl.num_blocks):
            if kind in ("transient", "reject"):
                o.rollback_last_frame(b)
            elif kind == "accept":
                o.execute_deferred_eviction(b, S, W)
        if kind == "transient":
            o.set_defer_eviction(False)

        H.gpu_step(cache, wl, kind, reset, qkv, outs, flags=flags, in_run=in_run)
        torch.cuda.synchronize()
        assert cache.get_plan() == plan_ref, f
        assert cache.get_plan_specials() == specials_ref, f
        for b in range(wl.num_blocks):
            assert o.special_visibility(b) == cache.get_block_specials(b), (f, b)
            assert list(o.block_state(b)) == list(cache.get_block_state(b)), (f, b)
            assert tuple(o.get_cache_stats(b)) == cache.get_cache_stats(b), (f, b)
            assert np.array_equal(synth.bf16_bits(cache.pools[b]), o.pools[b]), (f, b)
            mx, mean, rel = H.compare(outs[b], ref[b], (wl.name, f, b))
            worst = max(worst, mx)
    cache.close()
    return worst


def test_tiny_stream_every_frame():
    log("tiny stream, 12 keyframes")
    full_parity(synth.WORKLOADS["tiny"])


def test_tiny_stream_interval_reset_and_rollback():
    wl = synth.WORKLOADS["tiny"].with_(keyframe_interval=2, frames=14, reset_every=9)
    log("tiny stream, interval 2, reset at 9")
    full_parity(wl)
    wl2 = synth.WORKLOADS["tiny"].with_(dynamic=True, frames=20, seed=11)
    log("tiny stream, dynamic accept/rollback")
    full_parity(wl2)


MID = synth.Workload("mid-ragged", 2, 16, 64, 203, 200, 6, 2, 6, 2, 64, 16,
                     keyframe_interval=2, seed=21)


@pytest.mark.parametrize("flags", [(1, 1), (0, 0)])
def test_tiny_stream_eviction_flags(flags):
    """Evicted frames keep only their camera token, or none of their specials:
    the row map skips the hidden special slots (and the special pages left
    with none), the pool bytes do not change.  Keyframes, interval 2 with a
    reset, and accept/rollback under deferral (the deferred flags apply)."""
    tiny = synth.WORKLOADS["tiny"]
    log(f"tiny stream, flags {flags}")
    full_parity(tiny, flags=flags)
    full_parity(tiny.with_(keyframe_interval=2, frames=14, reset_every=9), flags=flags)
    full_parity(tiny.with_(dynamic=True, frames=20, seed=12), flags=flags)


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_append_folded_into_run_small_streams(splits):
    """append_frame_in_run + run: whole-pool bytes, plans and attention every
    frame on the tiny stream (keyframes; interval 2 with a reset; dynamic
    accept/rollback) and the 203-token-page stream with forced splits."""
    tiny = synth.WORKLOADS["tiny"]
    log(f"append in run, splits {splits}")
    full_parity(tiny, splits=splits, in_run=True)
    full_parity(tiny.with_(keyframe_interval=2, frames=14, reset_every=9), splits=splits,
                in_run=True)
    full_parity(tiny.with_(dynamic=True, frames=20, seed=13), splits=splits, in_run=True)
    full_parity(MID.with_(frames=30), splits=splits, in_run=True)


def test_append_folded_into_run_flushed_by_other_calls():
    """A frame admitted by append_frame_in_run is copied before any call that
    needs its bytes: the block's next append (both kinds), its rollback,
    run_own, run_noalloc, run_batch and reset.  The pool bytes follow the
    oracle, which copies at admission, after each of them."""
    need_gpu()
    import streaming_paged_kv_amd as spkv
    wl = MID.with_(num_blocks=2, frames=12, keyframe_interval=1)
    cfg = OracleConfig(**wl.cfg_kwargs())
    o = PagePoolOracle(cfg, track_pool=[0, 1])
    cache = new_cache(wl)
    S, W = wl.scale_frames, wl.sliding_window
    sm = wl.head_dim ** -0.5

    def admit(f, b, how):
        q, k, v = synth.frame_qkv(wl, f, b, device=DEV)
        if how == "in_run":
            cache.append_frame_in_run(b, k, v)
        else:
            cache.append_frame(b, k, v)
        o.append_frame(b, synth.bf16_bits(k), synth.bf16_bits(v))
        return q, k, v

    def same_pools(what):
        torch.cuda.synchronize()
        for b in range(2):
            assert np.array_equal(synth.bf16_bits(cache.pools[b]), o.pools[b]), (what, b)

    f = 0
    # the block's next append, of either kind, copies the pending frame first
    admit(f, 0, "in_run"); f += 1
    admit(f, 0, "in_run"); f += 1      # copies frame 0; frame 1 waits
    admit(f, 0, "plain"); f += 1       # copies frame 1
    cache.evict_frames(0, S, W); o.evict_frames(0, S, W)
    same_pools("next append")
    # block 1 catches up so that both blocks hold the same frames
    for g in range(f):
        admit(g, 1, "plain")
        cache.evict_frames(1, S, W); o.evict_frames(1, S, W)
    # rollback under deferral
    cache.set_defer_eviction(True); o.set_defer_eviction(True)
    admit(f, 0, "in_run")
    cache.rollback_last_frame(0); o.rollback_last_frame(0)
    cache.set_defer_eviction(False); o.set_defer_eviction(False)
    same_pools("rollback")
    f += 1
    # run_own / run_noalloc / run_batch on a block with a pending copy
    for call in ("run_own", "run_noalloc", "run_batch"):
        q, k, v = admit(f, 0, "in_run")
        admit(f, 1, "plain")
        for b in range(2):
            cache.evict_frames(b, S, W); o.evict_frames(b, S, W)
        cache.plan(); pl = o.plan()
        if call == "run_own":
            q2, k2, v2 = synth.frame_qkv(wl, f + 100, 0, device=DEV)
            out = cache.run_own(0, q2, k2, v2)
            from oracle.attention import paged_attention_with_own
            ref = paged_attention_with_own(o.pools[0], pl, cfg, synth.bf16_bits(q2),
                                           synth.bf16_bits(k2), synth.bf16_bits(v2), sm)
        elif call == "run_noalloc":
            out = cache.run_noalloc(0, q)
            ref = paged_attention(o.pools[0], pl, cfg, synth.bf16_bits(q), sm)
        else:
            out = spkv.run_batch([dict(cache=cache, block=0, q=q)])[0]
            ref = paged_attention(o.pools[0], pl, cfg, synth.bf16_bits(q), sm)
        same_pools(call)
        H.compare(out, ref, (call, f))
        f += 1
    # reset with a pending copy
    admit(f, 0, "in_run")
    cache.reset(); o.reset()
    same_pools("reset")
    cache.close()


@pytest.mark.parametrize("flags,splits", [((1, 1), 0), ((0, 0), 3), ((0, 1), 7)])
def test_mid_stream_eviction_flags(flags, splits):
    """200-token patch pages (33 frames per special page) with the special
    stream thinned to camera tokens or cut to the held frames, key-range
    splits crossing the special runs."""
    log(f"mid stream, flags {flags}, splits {splits}")
    full_parity(MID.with_(frames=60), flags=flags, splits=splits)


@pytest.mark.parametrize("splits", [0, 1, 3, 7])
def test_mid_stream_ragged_pages_and_splits(splits):
    """200 patch tokens in 203-token pages, 33 frames per special page: tiles
    cross pages at varying offsets; forced key-range splits."""
    log(f"mid stream, splits={splits}")
    full_parity(MID, splits=splits)


DEGENERATE = synth.Workload("degenerate", 2, 3, 64, 6, 5, 6, 0, 1, 1, 30, 30, seed=41)


@pytest.mark.parametrize("splits", [0, 3])
def test_degenerate_geometry(splits):
    """No scale frames, a one-page window with one page of headroom, 6-token
    pages (one frame per special page, so a 64-key tile spans 11 pages),
    5 patch tokens in 6-token pages, 3 heads, and the special stream filled
    to its last slot (30 frames, 30 special pages)."""
    log(f"degenerate geometry, splits={splits}")
    full_parity(DEGENERATE, splits=splits)
    cache = new_cache(DEGENERATE)
    import streaming_paged_kv_amd as spkv
    for f in range(DEGENERATE.frames):
        _, k, v = synth.frame_qkv(DEGENERATE, f, 0, device=DEV)
        cache.append_frame(0, k, v)
        cache.evict_frames(0, 0, 1)
    with pytest.raises(spkv.SpkvError) as ei:
        cache.append_frame(0, k, v)
    assert ei.value.name == "SPECIAL_OVERFLOW"
    cache.close()


def test_many_heads():
    """80 heads: 10 KiB token rows in the pool, 80 work items per query tile
    and split, head slices past the first 8 KiB of a row."""
    wl = synth.Workload("80-heads", 1, 80, 64, 64, 58, 6, 1, 3, 1, 40, 8, seed=42)
    log("80 heads")
    full_parity(wl)


BIGQ = synth.Workload("bigq", 1, 16, 64, 999, 999, 6, 1, 2, 1, 400, 6,
                      keyframe_interval=2, k_scale=0.5, seed=22)


def test_many_query_tiles_and_ragged_query_tail():
    """1005 query rows = one full 512-row query tile plus a 493-row tail."""
    log("1005 queries, 999-token pages")
    full_parity(BIGQ)


def test_exact_and_padded_pages_give_identical_outputs():
    """The same token stream in 999- and 1024-token pages: the kernel walks
    the same token sequence, so the outputs are bit-identical."""
    need_gpu()
    a = BIGQ.with_(name="exact", frames=5)
    b = BIGQ.with_(name="padded", page_size=1024, frames=5)
    ca, cb = new_cache(a), new_cache(b)
    for c in (ca, cb):
        c.set_num_splits(3)
    for f, (kind, reset) in enumerate(H.frame_kinds(a)):
        qkv = H.gen_frame(a, f, 1, DEV)
        oa = [torch.empty_like(qkv[0][0])]
        ob = [torch.empty_like(qkv[0][0])]
        H.gpu_step(ca, a, kind, reset, qkv, oa)
        H.gpu_step(cb, b, kind, reset, qkv, ob)
        torch.cuda.synchronize()
        assert torch.equal(oa[0], ob[0]), f
    ca.close()
    cb.close()


# ----------------------------------------------------------- edge cases
def test_edge_cases_nq_scale_and_sharp_keys():
    need_gpu()
    wl = MID.with_(name="edge", num_blocks=1, frames=6, keyframe_interval=1)
    cfg = OracleConfig(**wl.cfg_kwargs())
    o = PagePoolOracle(cfg, track_pool=[0])
    cache = new_cache(wl)
    for f in range(wl.frames):
        q, k, v = synth.frame_qkv(wl, f, 0, device=DEV)
        if f == 3:
            # plant: key of patch token 17 is a large multiple of query 0's
            k = k.clone()
            k[6 + 17] = (q[0].float() * 4.0).to(torch.bfloat16)
        cache.append_frame(0, k, v)
        cache.evict_frames(0, wl.scale_frames, wl.sliding_window)
        cache.plan()
        o.append_frame(0, synth.bf16_bits(k), synth.bf16_bits(v))
        o.evict_frames(0, wl.scale_frames, wl.sliding_window)
        pl = o.plan()
        qb = synth.bf16_bits(q)
        for nq, sm in ((1, 0.125), (7, 1.0), (wl.tokens_per_frame, 0.02),
                       (33, 0.125)):
            out = cache.run(0, q[:nq].contiguous(), sm_scale=sm)
            torch.cuda.synchronize()
            ref = paged_attention(o.pools[0], pl, cfg, qb[:nq], sm)
            H.compare(out, ref, ("edge", f, nq, sm))
    cache.close()


def test_maximum_query_rows():
    """The largest query count run() takes (2^20 rows, 2048 query tiles x 4
    heads = 8192 work items) over a tiny stream's 12 frames: sampled rows
    (first, last, tile edges, random) against the oracle, at the automatic
    split and at a forced split of 3 (2^20 x 4 x 64 fp32 partials)."""
    need_gpu()
    wl = synth.WORKLOADS["tiny"]
    cfg = OracleConfig(**wl.cfg_kwargs())
    o = PagePoolOracle(cfg, track_pool=[0])
    import streaming_paged_kv_amd as spkv
    nq = 1 << 20
    # workspace for 3 splits of 2^20 rows: partial O + (m, l)
    ws = spkv.query_sizes(**wl.cfg_kwargs())[2] + 3 * nq * wl.num_heads * (64 + 2) * 4 + 4096
    cache = new_cache(wl, workspace_bytes=ws)
    for f in range(wl.frames):
        q, k, v = synth.frame_qkv(wl, f, 0, device=DEV)
        cache.append_frame(0, k, v)
        cache.evict_frames(0, wl.scale_frames, wl.sliding_window)
        o.append_frame(0, synth.bf16_bits(k), synth.bf16_bits(v))
        o.evict_frames(0, wl.scale_frames, wl.sliding_window)
    cache.plan()
    pl = o.plan()
    gen = torch.Generator(device=DEV).manual_seed(77)
    q = torch.randn((nq, wl.num_heads, wl.head_dim), generator=gen,
                    device=DEV).to(torch.bfloat16)
    rows = H.sample_rows(nq, extra=48, seed=5) + [nq - 512, nq - 513, (nq >> 1) + 17]
    rows = sorted(set(rows))
    qb = synth.bf16_bits(q[rows])
    ref = paged_attention(o.pools[0], pl, cfg, qb, wl.head_dim ** -0.5)
    for splits in (0, 3):
        cache.set_num_splits(splits)
        out = cache.run(0, q)
        torch.cuda.synchronize()
        H.compare(out[rows], ref, ("max nq", splits))
    cache.close()


# 4094 patch pages + 2 special pages of 1 MiB (256 tokens x 16 heads x 64 dims,
# K and V): a pool of exactly 4 GiB, whose special pages lie at the top of
# the range that 32-bit byte offsets address.
POOL_4GIB = synth.Workload("pool-4GiB", 1, 16, 64, 256, 256, 6, 2, 4090, 2, 84, 44, seed=31)


def test_pool_offsets_up_to_4gib_and_pool_size_limits():
    """run() on a 4 GiB pool: the special pages sit at byte offsets 4094 MiB
    and 4095 MiB (the second from frame 42 on, 42 frames per special page),
    so the kernel's loads use offsets above 2^31 up to the top of the 32-bit
    range.  Attention and the visible pages' bytes against the oracle at
    chosen frames.  run_own() on that pool is UNSUPPORTED (its row map marks
    the caller's rows with the offsets' top bit), and run() on a pool one
    page over 4 GiB is UNSUPPORTED, with nothing enqueued."""
    need_gpu()
    import streaming_paged_kv_amd as spkv
    wl = POOL_4GIB
    assert spkv.query_sizes(**wl.cfg_kwargs())[1] == 1 << 32
    cfg = OracleConfig(**wl.cfg_kwargs())
    o = PagePoolOracle(cfg, track_pool=[0])
    cache = new_cache(wl)
    S, W = wl.scale_frames, wl.sliding_window
    sm = wl.head_dim ** -0.5
    checked = 0
    for f in range(wl.frames):
        q, k, v = synth.frame_qkv(wl, f, 0, device=DEV)
        cache.append_frame(0, k, v)
        cache.evict_frames(0, S, W)
        cache.plan()
        out = cache.run(0, q)
        o.append_frame(0, synth.bf16_bits(k), synth.bf16_bits(v))
        o.evict_frames(0, S, W)
        pl = o.plan()
        if f not in (0, 1, 5, 41, 42, 43):
            continue
        torch.cuda.synchronize()
        table = list(o.plan_state.table)
        assert cache.get_plan()[0] == table, f
        assert table[-1] == 4094 + f // 42, f
        ref = paged_attention(o.pools[0], pl, cfg, synth.bf16_bits(q), sm)
        H.compare(out, ref, ("4 GiB pool", f))
        for page in table:
            assert np.array_equal(synth.bf16_bits(cache.pools[0][page]), o.pools[0][page]), (f, page)
        checked += 1
        log(f"  4 GiB pool frame {f}: table ends at page {table[-1]}")
    assert checked == 6
    q, k, v = synth.frame_qkv(wl, wl.frames, 0, device=DEV)
    with pytest.raises(spkv.SpkvError) as ei:
        cache.run_own(0, q, k, v)
    assert ei.value.name == "UNSUPPORTED"
    cache.close()
    del cache
    torch.cuda.empty_cache()

    over = wl.with_(name="pool-4GiB+1MiB", sliding_window=4091, frames=1)
    assert spkv.query_sizes(**over.cfg_kwargs())[1] == (1 << 32) + (1 << 20)
    cache = new_cache(over)
    q, k, v = synth.frame_qkv(over, 0, 0, device=DEV)
    cache.append_frame(0, k, v)
    cache.plan()
    out = torch.full_like(q, 7.0)
    with pytest.raises(spkv.SpkvError) as ei:
        cache.run(0, q, out=out)
    assert ei.value.name == "UNSUPPORTED"
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    cache.close()


def test_run_batch_plain_run_on_4gib_pool_beside_run_own():
    """A batch that holds a run_own() request launches the kernel variant that
    reads the caller's own rows; a plain run() request in the same launch
    must still read its row offsets as pool rows, also those with the top bit
    set.  The plain request runs on the 4 GiB pool, whose special pages lie
    at byte offsets 4094 MiB and up; the run_own request on a small stream.
    Both against the oracle, with forced 1 and 3 splits."""
    need_gpu()
    import streaming_paged_kv_amd as spkv
    big = POOL_4GIB
    small = synth.WORKLOADS["tiny"].with_(name="tiny-own", seed=33)
    cfg_b = OracleConfig(**big.cfg_kwargs())
    cfg_s = OracleConfig(**small.cfg_kwargs())
    ob = PagePoolOracle(cfg_b, track_pool=[0])
    osm = PagePoolOracle(cfg_s, track_pool=[0])
    cb, cs = new_cache(big), new_cache(small)
    sm = 0.125
    for f in range(3):
        for wl, c, o in ((big, cb, ob), (small, cs, osm)):
            q, k, v = synth.frame_qkv(wl, f, 0, device=DEV)
            c.append_frame(0, k, v)
            c.evict_frames(0, wl.scale_frames, wl.sliding_window)
            o.append_frame(0, synth.bf16_bits(k), synth.bf16_bits(v))
            o.evict_frames(0, wl.scale_frames, wl.sliding_window)
    cb.plan()
    cs.plan()
    pb, ps = ob.plan(), osm.plan()
    qb = synth.frame_qkv(big, 10, 0, device=DEV)[0]
    qs, ks, vs = synth.frame_qkv(small, 10, 0, device=DEV)
    ref_b = paged_attention(ob.pools[0], pb, cfg_b, synth.bf16_bits(qb), sm)
    from oracle.attention import paged_attention_with_own
    ref_s = paged_attention_with_own(osm.pools[0], ps, cfg_s, synth.bf16_bits(qs),
                                     synth.bf16_bits(ks), synth.bf16_bits(vs), sm)
    assert cb.get_plan()[0][-1] == 4094
    for splits in (1, 3):
        cb.set_num_splits(splits)
        cs.set_num_splits(splits)
        log(f"  4 GiB run() beside a run_own(), splits {splits}")
        outs = spkv.run_batch([dict(cache=cb, block=0, q=qb, sm_scale=sm),
                               dict(cache=cs, block=0, q=qs, k=ks, v=vs, sm_scale=sm)])
        torch.cuda.synchronize()
        H.compare(outs[0], ref_b, ("4 GiB run in an own batch", splits))
        H.compare(outs[1], ref_s, ("run_own beside a 4 GiB run", splits))
    cb.close()
    cs.close()
    del cb
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["all_far_below", "all_far_above", "mixed"])
def test_extreme_logits(mode):
    """Scores far from 0: every score of a frame about -50 (every p would
    underflow unless the reference follows the maximum), every score about
    +50 (every p would overflow), and a mix of frames of both kinds with a
    planted sharp key.  Three forced key-range splits give several first
    tiles per run."""
    need_gpu()
    wl = MID.with_(name="extreme", num_blocks=1, frames=5, keyframe_interval=1)
    cfg = OracleConfig(**wl.cfg_kwargs())
    o = PagePoolOracle(cfg, track_pool=[0])
    cache = new_cache(wl)
    cache.set_num_splits(3)
    n, h, d = wl.tokens_per_frame, wl.num_heads, wl.head_dim
    u = torch.full((h, d), 2.5, device=DEV)          # |u|^2 = 400 per head
    gen = torch.Generator(device=DEV).manual_seed(31)
    for f in range(wl.frames):
        q, k, v = synth.frame_qkv(wl, f, 0, device=DEV)
        noise = 0.5 * torch.randn((n, h, d), generator=gen, device=DEV)
        if mode == "all_far_below":
            sign = -1.0                              # s * q.k ~ -50: x ~ -72
        elif mode == "all_far_above":
            sign = 1.0                               # x ~ +72
        else:
            sign = -1.0 if f % 2 else 1.0
        q = (u + 0.2 * q.float()).to(torch.bfloat16)
        k = (sign * u + noise).to(torch.bfloat16)
        if mode == "mixed" and f == 3:
            k[6 + 40] = (q[0].float() * 1.5).to(torch.bfloat16)
        cache.append_frame(0, k, v)
        cache.evict_frames(0, wl.scale_frames, wl.sliding_window)
        cache.plan()
        o.append_frame(0, synth.bf16_bits(k), synth.bf16_bits(v))
        o.evict_frames(0, wl.scale_frames, wl.sliding_window)
        pl = o.plan()
        out = cache.run(0, q, sm_scale=0.125)
        torch.cuda.synchronize()
        ref = paged_attention(o.pools[0], pl, cfg, synth.bf16_bits(q), 0.125)
        H.compare(out, ref, ("extreme", mode, f))
    cache.close()


@pytest.mark.parametrize("name", ["224x224", "518x378"])
def test_planted_sharp_keys_at_full_geometry(name):
    """Sharp softmax at the full-size geometries (one block, the window full
    and evicting): keys planted along chosen query rows of the last frame, in
    a scale frame's page, a live page and a special slot, plus one row with
    two nearly equal planted keys, so that a few keys carry almost all of the
    weight and the output is a visible value vector rather than an average of
    ~1e-3.  Sampled rows (the planted ones among them) of all heads against
    the oracle, at the automatic split and at a forced 5-way split."""
    need_gpu()
    base = synth.WORKLOADS[name]
    wl = base.with_(name=f"{name}-sharp", num_blocks=1, keyframe_interval=1,
                    frames=base.scale_frames + base.sliding_window + 8)
    cfg = OracleConfig(**wl.cfg_kwargs())
    o = PagePoolOracle(cfg, track_pool=[0])
    cache = new_cache(wl)
    last = wl.frames - 1
    q_fin = synth.frame_qkv(wl, last, 0, device=DEV)[0]
    # (frame, token of the frame, query row of the last frame, gain)
    nq = wl.tokens_per_frame
    plants = [(3, 6 + 100, 11, 4.0),            # scale page
              (last - 5, 6 + 200, 300 % nq, 4.0),   # live page
              (40, 2, 600 % nq, 4.0),           # special slot (register 2)
              (50, 6 + 17, 7, 3.0), (60, 6 + 18, 7, 2.95)]   # two close keys
    for f in range(wl.frames):
        q, k, v = synth.frame_qkv(wl, f, 0, device=DEV)
        for pf, tok, row, gain in plants:
            if pf == f:
                k = k.clone()
                k[tok] = (q_fin[row].float() * gain).to(torch.bfloat16)
        cache.append_frame(0, k, v)
        cache.evict_frames(0, wl.scale_frames, wl.sliding_window)
        o.append_frame(0, synth.bf16_bits(k), synth.bf16_bits(v))
        o.evict_frames(0, wl.scale_frames, wl.sliding_window)
    assert cache.get_cache_stats(0)[2] == wl.sliding_window
    cache.plan()
    pl = o.plan()
    rows = sorted(set(H.sample_rows(wl.tokens_per_frame, extra=16, seed=9)) |
                  {p[2] for p in plants})
    ref = paged_attention(o.pools[0], pl, cfg, synth.bf16_bits(q_fin[rows]), 0.125)
    sharp = np.abs(ref).max(axis=(1, 2))
    assert (sharp[[rows.index(p[2]) for p in plants]] > 0.5).all()   # planted rows are sharp
    for splits in (0, 5):
        cache.set_num_splits(splits)
        out = cache.run(0, q_fin, sm_scale=0.125)
        torch.cuda.synchronize()
        log(f"  {name} sharp keys, splits {splits}")
        H.compare(out[rows], ref, ("sharp", name, splits))
    cache.close()


def test_constant_v_is_reproduced():
    need_gpu()
    wl = MID.with_(name="constv", num_blocks=1, frames=4, keyframe_interval=1)
    cache = new_cache(wl)
    cvec = torch.randn(16, 64, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    for f in range(wl.frames):
        q, k, _ = synth.frame_qkv(wl, f, 0, device=DEV)
        v = cvec.to(DEV).expand(wl.tokens_per_frame, 16, 64).contiguous()
        cache.append_frame(0, k, v)
        cache.evict_frames(0, wl.scale_frames, wl.sliding_window)
        cache.plan()
        out = cache.run(0, q)
        torch.cuda.synchronize()
        want = cvec.double().numpy()[None].repeat(wl.tokens_per_frame, 0)
        H.compare(out, want, ("constv", f))
    cache.close()


# ------------------------------------------------------- full-size streams
def full_size(name, num_blocks=None, attn_blocks=(0, 11, 23), pool_blocks=(0, 23),
              frames=None, milestone_keys=None, flags=(1, 0), in_run=False):
    """The workload's whole stream on the GPU, with the oracle checking every
    plan and state bit-exact, and at milestone frames the attention of
    sampled rows (all heads) and the bytes of the visible pages."""
    need_gpu()
    wl = synth.WORKLOADS[name]
    if num_blocks is not None:
        wl = wl.with_(num_blocks=num_blocks)
    nb = wl.num_blocks
    attn_blocks = [b for b in attn_blocks if b < nb]
    pool_blocks = [b for b in pool_blocks if b < nb]
    kinds, plans, writers_at, ms = H.dry_run(wl, frames, flags=flags)
    milestones = sorted(set(ms.values()))
    need = H.needed_frames(wl, plans, writers_at, milestones)
    log(f"{name}: {len(kinds)} frames, {nb} blocks, milestones {ms}")
    cfg = OracleConfig(**wl.cfg_kwargs())
    tracked = sorted(set(attn_blocks) | set(pool_blocks))
    o = PagePoolOracle(cfg, track_pool=tracked)
    cache = new_cache(wl)
    sm = wl.head_dim ** -0.5
    ns = wl.num_special_tokens
    rows = H.sample_rows(wl.tokens_per_frame)
    assert len(rows) > 20
    outs = [torch.empty((wl.tokens_per_frame, wl.num_heads, wl.head_dim),
                        dtype=torch.bfloat16, device=DEV) for _ in range(nb)]
    checked = 0
    for f, (kind, reset) in enumerate(kinds):
        qkv = H.gen_frame(wl, f, nb, DEV)

        def kv_of(b):
            if b not in tracked:
                return None, None
            k, v = qkv[b][1], qkv[b][2]
            if f in need:
                return synth.bf16_bits(k), synth.bf16_bits(v)
            kb = np.zeros((wl.tokens_per_frame, wl.num_heads, wl.head_dim), np.uint16)
            vb = kb.copy()
            kb[:ns] = synth.bf16_bits(k[:ns])
            vb[:ns] = synth.bf16_bits(v[:ns])
            return kb, vb

        refs = {}
        snap = {}
        # oracle side, capturing the attention references before rollback
        S, W = wl.scale_frames, wl.sliding_window
        if reset:
            o.reset()
        if wl.dynamic or kind == "transient":
            o.set_defer_eviction(True)
        for b in range(nb):
            k, v = kv_of(b)
            o.append_frame(b, k, v)
            o.evict_frames(b, S, W, *flags)
            if b == 0:
                o.plan()
            pl = o.check_run(b)
            if f in milestones and b in attn_blocks:
                refs[b] = paged_attention(o.pools[b], pl, cfg,
                                          synth.bf16_bits(qkv[b][0]), sm, rows=rows)
            if f in milestones and b in pool_blocks:
                sp = pl.table[pl.n_patch:]
                vis = pl.table[:pl.n_patch]
                snap[b] = (vis, sp, o.pools[b][vis].copy(), o.pools[b][sp].copy())
        plan_ref = (list(o.plan_state.table), o.plan_state.n_patch,
                    o.plan_state.last_page_len)
        for b in range(nb):
            if kind in ("transient", "reject"):
                o.rollback_last_frame(b)
            elif kind == "accept":
                o.execute_deferred_eviction(b, S, W)
        if kind == "transient":
            o.set_defer_eviction(False)

        specials_ref = special_runs(o.plan_state.spec_vis)
        # HIP side
        H.gpu_step(cache, wl, kind, reset, qkv, outs, flags=flags, in_run=in_run)
        assert cache.get_plan() == plan_ref, f
        assert cache.get_plan_specials() == specials_ref, f
        if f in milestones:
            torch.cuda.synchronize()
            for b in range(nb):
                assert list(o.block_state(b)) == list(cache.get_block_state(b)), (f, b)
                assert tuple(o.get_cache_stats(b)) == cache.get_cache_stats(b), (f, b)
            for b, (vis, sp, pv, ps) in snap.items():
                gp = cache.pools[b]
                assert np.array_equal(synth.bf16_bits(gp[vis]), pv), (f, b)
                assert np.array_equal(synth.bf16_bits(gp[sp]), ps), (f, b)
            for b, ref in refs.items():
                got = outs[b][rows]
                mx, mean, rel = H.compare(got, ref, (name, f, b))
                checked += 1
            log(f"  frame {f} ({kind}) checked: {len(plans[f][0])} pages visible")
    cache.close()
    assert checked >= len(milestones)


def test_full_224x224_stream():
    full_size("224x224")


def test_full_518x378_exact_stream():
    full_size("518x378")


def test_full_518x378_padded_long_stream():
    # 4096 frames (2048 keyframes) on all 24 blocks
    full_size("518x378-padded")


def test_full_dynamic_stream():
    full_size("dynamic")


def test_full_518x378_stream_appends_folded_into_runs():
    """The 518x378 stream with every frame admitted by append_frame_in_run:
    each block's run copies the frame into its pages and reads its tokens
    from the caller's buffers (transient frames too, before their rollback);
    plans every frame, attention and the visible pages' bytes at milestones;
    four blocks."""
    full_size("518x378", num_blocks=4, attn_blocks=(0, 3), pool_blocks=(0, 3), in_run=True)


def test_full_518x378_stream_camera_tokens_only():
    """The 518x378 stream with camera_only: from the first eviction on, each
    evicted frame leaves its camera token in view; four blocks."""
    full_size("518x378", num_blocks=4, attn_blocks=(0, 3), pool_blocks=(0, 3),
              flags=(1, 1))


def test_full_dynamic_stream_without_cross_frame_specials():
    """The dynamic stream with cross_frame_special = 0: accepted frames'
    deferred evictions drop the evicted frames' specials; four blocks."""
    full_size("dynamic", num_blocks=4, attn_blocks=(0, 3), pool_blocks=(0, 3),
              flags=(0, 0))


# ------------------------------------------------- run_own (skip append)
def own_parity(wl, check_frames=None, rows=None, splits=0, flags=(1, 0)):
    """A stream where keyframes are appended and every non-keyframe attends
    through run_own over the committed cache plus its own K/V, with no
    append.  Checked at the chosen non-keyframes: attention against the
    oracle's definition, and the pool bytes and the allocator state unchanged
    by run_own."""
    need_gpu()
    from oracle.attention import paged_attention_with_own
    cache = new_cache(wl)
    if splits:
        cache.set_num_splits(splits)
    cfg = OracleConfig(**wl.cfg_kwargs())
    o = PagePoolOracle(cfg, track_pool=[0])
    S, W = wl.scale_frames, wl.sliding_window
    sm = wl.head_dim ** -0.5
    checked = 0
    for f in range(wl.frames):
        q, k, v = synth.frame_qkv(wl, f, 0, device=DEV)
        if synth.is_keyframe(wl, f):
            cache.append_frame(0, k, v)
            cache.evict_frames(0, S, W, *flags)
            cache.plan()
            cache.run(0, q)
            o.append_frame(0, synth.bf16_bits(k), synth.bf16_bits(v))
            o.evict_frames(0, S, W, *flags)
            o.plan()
            continue
        if check_frames is not None and f not in check_frames:
            continue
        cache.plan()                     # the committed cache, as the last keyframe left it
        pl = o.plan()
        before = cache.pools[0].clone()
        state = cache.get_block_state(0), cache.get_cache_stats(0)
        out = cache.run_own(0, q, k, v)
        torch.cuda.synchronize()
        ref = paged_attention_with_own(o.pools[0], pl, cfg, synth.bf16_bits(q),
                                       synth.bf16_bits(k), synth.bf16_bits(v), sm, rows=rows)
        got = out if rows is None else out[rows]
        H.compare(got, ref, ("run_own", wl.name, f))
        assert torch.equal(cache.pools[0], before), f
        assert (cache.get_block_state(0), cache.get_cache_stats(0)) == state, f
        checked += 1
        log(f"  run_own frame {f}: {pl.num_visible_tokens(cfg)} cached + "
            f"{wl.tokens_per_frame} own tokens")
    cache.close()
    assert checked > 0


@pytest.mark.parametrize("flags", [(1, 1), (0, 0)])
def test_run_own_with_eviction_flags(flags):
    """run_own's row map (plan tokens, then the caller's own rows) when the
    plan's special runs skip evicted frames' specials."""
    log(f"run_own, mid stream, flags {flags}")
    own_parity(MID.with_(num_blocks=1, frames=40), splits=3, flags=flags)


@pytest.mark.parametrize("splits", [0, 1, 5])
def test_run_own_mid_stream(splits):
    """203-token pages, interval 2: every non-keyframe through run_own."""
    log(f"run_own, mid stream, splits={splits}")
    own_parity(MID.with_(num_blocks=1, frames=24), splits=splits)


def test_run_own_tiny_stream_first_frames():
    """The first non-keyframe sees a single committed frame; 16-token pages."""
    wl = synth.WORKLOADS["tiny"].with_(keyframe_interval=3, frames=14)
    log("run_own, tiny stream")
    own_parity(wl)


def test_run_own_518x378_steady_state():
    """The 518x378 stream on one block up to a full window (72 keyframes),
    run_own at the first non-keyframes and at steady state, sampled rows."""
    wl = synth.WORKLOADS["518x378"].with_(num_blocks=1, frames=170)
    log("run_own, 518x378 one block")
    own_parity(wl, check_frames={1, 3, 17, 145, 159, 169},
               rows=H.sample_rows(wl.tokens_per_frame))


def test_run_own_pool_offsets_up_to_2gib():
    """run_own on a pool of exactly 2 GiB (the largest it takes: its row map
    marks the caller's rows with the top bit of the 32-bit offsets): 2046
    patch pages and 2 special pages of 1 MiB; from the 43rd keyframe on the
    cache's special rows sit in the last MiB below 2^31, next to the caller's
    marked rows in the same row map."""
    wl = synth.Workload("pool-2GiB", 1, 16, 64, 256, 256, 6, 2, 2042, 2, 84, 88,
                        keyframe_interval=2, seed=32)
    import streaming_paged_kv_amd as spkv
    assert spkv.query_sizes(**wl.cfg_kwargs())[1] == 1 << 31
    log("run_own, 2 GiB pool")
    own_parity(wl, check_frames={1, 3, 85, 87})


def test_run_own_rejects_overlap_and_missing_buffers():
    need_gpu()
    import streaming_paged_kv_amd as spkv
    wl = MID.with_(num_blocks=1, frames=2)
    cache = new_cache(wl)
    q, k, v = synth.frame_qkv(wl, 0, 0, device=DEV)
    cache.append_frame(0, k, v)
    cache.plan()
    with pytest.raises(spkv.SpkvError) as ei:
        cache.run_own(0, q, k, v, out=k)           # out overlaps own K
    assert ei.value.name == "INVALID_ARG"
    lib = cache.lib
    import ctypes
    rc = lib.spkv_run_own(cache._h, 0, ctypes.c_void_p(q.data_ptr()),
                          ctypes.c_void_p(torch.empty_like(q).data_ptr()), q.shape[0],
                          0.125, None, ctypes.c_void_p(v.data_ptr()), None)
    assert rc == -1
    torch.cuda.synchronize()
    cache.close()


# ---------------------------------------------------- batch mode (phase 1)
def batch_mode_parity(wl, n_frames, rows=None):
    """The batch mode of the first frames: their K/V appended to every block,
    one plan, then one run per block with all their queries at once.  The
    reference is dense bidirectional attention over the frames' tokens
    concatenated, with no pages involved."""
    need_gpu()
    from oracle import bf16_bits_to_f64, dense_attention
    cache = new_cache(wl)
    S, W = wl.scale_frames, wl.sliding_window
    sm = wl.head_dim ** -0.5
    frames = {b: [synth.frame_qkv(wl, f, b, device=DEV) for f in range(n_frames)]
              for b in range(wl.num_blocks)}
    for b in range(wl.num_blocks):
        for q, k, v in frames[b]:
            cache.append_frame(b, k, v)
            cache.evict_frames(b, S, W)
        if b == 0:
            cache.plan()
    for b in range(wl.num_blocks):
        q_all = torch.cat([x[0] for x in frames[b]]).contiguous()
        out = cache.run(b, q_all)
        torch.cuda.synchronize()
        k_all = bf16_bits_to_f64(synth.bf16_bits(torch.cat([x[1] for x in frames[b]])))
        v_all = bf16_bits_to_f64(synth.bf16_bits(torch.cat([x[2] for x in frames[b]])))
        q64 = bf16_bits_to_f64(synth.bf16_bits(q_all))
        if rows is not None:
            q64 = q64[rows]
        ref = dense_attention(q64, k_all, v_all, sm)
        H.compare(out if rows is None else out[rows], ref, ("batch", wl.name, b))
        log(f"  batch mode block {b}: {q_all.shape[0]} queries over {k_all.shape[0]} keys")
    cache.close()


def test_batch_mode_tiny_and_mid():
    batch_mode_parity(synth.WORKLOADS["tiny"], 2)
    batch_mode_parity(MID.with_(frames=2), 2)


def test_batch_mode_518x378_scale_frames():
    """Eight 1005-token frames at once: 8040 queries over 8040 keys."""
    wl = synth.WORKLOADS["518x378"].with_(num_blocks=2)
    rows = sorted(set(H.sample_rows(8 * wl.tokens_per_frame, extra=40)))
    batch_mode_parity(wl, 8, rows=rows)


# ------------------------------------------------------ random schedules
@pytest.mark.parametrize("seed,variants", [(101, False), (102, False), (103, False),
                                           (301, True), (302, True), (303, True)])
def test_random_schedules_every_frame(seed, variants):
    """Seeded random mixes of keyframes, transient (append + rollback)
    non-keyframes, run_own non-keyframes, deferred accept / reject and resets
    on a 2-block stream with 16-token pages: after every frame the whole pool,
    the plan (with its visible special runs), the stats and the allocator
    state are bit-exact, and every attention output matches the oracle.  With
    variants, each frame also draws its eviction flags and whether its
    appends are folded into the runs (append_frame_in_run)."""
    need_gpu()
    from oracle.attention import paged_attention_with_own
    rng = np.random.default_rng(seed)
    wl = synth.WORKLOADS["tiny"].with_(num_blocks=2, frames=40, seed=seed)
    cfg = OracleConfig(**wl.cfg_kwargs())
    o = PagePoolOracle(cfg, track_pool=range(wl.num_blocks))
    cache = new_cache(wl)
    cache.set_num_splits(int(rng.integers(0, 4)))
    S, W = wl.scale_frames, wl.sliding_window
    sm = wl.head_dim ** -0.5
    nb = wl.num_blocks
    committed = 0
    for f in range(wl.frames):
        ev = rng.choice(["key", "key", "transient", "own", "accept", "reject", "reset"])
        flags = (1, 0)
        in_run = False
        if variants:
            flags = [(1, 0), (1, 1), (0, 0), (0, 1)][int(rng.integers(0, 4))]
            in_run = bool(rng.integers(0, 2))
        if ev == "reset" or committed >= 30:       # 32 special slots: stay clear of overflow
            cache.reset()
            o.reset()
            committed = 0
            if ev == "reset":
                continue
            ev = "key"
        if committed == 0 and ev == "own":
            ev = "key"                             # run_own needs a committed cache
        qkv = H.gen_frame(wl, f, nb, DEV)
        bits = [[synth.bf16_bits(t) for t in x] for x in qkv]
        if ev == "own":
            cache.plan()
            pl = o.plan()
            for b in range(nb):
                out = cache.run_own(b, *qkv[b])
                ref = paged_attention_with_own(o.pools[b], pl, cfg, *bits[b], sm)
                torch.cuda.synchronize()
                H.compare(out, ref, ("random", seed, f, ev, b))
        else:
            defer = ev != "key"
            if defer:
                cache.set_defer_eviction(True)
                o.set_defer_eviction(True)
            for b in range(nb):
                if in_run:
                    cache.append_frame_in_run(b, qkv[b][1], qkv[b][2])
                else:
                    cache.append_frame(b, qkv[b][1], qkv[b][2])
                o.append_frame(b, bits[b][1], bits[b][2])
                cache.evict_frames(b, S, W, *flags)
                o.evict_frames(b, S, W, *flags)
                if b == 0:
                    cache.plan()
                    o.plan()
                    assert cache.get_plan_specials() == special_runs(o.plan_state.spec_vis)
                out = cache.run(b, qkv[b][0])
                ref = paged_attention(o.pools[b], o.check_run(b), cfg, bits[b][0], sm)
                torch.cuda.synchronize()
                H.compare(out, ref, ("random", seed, f, ev, b))
            for b in range(nb):
                if ev in ("transient", "reject"):
                    cache.rollback_last_frame(b)
                    o.rollback_last_frame(b)
                elif ev == "accept":
                    cache.execute_deferred_eviction(b, S, W)
                    o.execute_deferred_eviction(b, S, W)
            if defer:
                cache.set_defer_eviction(False)
                o.set_defer_eviction(False)
            committed += ev in ("key", "accept")
        torch.cuda.synchronize()
        for b in range(nb):
            assert list(o.block_state(b)) == list(cache.get_block_state(b)), (seed, f, b)
            assert tuple(o.get_cache_stats(b)) == cache.get_cache_stats(b), (seed, f, b)
            assert o.special_visibility(b) == cache.get_block_specials(b), (seed, f, b)
            assert np.array_equal(synth.bf16_bits(cache.pools[b]), o.pools[b]), (seed, f, b)
    cache.close()


# ------------------------------------------------- several streams per launch
def batch_streams_parity(wls, frames, splits=None, rows=None):
    """Streams of different shapes advanced together; every frame, one
    run_batch call runs block 0 of every stream: a run() request on a
    keyframe (appended, evicted, planned) and a run_own() request on a
    non-keyframe (the committed cache plus the frame's own K/V).  Each output
    is checked against the oracle's definition of that request."""
    need_gpu()
    import streaming_paged_kv_amd as spkv
    from oracle.attention import paged_attention_with_own
    caches = [new_cache(w) for w in wls]
    for c, sp in zip(caches, splits or [0] * len(wls)):
        if sp:
            c.set_num_splits(sp)
    cfgs = [OracleConfig(**w.cfg_kwargs()) for w in wls]
    oracles = [PagePoolOracle(cfg, track_pool=[0]) for cfg in cfgs]
    bits = synth.bf16_bits
    for f in range(frames):
        reqs, refs = [], []
        for w, c, o, cfg in zip(wls, caches, oracles, cfgs):
            q, k, v = synth.frame_qkv(w, f, 0, device=DEV)
            S, W = w.scale_frames, w.sliding_window
            sm = w.head_dim ** -0.5
            if synth.is_keyframe(w, f):
                c.append_frame(0, k, v)
                c.evict_frames(0, S, W)
                c.plan()
                o.append_frame(0, bits(k), bits(v))
                o.evict_frames(0, S, W)
                pl = o.plan()
                reqs.append(dict(cache=c, block=0, q=q))
                refs.append(paged_attention(o.pools[0], pl, cfg, bits(q), sm, rows=rows))
            else:
                c.plan()
                pl = o.plan()
                reqs.append(dict(cache=c, block=0, q=q, k=k, v=v))
                refs.append(paged_attention_with_own(o.pools[0], pl, cfg, bits(q), bits(k),
                                                     bits(v), sm, rows=rows))
        outs = spkv.run_batch(reqs)
        torch.cuda.synchronize()
        for i, (out, ref) in enumerate(zip(outs, refs)):
            H.compare(out if rows is None else out[rows], ref, ("batch", wls[i].name, f))
    for c in caches:
        c.close()


def test_run_batch_streams_of_different_shapes():
    """Three streams in one launch: 4 heads x 16-token pages (22 queries),
    16 heads x 203-token pages (206 queries), 16 heads x 999-token pages
    (1005 queries, two query tiles); keyframe intervals 3, 2, 2, so the
    batches mix run() and run_own() requests."""
    tiny = synth.WORKLOADS["tiny"].with_(keyframe_interval=3, seed=31)
    mid = MID.with_(num_blocks=1, seed=32)
    big = BIGQ.with_(seed=33)
    log("run_batch: tiny + mid + 1005-query streams, 9 frames")
    batch_streams_parity([tiny, mid, big], 9)


def test_run_batch_sixteen_streams_and_forced_splits():
    """The largest batch (16 tiny streams: one work item each, no merge), then
    mid streams with forced split counts 1, 3 and 7 in one batch (one merge
    launch over requests with different split counts)."""
    tiny = synth.WORKLOADS["tiny"]
    wls = [tiny.with_(name=f"tiny{i}", seed=40 + i, keyframe_interval=1 + i % 3)
           for i in range(16)]
    log("run_batch: 16 tiny streams, 7 frames")
    batch_streams_parity(wls, 7)
    mids = [MID.with_(name=f"mid{i}", num_blocks=1, seed=60 + i) for i in range(3)]
    log("run_batch: mid streams with splits 1/3/7, 10 frames")
    batch_streams_parity(mids, 10, splits=[1, 3, 7])


def test_run_batch_rejects_overlapping_requests():
    """A request whose out overlaps another request's q is refused before
    anything is enqueued: both outputs keep their sentinel bytes."""
    need_gpu()
    import streaming_paged_kv_amd as spkv
    wl = synth.WORKLOADS["tiny"]
    a, b = new_cache(wl.with_(num_blocks=1)), new_cache(wl.with_(num_blocks=1))
    for c in (a, b):
        q, k, v = synth.frame_qkv(wl, 0, 0, device=DEV)
        c.append_frame(0, k, v)
        c.evict_frames(0, wl.scale_frames, wl.sliding_window)
        c.plan()
    qa = synth.frame_qkv(wl, 1, 0, device=DEV, which=(synth.TENSOR_Q,))[0]
    oa = torch.full_like(qa, 7.0)
    shared = torch.full_like(qa, 7.0)          # b's out is a's q
    with pytest.raises(spkv.SpkvError) as e:
        spkv.run_batch([dict(cache=a, block=0, q=shared, out=oa),
                        dict(cache=b, block=0, q=qa, out=shared)])
    assert e.value.name == "INVALID_ARG"
    torch.cuda.synchronize()
    assert bool((oa == 7.0).all()) and bool((shared == 7.0).all())
    # the same two requests with separate buffers run
    spkv.run_batch([dict(cache=a, block=0, q=qa, out=oa),
                    dict(cache=b, block=0, q=qa.clone())])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(oa.float()).all())
    a.close()
    b.close()


@pytest.mark.parametrize("seed", [201, 202])
def test_run_batch_random_schedules(seed):
    """Three streams of different geometry and eviction flags (all specials,
    camera tokens only, none of an evicted frame), each with its own seeded
    random mix of keyframes, transient non-keyframes, run_own non-keyframes,
    deferred accept / reject and resets; per frame and block one run_batch
    covers the three streams.  After every frame each stream's whole pool,
    stats and allocator state are bit-exact and every output matches the
    oracle."""
    need_gpu()
    import streaming_paged_kv_amd as spkv
    from oracle.attention import paged_attention_with_own
    rng = np.random.default_rng(seed)
    wls = [synth.WORKLOADS["tiny"].with_(num_blocks=2, frames=30, seed=seed),
           synth.Workload("odd", 2, 2, 64, 13, 11, 4, 1, 3, 1, 40, 30, seed=seed + 1),
           MID.with_(name="mid2", frames=30, seed=seed + 2)]
    nb = 2
    flags = [(1, 0), (1, 1), (0, 0)]
    cfgs = [OracleConfig(**w.cfg_kwargs()) for w in wls]
    oracles = [PagePoolOracle(cfg, track_pool=range(nb)) for cfg in cfgs]
    caches = [new_cache(w) for w in wls]
    for c in caches:
        c.set_num_splits(int(rng.integers(0, 4)))
    committed = [0] * len(wls)
    limits = [30, 36, 60]                  # stay clear of special-slot overflow
    for f in range(30):
        evs = []
        for i, (c, o) in enumerate(zip(caches, oracles)):
            ev = str(rng.choice(["key", "key", "transient", "own", "accept", "reject", "reset"]))
            if ev == "reset" or committed[i] >= limits[i]:
                c.reset()
                o.reset()
                committed[i] = 0
                ev = "key"
            if committed[i] == 0 and ev == "own":
                ev = "key"
            evs.append(ev)
        qkvs = [H.gen_frame(w, f, nb, DEV) for w in wls]
        bits = [[[synth.bf16_bits(t) for t in x] for x in qkv] for qkv in qkvs]
        for i, ev in enumerate(evs):
            if ev in ("transient", "accept", "reject"):
                caches[i].set_defer_eviction(True)
                oracles[i].set_defer_eviction(True)
        for b in range(nb):
            reqs, refs = [], []
            for i, (w, c, o, cfg, ev) in enumerate(zip(wls, caches, oracles, cfgs, evs)):
                q, k, v = qkvs[i][b]
                qb, kb, vb = bits[i][b]
                S, W = w.scale_frames, w.sliding_window
                sm = w.head_dim ** -0.5
                if ev == "own":
                    if b == 0:
                        c.plan()
                        o.plan()
                    reqs.append(dict(cache=c, block=b, q=q, k=k, v=v))
                    refs.append(paged_attention_with_own(o.pools[b], o.check_run(b), cfg,
                                                         qb, kb, vb, sm))
                else:
                    c.append_frame(b, k, v)
                    o.append_frame(b, kb, vb)
                    c.evict_frames(b, S, W, *flags[i])
                    o.evict_frames(b, S, W, *flags[i])
                    if b == 0:
                        c.plan()
                        o.plan()
                    reqs.append(dict(cache=c, block=b, q=q))
                    refs.append(paged_attention(o.pools[b], o.check_run(b), cfg, qb, sm))
            outs = spkv.run_batch(reqs)
            torch.cuda.synchronize()
            for i, (out, ref) in enumerate(zip(outs, refs)):
                H.compare(out, ref, ("batch random", seed, f, wls[i].name, evs[i], b))
        for i, (w, c, o, ev) in enumerate(zip(wls, caches, oracles, evs)):
            for b in range(nb):
                if ev in ("transient", "reject"):
                    c.rollback_last_frame(b)
                    o.rollback_last_frame(b)
                elif ev == "accept":
                    c.execute_deferred_eviction(b, w.scale_frames, w.sliding_window)
                    o.execute_deferred_eviction(b, w.scale_frames, w.sliding_window)
            if ev in ("transient", "accept", "reject"):
                c.set_defer_eviction(False)
                o.set_defer_eviction(False)
            committed[i] += ev in ("key", "accept")
        torch.cuda.synchronize()
        for i, (c, o) in enumerate(zip(caches, oracles)):
            for b in range(nb):
                assert list(o.block_state(b)) == list(c.get_block_state(b)), (seed, f, i, b)
                assert tuple(o.get_cache_stats(b)) == c.get_cache_stats(b), (seed, f, i, b)
                assert np.array_equal(synth.bf16_bits(c.pools[b]), o.pools[b]), (seed, f, i, b)
    for c in caches:
        c.close()


def test_two_handles_on_concurrent_streams():
    """Two handles, each on its own HIP stream (default priority), with their
    frame steps interleaved and no synchronisation between the streams:
    every output equals, bit for bit, the same frames run one handle after
    the other on one stream.  Handles share nothing on the device (own pools
    and workspaces) or on the host (own staging)."""
    need_gpu()
    wls = [MID.with_(name="conc-a", num_blocks=2, frames=10, seed=51),
           BIGQ.with_(name="conc-b", frames=6, seed=52)]
    inputs = [[H.gen_frame(wl, f, wl.num_blocks, DEV) for f in range(wl.frames)] for wl in wls]

    def drive(cache, wl, f, outs, stream):
        for b in range(wl.num_blocks):
            q, k, v = inputs[wls.index(wl)][f][b]
            cache.append_frame(b, k, v, stream=stream)
            cache.evict_frames(b, wl.scale_frames, wl.sliding_window)
            if b == 0:
                cache.plan(stream=stream)
            cache.run(b, q, out=outs[b], stream=stream)

    # concurrent: frame steps alternate between the two streams
    caches = [new_cache(wl) for wl in wls]
    got = [[[torch.empty_like(x[0]) for x in inputs[i][f]] for f in range(wl.frames)]
           for i, wl in enumerate(wls)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:              # pools zeroed and inputs drawn on this stream
        s.wait_stream(torch.cuda.current_stream())
    for f in range(max(wl.frames for wl in wls)):
        for i, wl in enumerate(wls):
            if f < wl.frames:
                drive(caches[i], wl, f, got[i][f], streams[i])
    torch.cuda.synchronize()
    for c in caches:
        c.close()

    # reference: one handle after the other on the default stream
    for i, wl in enumerate(wls):
        cache = new_cache(wl)
        for f in range(wl.frames):
            outs = [torch.empty_like(x[0]) for x in inputs[i][f]]
            drive(cache, wl, f, outs, None)
            torch.cuda.synchronize()
            for b in range(wl.num_blocks):
                assert torch.equal(outs[b], got[i][f][b]), (wl.name, f, b)
        cache.close()


def test_run_captured_in_a_hip_graph():
    """run() enqueues kernels only (attention, and the merge when the key
    range is split): captured into a HIP graph after a plan, every replay
    equals the eager result bit for bit, with eager work and
    synchronisation between replays.  plan() is not capturable: it reads
    the host allocator's state of the moment."""
    need_gpu()
    wl = BIGQ.with_(name="graph", frames=4, seed=61)
    cache = new_cache(wl)
    frames = [H.gen_frame(wl, f, 1, DEV)[0] for f in range(wl.frames)]
    for f, (q, k, v) in enumerate(frames):
        cache.append_frame(0, k, v)
        cache.evict_frames(0, wl.scale_frames, wl.sliding_window)
        cache.plan()
        if f < wl.frames - 1:
            cache.run(0, q)
    q = frames[-1][0]
    for splits in (0, 1):
        cache.set_num_splits(splits)
        ref = cache.run(0, q)
        torch.cuda.synchronize()
        out = torch.empty_like(q)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            cache.run(0, q, out=out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cache.run(0, q, out=out)
        for i in range(4):
            out.fill_(0)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), (splits, i)
            # eager work of the program between replays
            junk = torch.randn(1 << 20, device=DEV)
            assert torch.isfinite(junk.sum())
            torch.cuda.synchronize()
        del g
    cache.close()


def test_run_own_and_run_batch_captured_in_a_hip_graph():
    """run_own() and run_batch() enqueue kernels only as well: captured after
    the streams' plans, their replays equal the eager results bit for bit,
    with eager work and synchronisation between replays."""
    need_gpu()
    import streaming_paged_kv_amd as spkv
    wls = [BIGQ.with_(name="graph-a", frames=5, seed=62),
           MID.with_(name="graph-b", num_blocks=1, frames=5, seed=63)]
    caches = [new_cache(wl) for wl in wls]
    last = []
    for wl, cache in zip(wls, caches):
        frames = [H.gen_frame(wl, f, 1, DEV)[0] for f in range(wl.frames)]
        for q, k, v in frames[:-1]:
            cache.append_frame(0, k, v)
            cache.evict_frames(0, wl.scale_frames, wl.sliding_window)
            cache.plan()
        last.append(frames[-1])

    def requests(outs):
        (qa, ka, va), (qb, _, _) = last
        return [dict(cache=caches[0], block=0, q=qa, k=ka, v=va, out=outs[0]),
                dict(cache=caches[1], block=0, q=qb, out=outs[1])]

    cases = {
        "run_own": lambda outs: caches[0].run_own(0, last[0][0], last[0][1], last[0][2],
                                                  out=outs[0]),
        "run_batch": lambda outs: spkv.run_batch(requests(outs)),
    }
    for name, call in cases.items():
        ref = [torch.empty_like(last[0][0]), torch.empty_like(last[1][0])]
        call(ref)
        torch.cuda.synchronize()
        outs = [torch.empty_like(x) for x in ref]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(outs)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(outs)
        n_out = 1 if name == "run_own" else 2
        for i in range(3):
            for o in outs:
                o.fill_(0)
            g.replay()
            torch.cuda.synchronize()
            for j in range(n_out):
                assert torch.equal(outs[j], ref[j]), (name, i, j)
            junk = torch.randn(1 << 20, device=DEV)
            assert torch.isfinite(junk.sum())
            torch.cuda.synchronize()
        del g
    for c in caches:
        c.close()


def test_run_folding_a_copy_captured_in_a_hip_graph():
    """A run that folds the copy of a frame admitted by append_frame_in_run,
    captured into a HIP graph: the copy belongs to the captured attention
    launch, so it happens at every replay and not at capture.  After each
    replay the whole pool equals the oracle's (which copies at admission)
    and the output equals, bit for bit, the same run done eagerly on a twin
    cache that admitted the frame with append_frame (same bytes, same order,
    same split); eager work and synchronisation between replays."""
    need_gpu()
    wl = MID.with_(name="graph-fold", num_blocks=1, frames=9, keyframe_interval=1, seed=67)
    cfg = OracleConfig(**wl.cfg_kwargs())
    o = PagePoolOracle(cfg, track_pool=[0])
    fold, twin = new_cache(wl), new_cache(wl)
    S, W = wl.scale_frames, wl.sliding_window
    sm = wl.head_dim ** -0.5
    frames = [synth.frame_qkv(wl, f, 0, device=DEV) for f in range(wl.frames)]
    for f, (q, k, v) in enumerate(frames):
        fold.append_frame_in_run(0, k, v)
        twin.append_frame(0, k, v)
        o.append_frame(0, synth.bf16_bits(k), synth.bf16_bits(v))
        for c in (fold, twin):
            c.evict_frames(0, S, W)
            c.plan()
        o.evict_frames(0, S, W)
        pl = o.plan()
        if f < wl.frames - 1:
            fold.run(0, q, sm_scale=sm)     # folds frame f's copy, eagerly
            twin.run(0, q, sm_scale=sm)
    q = frames[-1][0]
    ref = twin.run(0, q, sm_scale=sm)
    torch.cuda.synchronize()
    H.compare(ref, paged_attention(o.pools[0], pl, cfg, synth.bf16_bits(q), sm), "twin")
    out = torch.empty_like(q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fold.run(0, q, out=out, sm_scale=sm)
    torch.cuda.synchronize()
    # the frame's page (never written before) still differs: nothing copied yet
    assert not np.array_equal(synth.bf16_bits(fold.pools[0]), o.pools[0])
    for i in range(3):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), i
        assert np.array_equal(synth.bf16_bits(fold.pools[0]), o.pools[0]), i
        junk = torch.randn(1 << 20, device=DEV)
        assert torch.isfinite(junk.sum())
        torch.cuda.synchronize()
    del g
    fold.close()
    twin.close()
