"""Benchmark: streamed frames/s of the 24-block paged-attention hot path.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 518x378]

A step is one frame of the stream through the whole hot path: for a keyframe,
on each of the 24 blocks, append the frame's K/V to the block's pages, evict,
plan (block 0) and run the paged attention; a non-keyframe attends to the
cache plus its own K/V on each block without appending them (run_own).  The
dynamic workload appends every frame under deferred eviction and then
accepts or rolls it back.  Before anything is timed, the stream runs untimed
until its scale pages and its live window are full (143 frames for the
518x378 stream: 8 + 64 keyframes at interval 2), whatever W is, and then W
more untimed frames; the K timed frames therefore run at steady state.
Inputs (Q, K, V of every block for a bank of frames, synthetic N(0,1) bf16)
are resident in HBM before the timed region.

Alongside the throughput it reports the roofline of the attention kernel (its
algorithmic bf16 flops over its duration measured with HIP events on the
stream it runs on), the append kernel's bandwidth, and the CPU oracle timed on
a bounded sample of the same workload on the host cores.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "streamed frames/s (24-block paged attn, 999-token pages); % bf16 MFMA peak"
ATTN_SRC = os.path.join(ROOT, "streaming_paged_kv_amd", "csrc", "attn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kernel-518x378-traffic.txt")
COPY_BYTES = 256 << 20        # plain copy used to calibrate the byte counters
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=16,
                    help="untimed frames after the ones that fill the scale pages "
                         "and the live window")
    ap.add_argument("--workload", default="518x378")
    ap.add_argument("--bank", type=int, default=16, help="distinct input frames")
    ap.add_argument("--append", choices=("in_run", "plain"), default="in_run",
                    help="in_run: keyframes are admitted with append_frame_in_run, so "
                         "each block's run copies the frame inside the attention "
                         "launch; plain: append_frame launches its own copy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-blocks", type=int, default=2,
                    help="blocks of the oracle frame timed (scaled to all)")
    ap.add_argument("--no-full-stream", action="store_true",
                    help="skip the timed pass over the whole stream from an empty cache")
    ap.add_argument("--no-events", action="store_true",
                    help="time without per-kernel events (roofline omitted)")
    ap.add_argument("--append-sweep", action="store_true",
                    help="only measure the append kernel against frame size")
    ap.add_argument("--streams", type=int, default=1,
                    help="R > 1: R independent streams of the workload, whose "
                         "attention runs as one run_batch per block, timed against "
                         "the same streams with one run per stream and block")
    return ap.parse_args()


def frame_schedule(wl, n):
    import synth
    dec = synth.accept_decisions(wl, n) if wl.dynamic else None
    out = []
    for f in range(n):
        if wl.dynamic:
            out.append("accept" if dec[f] else "reject")
        else:
            out.append("key" if synth.is_keyframe(wl, f) else "transient")
    return out


def fill_frames(wl):
    """Frames after which the stream's scale pages and live window are full:
    the frame count at which S + W frames have been committed (keyframes;
    accepted frames of the dynamic stream)."""
    need = wl.scale_frames + wl.sliding_window
    sched = frame_schedule(wl, wl.frames)
    done = 0
    for f, kind in enumerate(sched):
        done += kind in ("key", "accept")
        if done >= need:
            return f + 1
    raise SystemExit(f"{wl.name}: the stream never fills its window")


def cpu_baseline(wl, warm_frames, n_blocks_timed):
    """The oracle, as it is, on the host cores: warm its state machine through
    the stream (untimed, block 0's pool fed seeded bits), then time one
    steady-state frame: append + evict + plan on every block and the dense
    float64 attention of n_blocks_timed blocks (each a full 1005-row query
    over block 0's gathered K/V), scaled to all blocks."""
    import numpy as np
    from oracle import OracleConfig, PagePoolOracle
    from oracle.attention import paged_attention

    cfg = OracleConfig(**wl.cfg_kwargs())
    o = PagePoolOracle(cfg, track_pool=[0])
    rng = np.random.default_rng(123)
    shape = (wl.tokens_per_frame, wl.num_heads, wl.head_dim)
    # a few distinct frames of bf16-pattern N(0,1)-like bits, reused
    frames = []
    for _ in range(4):
        x = rng.standard_normal((2,) + shape).astype(np.float32)
        frames.append((x.view(np.uint32) >> 16).astype(np.uint16))
    sched = frame_schedule(wl, warm_frames + 1)
    S, W = wl.scale_frames, wl.sliding_window

    def one_frame(f, kind, attend_blocks):
        kv = frames[f % 4]
        if o.get_cache_stats(0)[0] >= cfg.special_capacity_frames:
            o.reset()   # special stream full (short streams): start over
        if wl.dynamic or kind == "transient":
            o.set_defer_eviction(True)
        for b in range(wl.num_blocks):
            o.append_frame(b, kv[0] if b == 0 else None, kv[1] if b == 0 else None)
            o.evict_frames(b, S, W)
            if b == 0:
                o.plan()
            pl = o.check_run(b)
            if b < attend_blocks:
                q = frames[(f + b) % 4][0]
                paged_attention(o.pools[0], pl, cfg, q, wl.head_dim ** -0.5)
        for b in range(wl.num_blocks):
            if kind in ("transient", "reject"):
                o.rollback_last_frame(b)
            elif kind == "accept":
                o.execute_deferred_eviction(b, S, W)
        if kind == "transient":
            o.set_defer_eviction(False)

    for f in range(warm_frames):
        one_frame(f, sched[f], 0)
    f = warm_frames
    t0 = time.perf_counter()
    one_frame(f, "key", 0)          # the host steps of a frame, all blocks
    t_host = time.perf_counter() - t0
    t0 = time.perf_counter()
    pl = o.plan()
    for b in range(n_blocks_timed):
        q = frames[b % 4][0]
        paged_attention(o.pools[0], pl, cfg, q, wl.head_dim ** -0.5)
    t_attn = (time.perf_counter() - t0) / n_blocks_timed
    per_frame = t_host + t_attn * wl.num_blocks
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        blas = 1
    cores = len(os.sched_getaffinity(0))
    return {
        "value": 1.0 / per_frame,
        "unit": "frames/s",
        "cores": int(max(1, min(cores, blas))),
        "kind": "oracle",
        "sample": (f"one steady-state frame (frame {f}) of {wl.name}: page-pool "
                   f"steps on all {wl.num_blocks} blocks ({t_host*1e3:.1f} ms) + "
                   f"float64 dense attention of {n_blocks_timed} blocks, all "
                   f"{wl.tokens_per_frame} rows x {wl.num_heads} heads over "
                   f"{pl.num_visible_tokens(cfg)} visible tokens "
                   f"({t_attn:.2f} s per block), scaled to {wl.num_blocks} blocks; "
                   f"host cores {cores}, BLAS threads {blas}"),
    }


def append_sweep(reps=40):
    """Bandwidth of the append kernel against frame size: one block, H=16,
    D=64, P patch tokens per frame in P-token pages, P from 999 (the 518x378
    frame, 8.2 MB of K/V read + written per append) up to 256k tokens (2 GB).
    Pages and source frames rotate through about 1 GB each, so that neither
    side sits in the 256 MB last-level cache.  Prints one line per size with
    the event time per append (which includes the launch gap between
    back-to-back launches); the kernel's own duration comes from a kernel
    trace of this command."""
    import torch
    import streaming_paged_kv_amd as spkv

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    h, d, ns = 16, 64, 6
    for p in (999, 1999, 3999, 7999, 15999, 31999, 63999, 127999, 255999):
        page_bytes = 2 * p * h * d * 2
        live = max(1, min(254, (1 << 30) // page_bytes))
        frame_bytes = 2 * (p + ns) * h * d * 2
        nbank = max(2, min(256, (1 << 30) // frame_bytes))
        cfg = dict(num_blocks=1, num_heads=h, head_dim=d, page_size=p, patch_tokens=p,
                   num_special_tokens=ns, scale_frames=1, sliding_window=live, headroom=1,
                   max_total_frames=max(1, p // ns) * 4)
        min_ws = spkv.query_sizes(**cfg)[2]
        cache = spkv.PagedKVCache(**cfg, device=dev, workspace_bytes=min_ws)
        g = torch.Generator(device=dev).manual_seed(p)
        src = torch.randn((nbank, 2, p + ns, h, d), generator=g, device=dev).to(torch.bfloat16)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        nbytes = 4 * (p + ns) * h * d * 2
        nrep = max(reps, min(400, (2 << 30) // nbytes))   # touch >= 2 GB
        n = 0
        for r in range(nrep + 5):
            if cache.get_cache_stats(0)[0] >= max(1, p // ns) * 4:
                cache.reset()
            if r == 5:
                e0.record(stream)
            f = r % nbank
            cache.append_frame(0, src[f, 0], src[f, 1], stream=stream)
            cache.evict_frames(0, 1, live)
            n += r >= 5
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        print(f"append P={p:6d}: {nbytes:11d} bytes/append, {us:8.2f} us/append by events "
              f"(launch gaps included), {nbytes / us / 1e3:7.0f} GB/s", flush=True)
        cache.close()
        del src, cache
        torch.cuda.empty_cache()


def multi_stream(args, wl, R):
    """R independent streams of `wl` (each its own cache), advanced frame by
    frame; per block, every stream appends / evicts / plans as its schedule
    says, then the R attention requests run either as one run_batch launch or
    as R separate run() / run_own() calls.  Both modes are timed over the same
    frames (after the same warmup) and reported with the attention time per
    block from HIP events around the launches."""
    import torch
    import streaming_paged_kv_amd as spkv
    import synth

    if wl.dynamic or not 1 < R <= spkv.MAX_BATCH:
        raise SystemExit(f"--streams takes 2..{spkv.MAX_BATCH} on a fixed-schedule workload")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    nb, nq = wl.num_blocks, wl.tokens_per_frame
    S, W = wl.scale_frames, wl.sliding_window
    sm = wl.head_dim ** -0.5
    hd = wl.num_heads * wl.head_dim
    nbank = max(1, args.bank)
    bank = [[synth.frame_qkv(wl, f, b, device=dev) for b in range(nb)]
            for f in range(nbank)]
    res = {}
    for mode in ("batched", "separate"):
        caches = [spkv.PagedKVCache(**wl.cfg_kwargs(), device=dev) for _ in range(R)]
        outs = [[torch.empty((nq, wl.num_heads, wl.head_dim), dtype=torch.bfloat16,
                             device=dev) for _ in range(nb)] for _ in range(R)]
        warm = fill_frames(wl) + max(0, args.warmup)
        total = warm + 2 * args.steps
        sched = frame_schedule(wl, total)
        ev, flops = [], []

        def visible(c):
            tab, npatch, lpl = c.get_plan()
            return (npatch * wl.patch_tokens + (len(tab) - npatch - 1) *
                    wl.num_special_tokens * (wl.page_size // wl.num_special_tokens) + lpl)

        def step(f, events):
            key = sched[f] == "key"
            for b in range(nb):
                reqs = []
                for r, c in enumerate(caches):
                    q, k, v = bank[(f + r) % nbank][b]
                    if key:
                        c.append_frame(b, k, v, stream=stream)
                        c.evict_frames(b, S, W)
                        if b == 0:
                            c.plan(stream=stream)
                        reqs.append(dict(cache=c, block=b, q=q, out=outs[r][b], sm_scale=sm))
                    else:
                        reqs.append(dict(cache=c, block=b, q=q, k=k, v=v, out=outs[r][b],
                                         sm_scale=sm))
                batch = spkv.Batch(reqs) if mode == "batched" else None
                if events:
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                if mode == "batched":
                    batch.launch(stream=stream)
                else:
                    for rq in reqs:
                        c = rq["cache"]
                        if key:
                            c.run(b, rq["q"], out=rq["out"], sm_scale=sm, stream=stream)
                        else:
                            c.run_own(b, rq["q"], rq["k"], rq["v"], out=rq["out"],
                                      sm_scale=sm, stream=stream)
                if events:
                    e1.record(stream)
                    ev.append((e0, e1))
                    flops.append(sum(4.0 * nq * (visible(c) + (0 if key else nq)) * hd
                                     for c in caches))

        for f in range(warm):
            step(f, False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for f in range(warm, warm + args.steps):
            step(f, False)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        for f in range(warm + args.steps, total):
            step(f, True)
        torch.cuda.synchronize()
        t_attn = [a.elapsed_time(b) * 1e-3 for a, b in ev]
        achieved = sum(flops) / sum(t_attn) / 1e12
        res[mode] = {
            "frames_per_s": R * args.steps / dt,
            "ms_per_step": dt / args.steps * 1e3,
            "attention_us_per_block": sum(t_attn) / len(t_attn) * 1e6,
            "attention_tflops": achieved,
            "attention_frac_bf16_peak": achieved / PEAK_BF16_TFLOPS,
        }
        for c in caches:
            c.close()
        del caches, outs
        torch.cuda.empty_cache()
    print(json.dumps({
        "metric": f"streamed frames/s over {R} independent streams (all streams' frames)",
        "value": res["batched"]["frames_per_s"],
        "unit": "frames/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": res["batched"]["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{R} x {wl.name}: {nb} blocks, H={wl.num_heads}, "
                               f"page_size={wl.page_size}, {nq} tokens/frame, "
                               f"keyframe_interval={wl.keyframe_interval}; per block one "
                               f"run_batch over the {R} streams",
                   "frames_timed": f"{warm}..{warm + args.steps - 1}",
                   "input_bank_frames": nbank},
        "batched": res["batched"],
        "separate": res["separate"],
    }), flush=True)


def kernel_hash():
    import hashlib
    with open(ATTN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_traffic(workload, visible_tokens):
    """HBM bytes per attention launch from the committed counter summary, if
    it was taken on the current kernel source and this workload, at a number
    of visible tokens within 5% of this window's (the launch's bytes grow
    with them)."""
    try:
        kv = {}
        for line in open(TRAFFIC_FILE):
            if ":" in line and not line.startswith(("#", "|")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256_16") != kernel_hash():
            return None
        if kv.get("workload") != workload:
            return None
        nk = float(kv["visible_tokens"])
        if abs(nk - visible_tokens) > 0.05 * nk:
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    if args.append_sweep:
        append_sweep()
        return
    if args.streams > 1:
        import synth
        multi_stream(args, synth.WORKLOADS[args.workload], args.streams)
        return
    import torch
    import streaming_paged_kv_amd as spkv
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    cache = spkv.PagedKVCache(**wl.cfg_kwargs(), device=dev)
    nb = wl.num_blocks
    S, W = wl.scale_frames, wl.sliding_window
    n_attn = 0 if args.no_events else args.steps     # window B frames
    n_app = 0 if args.no_events else min(args.steps, 20)  # window C frames
    # Untimed frames: those that fill the scale pages and the live window,
    # then --warmup more, so that every window below is at steady state.
    n_fill = fill_frames(wl)
    warm = n_fill + max(0, args.warmup)
    total = warm + args.steps + n_attn
    sched = frame_schedule(wl, max(total + n_app, wl.frames))

    # input bank, resident in HBM before timing
    nbank = max(1, min(args.bank, total))
    bank = [[synth.frame_qkv(wl, f, b, device=dev) for b in range(nb)]
            for f in range(nbank)]
    outs = [torch.empty((wl.tokens_per_frame, wl.num_heads, wl.head_dim),
                        dtype=torch.bfloat16, device=dev) for _ in range(nb)]
    sm = wl.head_dim ** -0.5
    hd = wl.num_heads * wl.head_dim
    nq = wl.tokens_per_frame
    fpp = wl.page_size // wl.num_special_tokens
    special_cap = -(-wl.max_total_frames // fpp) * fpp   # frames the special pages hold

    # Three windows over consecutive frames of the same stream:
    #   A  the timed region (value, ms_per_step): no events at all, since each
    #      timing event adds a few microseconds of idle time on the stream;
    #   B  per frame, every block's admit, eviction and plan first, then one
    #      pair of events around its runs back to back: the attention
    #      kernel's duration (with the split merge);
    #   C  events around each keyframe's appends (all blocks back to back):
    #      the append kernel's bandwidth.
    ev_attn, ev_app = [], []
    flops, app_bytes = [], []

    def planned_tokens():
        tab, npatch, lpl = cache.get_plan()
        nsp = len(tab) - npatch
        return (npatch * wl.patch_tokens +
                (nsp - 1) * wl.num_special_tokens *
                (wl.page_size // wl.num_special_tokens) + lpl)

    admit = cache.append_frame_in_run if args.append == "in_run" else cache.append_frame

    def step(f, mode):
        kind = sched[f]
        qkv = bank[f % nbank]
        if kind == "transient":
            # A non-keyframe attends to the cache and to its own K/V and skips
            # the append: run_own on every block, over the plan the last
            # keyframe left (the cache has not changed since).
            if mode == "B":
                nk = planned_tokens() + nq
                a0 = torch.cuda.Event(enable_timing=True)
                a1 = torch.cuda.Event(enable_timing=True)
                a0.record(stream)
            for b in range(nb):
                q, k, v = qkv[b]
                cache.run_own(b, q, k, v, out=outs[b], sm_scale=sm, stream=stream)
            if mode == "B":
                a1.record(stream)
                ev_attn.append((a0, a1, nb))
                flops.extend([4.0 * nq * nk * hd] * nb)
            return
        if wl.dynamic:
            cache.set_defer_eviction(True)
        if cache.get_cache_stats(0)[0] >= special_cap:
            # The special stream is full (only short streams get there within
            # the run): start over, as a streaming system resets its cache.
            cache.reset()
            if wl.dynamic:
                cache.set_defer_eviction(True)
        nk = None
        if mode == "C":
            # The frame's appends of all blocks back to back between two
            # events (blocks are independent, so appending every block before
            # the first evict/plan/run leaves each block's steps in order).
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for b in range(nb):
                cache.append_frame(b, qkv[b][1], qkv[b][2], stream=stream)
            e1.record(stream)
            ev_app.append((e0, e1))
            app_bytes.append(8 * nq * hd * nb)
        if mode == "B":
            # Every block's admit and eviction and the plan first, then the
            # 24 runs back to back between one pair of events, so that the
            # events hold the attention launches only (blocks are
            # independent: each block's own steps stay in order).
            for b in range(nb):
                admit(b, qkv[b][1], qkv[b][2], stream=stream)
                cache.evict_frames(b, S, W)
            cache.plan(stream=stream)
            nk = planned_tokens()
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            for b in range(nb):
                cache.run(b, qkv[b][0], out=outs[b], sm_scale=sm, stream=stream)
            a1.record(stream)
            ev_attn.append((a0, a1, nb))
            flops.extend([4.0 * nq * nk * hd] * nb)
        for b in range(nb if mode != "B" else 0):
            q, k, v = qkv[b]
            if mode != "C":
                admit(b, k, v, stream=stream)
            cache.evict_frames(b, S, W)
            if b == 0:
                cache.plan(stream=stream)
            cache.run(b, q, out=outs[b], sm_scale=sm, stream=stream)
        for b in range(nb):
            if kind == "reject":
                cache.rollback_last_frame(b)
            elif kind == "accept":
                cache.execute_deferred_eviction(b, S, W)

    def visible_now(f):
        # tokens a frame attends to: the plan's, plus its own for a non-keyframe
        return planned_tokens() + (nq if sched[f] == "transient" else 0)

    for f in range(warm):
        step(f, None)
    torch.cuda.synchronize()
    assert cache.get_cache_stats(0)[2] == W, "the live window is not full"
    nk_lo = visible_now(warm - 1)
    t0 = time.perf_counter()
    for f in range(warm, warm + args.steps):
        step(f, None)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    nk_hi = visible_now(warm + args.steps - 1)
    use_ev = not args.no_events
    if use_ev:
        for f in range(warm + args.steps, total):
            step(f, "B")
        for f in range(total, total + n_app):
            step(f, "C")
        torch.cuda.synchronize()

    # The whole stream as its configuration defines it (frames 0..frames-1)
    # from an empty cache, no events: the scale pages and the window filling
    # up are included, so this rate is above the steady-state one.
    full = None
    if not args.no_full_stream:
        cache.reset()
        torch.cuda.synchronize()
        t_full = time.perf_counter()
        for f in range(wl.frames):
            step(f, None)
        torch.cuda.synchronize()
        t_full = time.perf_counter() - t_full
        full = {"value": wl.frames / t_full, "unit": "frames/s", "frames": wl.frames,
                "window": f"frames 0..{wl.frames - 1} from an empty cache, no events"}

    result = {
        "metric": METRIC,
        "value": args.steps / dt,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dt / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"{wl.name}: {nb} blocks, H={wl.num_heads}, D={wl.head_dim}, "
                         f"page_size={wl.page_size}, {wl.patch_tokens} patch + "
                         f"{wl.num_special_tokens} special tokens/frame, "
                         f"S/W/R={wl.scale_frames}/{wl.sliding_window}/{wl.headroom}, "
                         f"keyframe_interval={wl.keyframe_interval}"
                         + (", dynamic accept/rollback" if wl.dynamic else
                            (", non-keyframes attend to cache + own K/V and skip the append"
                             if wl.keyframe_interval > 1 else ""))),
            "frames_timed": f"{warm}..{warm + args.steps - 1}",
            "untimed_frames": (f"{warm}: {n_fill} fill the scale pages and the "
                               f"{W}-page live window, then --warmup {args.warmup}"),
            "visible_tokens_timed": [nk_lo, nk_hi],
            "input_bank_frames": nbank,
            "keyframe_append": ("append_frame_in_run: each block's run copies the frame "
                                "into its pages inside the attention launch"
                                if args.append == "in_run" else
                                "append_frame: one copy launch per block"),
        },
    }
    if full is not None:
        result["full_stream"] = full
    if use_ev:
        t_attn = [a.elapsed_time(b) * 1e-3 for a, b, _ in ev_attn]
        t_app = [a.elapsed_time(b) * 1e-3 for a, b in ev_app]
        avg_attn = sum(t_attn) / sum(n for _, _, n in ev_attn)
        achieved = sum(flops) / sum(t_attn) / 1e12
        avg_flops = sum(flops) / len(flops)
        nk_b = [f / (4.0 * nq * hd) for f in flops]
        result["roofline"] = {
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": recorded_traffic(wl.name, sum(nk_b) / len(nk_b)),
            "kernel": "attn_kernel (+ split merge) per run()",
            "window": (f"frames {warm + args.steps}..{total - 1}, one pair of HIP "
                       f"events per frame around its {nb} run() calls, back to back "
                       f"on their stream"),
            "visible_tokens": [int(min(nk_b)), int(max(nk_b))],
            "avg_launch_us": avg_attn * 1e6,
            "algorithmic_flops_per_launch": avg_flops,
        }
        app_gbs = sum(app_bytes) / sum(t_app) / 1e9
        n_launch = len(t_app) * nb
        result["append"] = {
            "bound": "hbm", "achieved": app_gbs, "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": app_gbs / PEAK_HBM_GBS,
            "avg_launch_us": sum(t_app) / n_launch * 1e6,
            "window": (f"keyframes among frames {total}..{total + n_app - 1}: per frame, "
                       f"events around its {nb} plain appends (append_frame) issued back "
                       f"to back (launch gaps included)"),
            "bytes_per_launch": app_bytes[0] // nb,
        }
    cache.close()
    del bank
    # Plain copy of known size, outside every window: the factor between its
    # byte counters and COPY_BYTES calibrates the attention kernel's.
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, warm, args.cpu_blocks)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
