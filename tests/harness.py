"""Stream drivers for the GPU parity tests: the HIP path (through the binding)
and the oracle are each driven frame by frame with the same seeded inputs and
compared at chosen frames.  The two sides share only the inputs (synth)."""

import numpy as np
import torch

import synth
from oracle import OracleConfig, PagePoolOracle

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
REL_L2 = 1e-2


def frame_kinds(wl, frames=None):
    """Per frame: 'key' (append + evict, kept), 'transient' (non-keyframe:
    deferred append, attend, roll back), 'accept' / 'reject' (dynamic stream:
    deferred append, attend, then execute the eviction / roll back); and
    whether the cache is reset before the frame."""
    n = wl.frames if frames is None else frames
    dec = synth.accept_decisions(wl, n) if wl.dynamic else None
    out = []
    for f in range(n):
        reset = bool(wl.reset_every) and f > 0 and f % wl.reset_every == 0
        if wl.dynamic:
            kind = "accept" if dec[f] else "reject"
        else:
            kind = "key" if synth.is_keyframe(wl, f) else "transient"
        out.append((kind, reset))
    return out


def gpu_step(cache, wl, kind, reset, qkv, outs, stream=None, flags=(1, 0), in_run=False):
    """One frame on the HIP side.  qkv[b] = (q, k, v) device tensors; the
    run's output for block b is written into outs[b]; evict_frames gets the
    eviction flags (cross_frame_special, camera_only).  in_run: frames are
    admitted with append_frame_in_run, so each block's run copies them."""
    S, W = wl.scale_frames, wl.sliding_window
    if reset:
        cache.reset()
    if wl.dynamic:
        cache.set_defer_eviction(True)
    if kind == "transient":
        cache.set_defer_eviction(True)
    for b in range(wl.num_blocks):
        q, k, v = qkv[b]
        if in_run:
            cache.append_frame_in_run(b, k, v, stream=stream)
        else:
            cache.append_frame(b, k, v, stream=stream)
        cache.evict_frames(b, S, W, *flags)
        if b == 0:
            cache.plan(stream=stream)
        cache.run(b, q, out=outs[b], stream=stream)
    for b in range(wl.num_blocks):
        if kind in ("transient", "reject"):
            cache.rollback_last_frame(b)
        elif kind == "accept":
            cache.execute_deferred_eviction(b, S, W)
    if kind == "transient":
        cache.set_defer_eviction(False)


def dry_run(wl, frames=None, flags=(1, 0)):
    """State-machine-only pass over the schedule: for each frame, the plan
    (table, n_patch) and the frame that last wrote each page, plus
    milestone frames."""
    cfg = OracleConfig(**wl.cfg_kwargs())
    o = PagePoolOracle(cfg)
    kinds = frame_kinds(wl, frames)
    writer = {}
    plans = []
    writers_at = []
    ms = {}
    fpp = cfg.frames_per_special_page
    first_rb = None
    for f, (kind, reset) in enumerate(kinds):
        if reset:
            o.reset()
        if wl.dynamic or kind == "transient":
            o.set_defer_eviction(True)
        p, _, _ = o.append_frame(0)
        writer[p] = f
        moved = o.evict_frames(0, wl.scale_frames, wl.sliding_window, *flags)
        pl = o.plan()
        plans.append((list(pl.table), pl.n_patch))
        writers_at.append(dict(writer))
        scale, live, free, nsf = o.block_state(0)
        ms.setdefault("first", f)
        if len(scale) == wl.scale_frames and "scale_full" not in ms:
            ms["scale_full"] = f
        if live and "first_live" not in ms:
            ms["first_live"] = f
        if len(live) >= wl.sliding_window and "window_full" not in ms:
            ms["window_full"] = f
        if nsf == fpp and "nsf_fpp" not in ms:
            ms["nsf_fpp"] = f
        if nsf == fpp + 1 and "nsf_fpp1" not in ms:
            ms["nsf_fpp1"] = f
        if kind == "transient" and "first_transient" not in ms:
            ms["first_transient"] = f
        if kind in ("transient", "reject"):
            o.rollback_last_frame(0)
            if first_rb is None:
                first_rb = f
                ms["first_rollback"] = f
                if f + 1 < len(kinds):
                    ms["after_rollback"] = f + 1
        elif kind == "accept":
            moved += o.execute_deferred_eviction(0, wl.scale_frames, wl.sliding_window)
        if moved and "first_eviction" not in ms:
            ms["first_eviction"] = f
        if kind == "transient":
            o.set_defer_eviction(False)
    ms["last"] = len(kinds) - 1
    return kinds, plans, writers_at, ms


def needed_frames(wl, plans, writers_at, milestone_frames):
    """Frames whose patch tokens are visible at some milestone."""
    need = set()
    for m in milestone_frames:
        table, n_patch = plans[m]
        w = writers_at[m]
        for p in table[:n_patch]:
            need.add(w[p])
    return need


def sample_rows(nq, extra=24, seed=0):
    base = {0, 1, 5, 6, 7, 31, 32, 63, 64, 127, 128, 255, 256, 257, 511, 512,
            767, 768, 1000, nq - 1, nq - 2}
    rng = np.random.default_rng(seed)
    base |= set(int(x) for x in rng.integers(0, nq, extra))
    return sorted(r for r in base if 0 <= r < nq)


def compare(gpu_bf16, ref_f64, what):
    got = gpu_bf16.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref_f64)
    max_abs = float(err.max())
    mean_abs = float(err.mean())
    rel = float(np.linalg.norm(got - ref_f64) / max(np.linalg.norm(ref_f64), 1e-300))
    assert np.isfinite(got).all(), what
    assert max_abs <= MAX_ABS, (what, max_abs)
    assert mean_abs <= MEAN_ABS, (what, mean_abs)
    assert rel <= REL_L2, (what, rel)
    return max_abs, mean_abs, rel


def gen_frame(wl, f, nblocks, device):
    return [synth.frame_qkv(wl, f, b, device=device) for b in range(nblocks)]
