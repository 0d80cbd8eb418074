"""Planted mistakes in the oracle (on the CPU only) must each fail a pin.

Every mutant below is a plausible slip in writing the oracle -- a wrong end of
a deque, an off-by-one in the special packing, K and V swapped, a dropped max
subtraction that changes nothing in exact arithmetic but a missing scale
that does, a transposed operand.  Each is patched in, the pins that should
catch it are run, and at least one of them must fail.
"""

import collections
import json
import os

import numpy as np
import pytest

import oracle.attention as att
import oracle.pagepool as pp
from oracle import OracleConfig, PagePoolOracle

import oracle.bf16 as bf
import test_oracle_attention as ta
import test_oracle_bf16 as tb
import test_oracle_pins as tp


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, Exception):
        return True
    return False


def _pin_suite(golden_dir):
    return [
        lambda: tp.test_tiny_stream_worked_example(golden_dir),
        lambda: tp.test_special_tokens_land_in_order_after_patch_pages(golden_dir),
        lambda: tp.test_healthy_stats_224_stream(golden_dir),
        lambda: tp.test_42_frames_per_special_page_at_256(golden_dir),
        ta.test_brute_force_tiny_keyframes,
        ta.test_brute_force_interval_two,
        ta.test_brute_force_dynamic_accept_reject,
        ta.test_brute_force_padded_pages_and_odd_sizes,
        ta.test_matches_torch_sdpa_float64,
        ta.test_two_tokens_closed_form,
        ta.test_gather_reads_only_valid_slots,
        lambda: [tb.test_widening_hand_values(b, x) for b, x in tb.HAND],
        tb.test_widening_signed_zero_and_infinities,
        tb.test_widening_every_pattern_matches_torch,
        lambda: [tb.test_narrowing_rounds_to_nearest_even(x, b) for x, b in tb.NARROW],
        lambda: tp.test_eviction_flags_worked_example(golden_dir),
        lambda: [ta.test_brute_force_eviction_flags(f) for f in ta.EVICTION_FLAGS],
    ]


def _any_pin_fails(golden_dir):
    return any(_fails(f) for f in _pin_suite(golden_dir))


def test_unmutated_oracle_passes_every_pin(golden_dir):
    assert not _any_pin_fails(golden_dir)


class _FreeAppendLeft(collections.deque):
    pass


MUTANTS = {}


def mutant(name):
    def deco(fn):
        MUTANTS[name] = fn
        return fn
    return deco


@mutant("evicted page returned to head of free list")
def _m1(mp):
    def evict_to(self, blk, w):
        moved = 0
        while len(blk.live) > w:
            blk.free.appendleft(blk.live.popleft())
            moved += 1
        if moved:
            blk.last = None
        return moved
    mp.setattr(pp.PagePoolOracle, "_evict_to", evict_to)


@mutant("newest live page evicted instead of oldest")
def _m2(mp):
    def evict_to(self, blk, w):
        moved = 0
        while len(blk.live) > w:
            blk.free.append(blk.live.pop())
            moved += 1
        if moved:
            blk.last = None
        return moved
    mp.setattr(pp.PagePoolOracle, "_evict_to", evict_to)


@mutant("special slot off by one frame")
def _m3(mp):
    orig = pp.PagePoolOracle.special_slot

    def special_slot(self, f):
        return orig(self, f + 1)
    mp.setattr(pp.PagePoolOracle, "special_slot", special_slot)


@mutant("frames per special page rounds up")
def _m4(mp):
    mp.setattr(pp.OracleConfig, "frames_per_special_page",
               property(lambda self: -(-self.page_size // self.num_special_tokens)))


@mutant("last_page_len counts frames, not tokens")
def _m5(mp):
    orig = pp.PagePoolOracle.plan

    def plan(self):
        pl = orig(self)
        pl.last_page_len = pl.last_page_len // self.cfg.num_special_tokens
        return pl
    mp.setattr(pp.PagePoolOracle, "plan", plan)


@mutant("specials placed before the live window")
def _m6(mp):
    orig = pp.PagePoolOracle.plan

    def plan(self):
        pl = orig(self)
        n_sc = len(pl.scale)
        sp = pl.table[pl.n_patch:]
        pl.table = pl.table[:n_sc] + sp + pl.table[n_sc:pl.n_patch]
        return pl
    mp.setattr(pp.PagePoolOracle, "plan", plan)


@mutant("K and V swapped in the gather")
def _m7(mp):
    orig = att.gather_visible

    def gather(pool, plan, cfg):
        k, v = orig(pool, plan, cfg)
        return v, k
    mp.setattr(att, "gather_visible", gather)


@mutant("softmax scale dropped")
def _m8(mp):
    orig = att.dense_attention

    def dense(q, k, v, sm_scale, row_chunk=128):
        return orig(q, k, v, 1.0, row_chunk)
    mp.setattr(att, "dense_attention", dense)
    import oracle.brute as br
    mp.setattr(br, "dense_attention", dense)


@mutant("patch rows taken from the front of the frame")
def _m9(mp):
    orig = pp.PagePoolOracle.append_frame

    def append(self, b, k=None, v=None):
        if k is not None:
            ns = self.cfg.num_special_tokens
            k = np.concatenate([k[-ns:], k[:-ns]])
            v = np.concatenate([v[-ns:], v[:-ns]])
        return orig(self, b, k, v)
    mp.setattr(pp.PagePoolOracle, "append_frame", append)


@mutant("rollback returns the page to the tail of the free list")
def _m10(mp):
    def rollback(self, b):
        self._check_block(b)
        blk = self.blocks[b]
        if blk.last is None:
            raise pp.OracleError("NOTHING_TO_ROLLBACK")
        p, where = blk.last
        (blk.scale if where == "scale" else blk.live).pop()
        blk.free.append(p)
        blk.nsf -= 1
        blk.last = None
        return p
    mp.setattr(pp.PagePoolOracle, "rollback_last_frame", rollback)


@mutant("transposed product in the score matrix")
def _m11(mp):
    def dense(q, k, v, sm_scale, row_chunk=128):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        nq, nh, d = q.shape
        out = np.empty((nq, nh, v.shape[2]))
        for h in range(nh):
            # normalise over queries instead of keys
            sc = sm_scale * (q[:, h, :] @ k[:, h, :].T)
            sc -= sc.max(axis=0, keepdims=True)
            p = np.exp(sc)
            p /= p.sum(axis=0, keepdims=True)
            out[:, h, :] = p @ v[:, h, :]
        return out
    mp.setattr(att, "dense_attention", dense)
    import oracle.brute as br
    mp.setattr(br, "dense_attention", dense)


@mutant("scale routing uses <= instead of <")
def _m12(mp):
    orig = pp.PagePoolOracle.append_frame

    def append(self, b, k=None, v=None):
        blk = self.blocks[b] if 0 <= b < self.cfg.num_blocks else None
        r = orig(self, b, k, v)
        if blk is not None and blk.last[1] == "live" and len(blk.scale) == self.cfg.scale_frames \
                and len(blk.live) == 1 and self.cfg.scale_frames > 0:
            p = blk.live.pop()
            blk.scale.append(p)
            blk.last = (p, "scale")
        return r
    mp.setattr(pp.PagePoolOracle, "append_frame", append)


def _patch_widening(mp, fn):
    mp.setattr(bf, "bf16_bits_to_f64", fn)
    mp.setattr(att, "bf16_bits_to_f64", fn)


@mutant("bf16 widening shifts the uint16 without widening it first")
def _m13(mp):
    def widen(bits):
        b = np.asarray(bits, dtype=np.uint16)
        return (b << np.uint16(16)).astype(np.uint32).view(np.float32).astype(np.float64)
    _patch_widening(mp, widen)


@mutant("bf16 widening shifts by 15")
def _m14(mp):
    def widen(bits):
        b = np.asarray(bits, dtype=np.uint16)
        return (b.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    _patch_widening(mp, widen)


@mutant("bf16 pattern read as float16")
def _m15(mp):
    def widen(bits):
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    _patch_widening(mp, widen)


@mutant("bf16 narrowing truncates instead of rounding")
def _m16(mp):
    def narrow(x):
        f = np.asarray(x, dtype=np.float64).astype(np.float32)
        return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    mp.setattr(bf, "f64_to_bf16_bits", narrow)


@mutant("bf16 narrowing rounds ties away from zero")
def _m17(mp):
    def narrow(x):
        f = np.asarray(x, dtype=np.float64).astype(np.float32)
        u = f.view(np.uint32).astype(np.uint64)
        return ((u + np.uint64(0x8000)) >> np.uint64(16)).astype(np.uint16)
    mp.setattr(bf, "f64_to_bf16_bits", narrow)


@mutant("camera token taken as the last of a frame's specials")
def _m18(mp):
    def visible_slots(self, cfg):
        ns, fpp, m = cfg.num_special_tokens, cfg.frames_per_special_page, cfg.num_patch_pages
        out = []
        for i, (page, n) in enumerate(zip(self.table, self.page_lengths(cfg))):
            if i < self.n_patch:
                out.append(list(range(n)))
                continue
            out.append([o for o in range(n)
                        if o % ns >= ns - self.spec_vis[(page - m) * fpp + o // ns]])
        return out
    mp.setattr(pp.Plan, "visible_slots", visible_slots)


@mutant("evicted frames keep every special whatever the flags")
def _m19(mp):
    mp.setattr(pp, "special_tokens_kept", lambda cfg, cross, camera: cfg.num_special_tokens)


@mutant("a deferred evict_frames call does not record its flags")
def _m20(mp):
    orig = pp.PagePoolOracle.evict_frames

    def evict(self, b, s, w, cross_frame_special=1, camera_only=0):
        if self.defer:
            self._check_block(b)
            self._check_evict_args(s, w)
            return 0
        return orig(self, b, s, w, cross_frame_special, camera_only)
    mp.setattr(pp.PagePoolOracle, "evict_frames", evict)


@mutant("special pages with no visible token stay in the table")
def _m21(mp):
    orig = pp.PagePoolOracle.plan

    def plan(self):
        pl = orig(self)
        c = self.cfg
        n_sp = -(-pl.nsf // c.frames_per_special_page)
        pl.table = pl.table[:pl.n_patch] + [c.num_patch_pages + i for i in range(n_sp)]
        return pl
    mp.setattr(pp.PagePoolOracle, "plan", plan)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, golden_dir, monkeypatch):
    MUTANTS[name](monkeypatch)
    assert _any_pin_fails(golden_dir), f"no pin caught mutant: {name}"
