"""Every global and LDS address of the attention kernel's loads, modelled on
the host (tests/attn_address_model.py), stays inside its buffer for the
geometries the GPU tests and the benchmark run, at every split count the host
may choose.  The plans come from the C++ allocator through the C ABI
(host-only handles); the row maps are what the plan's expansion writes.

Checked per launch: the block-id to work-item mapping is a bijection; no
split is empty; the staged row-map reads stay inside the padded map; the
32-bit byte offsets do not wrap, and pool offsets never carry the own-row
mark in run_own's map; each tile's loads fill every LDS slot of its stage
exactly once under the chunk swizzle; every pool load lies in the pool and
every load of the caller's rows in the caller's frame; fragment reads stay
inside a tile; queries, outputs, partials and the merge stay in range.  The
same for the map of a run that copies the newest frame, whose tokens it reads
from the caller's frame."""

import pytest

import attn_address_model as M
import streaming_paged_kv_amd as spkv
import synth

SPLITS = (1, 2, 3, 5, 7, 8, 13, 16, 32)


def _geometries():
    W = synth.Workload
    return [
        # name, workload, frames driven, frames modelled, flags
        ("tiny", synth.WORKLOADS["tiny"], 12, (0, 5, 11), (1, 0)),
        ("mid", W("mid", 1, 16, 64, 203, 200, 6, 2, 6, 2, 64, 40, keyframe_interval=2),
         40, (0, 10, 38), (1, 1)),
        ("degenerate", W("degenerate", 1, 3, 64, 6, 5, 6, 0, 1, 1, 30, 30), 30, (0, 29),
         (1, 0)),
        ("80-heads", W("80-heads", 1, 80, 64, 64, 58, 6, 1, 3, 1, 40, 8), 8, (7,), (1, 0)),
        ("224x224", synth.WORKLOADS["224x224"].with_(num_blocks=1), 200, (0, 71, 199), (1, 0)),
        ("518x378", synth.WORKLOADS["518x378"].with_(num_blocks=1), 600, (0, 150, 598), (1, 0)),
        ("518x378 camera", synth.WORKLOADS["518x378"].with_(num_blocks=1), 600, (598,),
         (1, 1)),
        ("padded", synth.WORKLOADS["518x378-padded"].with_(num_blocks=1), 4096, (4094,),
         (1, 0)),
        ("dynamic", synth.WORKLOADS["dynamic"].with_(num_blocks=1), 1000, (999,), (0, 0)),
        ("pool-4GiB", W("pool-4GiB", 1, 16, 64, 256, 256, 6, 2, 4090, 2, 84, 44), 44,
         (0, 43), (1, 0)),
        ("pool-2GiB", W("pool-2GiB", 1, 16, 64, 256, 256, 6, 2, 2042, 2, 84, 84), 84,
         (0, 83), (1, 0)),
    ]


@pytest.fixture(scope="module", autouse=True)
def _fragments():
    M.check_fragment_offsets()


@pytest.mark.parametrize("name,wl,frames,at,flags", _geometries(),
                         ids=[g[0] for g in _geometries()])
def test_attention_loads_stay_in_bounds(name, wl, frames, at, flags):
    cfg = wl.cfg_kwargs()
    c = spkv.PagedKVCache(host_only=True, **cfg)
    pool_bytes = c.pool_bytes
    S, W = wl.scale_frames, wl.sliding_window
    n_own = wl.tokens_per_frame
    checked = 0
    for f in range(frames):
        key = synth.is_keyframe(wl, f) if not wl.dynamic else True
        if not key:
            continue                      # non-keyframes: run_own on the committed cache
        c.append_frame(0)
        c.evict_frames(0, S, W, *flags)
        if f not in at:
            continue
        c.plan()
        table, n_patch, _ = c.get_plan()
        rows = M.plan_rows(table, n_patch, c.get_plan_specials(), cfg)
        nk = len(rows)
        first_new = (n_patch - 1) * wl.patch_tokens
        rm, rm_own, rm_new = M.expand(rows, n_own, first_new, wl.num_special_tokens)
        for nq in sorted({1, wl.tokens_per_frame, 8 * wl.tokens_per_frame}):
            for s in SPLITS:
                M.check_launch(rm, nk, nk, nq, wl.num_heads, wl.page_size, pool_bytes, s)
                if pool_bytes <= 1 << 31:     # own rows need pools up to 2 GiB
                    M.check_launch(rm_own, nk + n_own, nk, nq, wl.num_heads, wl.page_size,
                                   pool_bytes, s, own_frame_rows=n_own)
                    # a run that copies the newest frame (append_frame_in_run)
                    M.check_launch(rm_new, nk, first_new, nq, wl.num_heads, wl.page_size,
                                   pool_bytes, s, own_frame_rows=n_own)
        checked += 1
    c.close()
    assert checked == len(at), name


def test_model_catches_a_row_past_the_pool():
    """The model itself: a row map entry one page past the pool, or a staged
    read past the padded map, is reported."""
    rows = M.plan_rows([0, 1], 2, [[0, 2, 6]],
                       dict(page_size=16, patch_tokens=16, num_special_tokens=6,
                            scale_frames=1, sliding_window=1, headroom=0))
    rm, _ = M.expand(rows, 22)
    pool_bytes = 4 * 2 * 16 * 4 * 128   # 4 pages of 4 heads
    M.check_launch(rm, len(rows), len(rows), 22, 4, 16, pool_bytes, 1)
    bad = rm.copy()
    bad[5] = 4 * 2 * 16                  # first row of page 4: outside the pool
    with pytest.raises(AssertionError):
        M.check_launch(bad, len(rows), len(rows), 22, 4, 16, pool_bytes, 1)
    with pytest.raises(AssertionError):
        M.check_launch(rm[:40], len(rows), len(rows), 22, 4, 16, pool_bytes, 1)
