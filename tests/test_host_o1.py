"""The page-pool operations cost the same however long the stream has run.

"How LingBot-Map Implements the KV Cache Mechanism for Streaming Inference
with FlashInfer Integration", section "Append and Evict API": eviction runs in
O(1) amortized time per frame, and the summary calls append and evict O(1)
operations; "How to Improve Streaming Inference Performance with FlashInfer
KV Cache Backend", section "Two-Stream Page Pool Architecture": the manager
only moves page ids between deques and allocates nothing per frame.

Checked on a host-only handle (the C++ allocator through the C ABI, no GPU)
over a stream of 60,000 frames on 24 blocks (the special stream sized for
all of them): per frame at most one page moves per block; the handle's host
memory does not grow; and the time of a batch of frames late in the stream
is that of the same batch early on.  plan() is left out: it copies the
visible table, which grows with the special stream by design."""

import os
import time

import psutil

import streaming_paged_kv_amd as spkv

FRAMES = 60_000
BATCH = 1_000
BLOCKS = 24
S, W, R = 8, 64, 16


def _frame(c, lib, h, f):
    """One frame on every block: keyframes (even) are appended and evicted;
    odd frames are appended under deferral and rolled back, every fourth
    frame is appended under deferral and then accepted."""
    moved = 0
    if f % 4 == 3:
        lib.spkv_set_defer_eviction(h, 1)
        for b in range(BLOCKS):
            assert lib.spkv_append_frame(h, b, None, None, None) == 0
            assert lib.spkv_evict_frames(h, b, S, W, 1, 0) == 0
        for b in range(BLOCKS):
            before = c.get_cache_stats(b)[2] if b == 0 else None
            assert lib.spkv_execute_deferred_eviction(h, b, S, W) == 0
            if b == 0:
                moved = before - c.get_cache_stats(0)[2]
        lib.spkv_set_defer_eviction(h, 0)
    elif f % 2:
        lib.spkv_set_defer_eviction(h, 1)
        for b in range(BLOCKS):
            assert lib.spkv_append_frame(h, b, None, None, None) == 0
            assert lib.spkv_evict_frames(h, b, S, W, 1, 0) == 0
        for b in range(BLOCKS):
            assert lib.spkv_rollback_last_frame(h, b) == 0
        lib.spkv_set_defer_eviction(h, 0)
    else:
        for b in range(BLOCKS):
            assert lib.spkv_append_frame(h, b, None, None, None) == 0
            assert lib.spkv_evict_frames(h, b, S, W, 1, 0) == 0
    return moved


def test_append_evict_rollback_cost_does_not_grow_with_the_stream():
    c = spkv.PagedKVCache(num_blocks=BLOCKS, num_heads=16, head_dim=64, page_size=999,
                          patch_tokens=999, num_special_tokens=6, scale_frames=S,
                          sliding_window=W, headroom=R, max_total_frames=FRAMES,
                          host_only=True)
    lib, h = c.lib, c._h
    proc = psutil.Process(os.getpid())
    times = []
    rss = []
    max_moved = 0
    for f0 in range(0, FRAMES, BATCH):
        t0 = time.perf_counter()
        for f in range(f0, f0 + BATCH):
            max_moved = max(max_moved, _frame(c, lib, h, f))
        times.append(time.perf_counter() - t0)
        rss.append(proc.memory_info().rss)
        if f0 == 0:
            st = c.get_cache_stats(0)
            assert st[1] == S and st[2] == W and st[3] == R   # steady state reached
    # a frame moves at most one page per block out of the window
    assert max_moved <= 1
    st = c.get_cache_stats(0)
    assert (st[1], st[2], st[3]) == (S, W, R)
    # committed frames: keyframes (even) and accepted frames (f % 4 == 3)
    assert st[0] == FRAMES // 2 + FRAMES // 4
    # no host memory per frame: flat after the first batches
    assert rss[-1] - rss[2] < 4 << 20, (rss[2], rss[-1])
    # time per batch: the late batches are no slower than the early ones
    early = sorted(times[1:6])[2]
    late = sorted(times[-5:])[2]
    assert late < 1.5 * early + 0.01, (early, late)
    c.close()
