"""Host model of the memory addresses the attention kernel forms (CPU only).

The paged attention kernel ("How LingBot-Map Implements the KV Cache
Mechanism for Streaming Inference with FlashInfer Integration", section
"Kernel-Level Execution Flow") reads K/V rows of the pool through a per-token
row map, with direct-to-LDS loads whose global address is a 64-bit base plus
a 32-bit byte offset and whose LDS address comes from M0.  This module
restates, in numpy, every index the kernel and its launch compute:

  * the work-item mapping of the launch (XCD-ordered block ids -> items);
  * the key range of each item (split, chunks of at most 16384 tokens, 64-key
    tiles, the last one partial);
  * the row map the plan's expansion writes (padded past the last token),
    its byte offsets (32-bit products, the caller's rows marked by the top
    bit in run_own's map), and which rows of it each chunk stages;
  * for every tile, wave and lane, the two 16-byte loads: the global address
    (pool or caller's frame, head slice, swizzled chunk) and the LDS slot;
  * the fragment reads inside a stage, the query loads, the output and
    split-partial stores, and the merge's reads.

check_launch() asserts that each of them stays inside its buffer for one
launch, and that the loads of a tile fill every LDS slot of the stage
exactly once.  The tests run it for every geometry the GPU tests and the
benchmark use, at every split count the host may choose.
"""

import numpy as np

KEY_TILE = 64          # keys per tile
QUERY_TILE = 512       # query rows per workgroup (8 waves x 64)
STAGES = 4             # LDS ring depth
ROW_B = 128            # bytes of one key row of one head (64 bf16)
TILE_B = KEY_TILE * ROW_B
STAGE_B = 2 * TILE_B   # K tile, then V tile
RM_MAX = 16384         # row-map entries staged in LDS at a time
ROW_PAD = 2 * KEY_TILE
OWN = 0x80000000       # row-map mark of the caller's own rows
MAX_SPLITS = 32


def round_up(x, a):
    return (x + a - 1) // a * a


def swz(x):
    x = np.asarray(x)
    return ((x & 3) << 1) | ((x >> 2) & 1)


def plan_rows(table, n_patch, specials, cfg):
    """Pool row (page * 2 * page_size + slot) of every visible token, in run()
    order: the patch pages' tokens, then the special runs [first frame,
    frames, kept] (frame f at page M + f // fpp, slot 6 * (f % fpp))."""
    ps, pt, ns = cfg["page_size"], cfg["patch_tokens"], cfg["num_special_tokens"]
    m = cfg["scale_frames"] + cfg["sliding_window"] + cfg["headroom"]
    fpp = ps // ns
    rows = [np.int64(p) * 2 * ps + np.arange(pt, dtype=np.int64) for p in table[:n_patch]]
    for first, count, kept in specials:
        f = np.arange(first, first + count, dtype=np.int64)
        page = m + f // fpp
        slot = ns * (f % fpp)
        rows.append(((page * 2 * ps + slot)[:, None] + np.arange(kept)[None, :]).reshape(-1))
    return np.concatenate(rows)


def expand(rows, n_own, new_patch_begin=None, num_special=6):
    """The row maps the expansion kernel writes: run()'s (entries past the
    last token repeat it), run_own()'s (the caller's n_own rows after the
    plan's tokens, marked; entries past them repeat the last) and, given the
    first token of the newest frame's patch page, the map of a run that
    copies that frame (its patch tokens and the last num_special tokens
    marked as rows of the caller's frame)."""
    nk = len(rows)
    n_out = round_up(nk, KEY_TILE) + ROW_PAD
    rm = rows[np.minimum(np.arange(n_out), nk - 1)]
    n_out_own = round_up(nk + n_own, KEY_TILE) + ROW_PAD
    t = np.arange(n_out_own)
    rm_own = np.where(t < nk, rows[np.minimum(t, nk - 1)],
                      OWN | np.minimum(t - nk, n_own - 1))
    if new_patch_begin is None:
        return rm.astype(np.int64), rm_own.astype(np.int64)
    t = np.arange(n_out)
    patch_len = n_own - num_special
    d_patch = t - new_patch_begin
    d_spec = t - (nk - num_special)
    rm_new = np.where((d_patch >= 0) & (d_patch < patch_len), OWN | (num_special + d_patch),
                      np.where((d_spec >= 0) & (t < nk), OWN | d_spec, rm))
    return rm.astype(np.int64), rm_own.astype(np.int64), rm_new.astype(np.int64)


def item_of_block(n_items):
    """Work item of every workgroup of the launch (-1: returns at once)."""
    grid = round_up(n_items, 8)
    per_xcd = grid >> 3
    bid = np.arange(grid)
    item = (bid & 7) * per_xcd + (bid >> 3)
    return np.where(item < n_items, item, -1)


def split_layout(nk, splits_wanted):
    """(splits, tokens_per_split) the host derives from a wanted split count."""
    n_ktiles = -(-nk // KEY_TILE)
    s = max(1, min(splits_wanted, n_ktiles))
    tiles_per_split = -(-n_ktiles // s)
    return -(-n_ktiles // tiles_per_split), tiles_per_split * KEY_TILE


def lane_loads():
    """Per (kv, wq, lane, load): the key row inside the tile, the source chunk
    and the LDS byte offset inside the stage."""
    kv, wq, lane, second = np.meshgrid(np.arange(2), np.arange(4), np.arange(64),
                                       np.arange(2), indexing="ij")
    r = lane >> 3
    row = 16 * wq + r + 8 * second
    chunk = (lane & 7) ^ swz(r)
    lds = kv * TILE_B + 16 * wq * ROW_B + 1024 * second + 16 * lane
    return kv.ravel(), row.ravel(), chunk.ravel(), lds.ravel()


def check_fragment_offsets():
    """The MFMA fragment reads (K: 16 B per lane, V^T: two 8 B transposing
    reads per lane) stay inside one 8 KiB tile."""
    lane = np.arange(64)
    col, half = lane & 31, lane >> 5
    fk = swz(col & 7)
    hi_k = 0
    for s in range(4):
        for mt in range(2):
            kofs = col * ROW_B + (((2 * s + half) ^ fk) * 16) + 32 * mt * ROW_B
            assert kofs.min() >= 0
            hi_k = max(hi_k, int(kofs.max()) + 16)
    q16, j = lane >> 4, lane & 15
    r = 4 * (q16 >> 1) + (j >> 2)
    fv = swz(r)
    hi_v = 0
    for dt in range(2):
        vofs = r * ROW_B + (((4 * dt + 2 * (q16 & 1) + ((j >> 1) & 1)) ^ fv) * 16) + (j & 1) * 8
        for k2 in range(4):
            for upper in range(2):
                p = vofs + 16 * k2 * ROW_B + upper * 8 * ROW_B
                assert p.min() >= 0
                hi_v = max(hi_v, int(p.max()) + 8)
    assert hi_k <= TILE_B and hi_v <= TILE_B, (hi_k, hi_v)


def check_launch(rowmap, nk, n_cached, nq, num_heads, page_size, pool_bytes,
                 splits_wanted, own_frame_rows=0):
    """Every address one attention launch forms, against its buffers.

    rowmap: the map the launch reads (run()'s, or run_own()'s when
    own_frame_rows > 0); nk: tokens it attends to (n_cached of them from the
    pool).  Returns the number of global loads modelled."""
    own = own_frame_rows > 0
    hd = num_heads * 64
    row_bytes = hd * 2
    splits, tps = split_layout(nk, splits_wanted)
    n_qtiles = -(-nq // QUERY_TILE)
    n_items = n_qtiles * num_heads * splits
    item = item_of_block(n_items)
    live = item[item >= 0]
    assert np.array_equal(np.sort(live), np.arange(n_items)), "item mapping"
    # the row map's byte offsets, as the staging loop forms them (32-bit)
    e = rowmap & ~OWN
    prod = e * row_bytes
    assert prod.max() < (1 << 32), "32-bit byte offset wraps"
    ofs = prod | (rowmap & OWN)
    if own:
        assert (prod[rowmap & OWN == 0] < (1 << 31)).all(), "pool offset reads as own"
    kv, row_in_tile, chunk, lds = lane_loads()
    # the loads of one tile fill every 16-byte slot of its K and V tiles once
    slot = kv * TILE_B + row_in_tile * ROW_B + (chunk ^ swz(row_in_tile & 7)) * 16
    assert np.array_equal(np.sort(lds), np.arange(0, STAGE_B, 16)), "LDS slots"
    assert np.array_equal(np.sort(slot), np.arange(0, STAGE_B, 16)), "swizzle"
    assert lds.max() + 16 <= STAGE_B and (STAGES - 1) * STAGE_B + STAGE_B <= STAGES * STAGE_B
    v_off = np.where(kv == 1, page_size * row_bytes, 0)
    n_loads = 0
    for split in range(splits):
        t_begin, t_end = split * tps, min(nk, (split + 1) * tps)
        assert t_begin < t_end, "empty split"
        for c0 in range(t_begin, t_end, RM_MAX):
            c1 = min(t_end, c0 + RM_MAX)
            T = -(-(c1 - c0) // KEY_TILE)
            assert T * KEY_TILE <= RM_MAX
            assert c0 + T * KEY_TILE <= len(rowmap), "row map read past its end"
            staged = ofs[c0:c0 + T * KEY_TILE]
            own_tile = (n_cached - c0) // KEY_TILE if n_cached > c0 else 0
            # all tiles, all (kv, row, chunk) loads: offset inside the row
            o = staged.reshape(T, KEY_TILE)[:, row_in_tile] | (chunk * 16)[None, :]
            tile = np.arange(T)[:, None]
            from_own = own & (tile >= own_tile) & ((o & OWN) != 0)
            if own:
                assert not ((tile < own_tile) & ((o & OWN) != 0)).any(), "own row before own_tile"
            o = o & ~OWN
            for h in (0, num_heads - 1):
                pool_addr = h * 64 * 2 + v_off[None, :] + o
                own_addr = h * 64 * 2 + o
                bad_pool = (~from_own) & ((pool_addr < 0) | (pool_addr + 16 > pool_bytes))
                bad_own = from_own & ((own_addr < 0) |
                                      (own_addr + 16 > own_frame_rows * row_bytes))
                assert not bad_pool.any(), ("pool load out of bounds", split, c0, h)
                assert not bad_own.any(), ("own load out of bounds", split, c0, h)
            n_loads += o.size * num_heads * n_qtiles
    # queries, outputs and split partials
    q0 = np.arange(0, n_qtiles * QUERY_TILE, 64)
    qi = (q0[:, None, None] + np.arange(2)[None, :, None] * 32 +
          np.arange(32)[None, None, :]).ravel()
    qi = qi[qi < nq]
    assert (qi.max() + 1) * hd <= nq * hd
    if splits > 1:
        rows = (splits - 1) * nq * num_heads + (nq - 1) * num_heads + num_heads - 1
        assert (rows + 1) * 64 <= splits * nq * num_heads * 64
        # merge: threads gid < rows*16 read (m, l) and O of every split
        merge_rows = nq * num_heads
        assert ((splits - 1) * merge_rows + merge_rows - 1 + 1) * 2 <= splits * merge_rows * 2
    return n_loads
