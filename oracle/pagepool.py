"""Part 1 of the oracle: the two-stream page-pool state machine, step by step.

TEST INFRASTRUCTURE ONLY (see the package docstring for the page tags).

The result of the method here is a data-structure state, so this module walks
the method's steps in the order the pages give them, on plain Python deques,
lists and a numpy byte pool.  Nothing is blocked, fused or reordered.

Where the pages are silent or garbled the reading taken is stated next to the
step; the same readings are listed, numbered R1..R18, in the design notes.

Per block the state is
  free   deque of patch page ids, initially [0, 1, ..., M-1]
  scale  list of patch page ids holding the first S appended frames
  live   deque of patch page ids of the sliding window, oldest first
  nsf    number of frames whose special tokens are in the special stream
  last   (page, 'scale'|'live') of the most recent append, or None
  frame_of  page id -> index (in the special stream) of the frame it holds
  spec_vis  per committed frame, how many of its special tokens are visible
  flags  (cross_frame_special, camera_only) of the block's last evict_frames
plus one manager-wide ``defer`` flag, and optionally the pool bytes
  pool   uint16 [max_num_pages, 2, page_size, H, D]  (bf16 patterns, 0=K 1=V)
"""

from collections import deque
from dataclasses import dataclass, field
import numpy as np


# Error names are shared with the C ABI by *name* only (the tests map them).
ERRORS = (
    "INVALID_ARG",
    "BAD_BLOCK",
    "POOL_EXHAUSTED",
    "SPECIAL_OVERFLOW",
    "NOTHING_TO_ROLLBACK",
    "EMPTY",
    "NOT_PLANNED",
    "STALE_PLAN",
    "UNSUPPORTED",
)


class OracleError(Exception):
    """Raised with one of ERRORS; the state is unchanged when it is raised."""

    def __init__(self, name):
        assert name in ERRORS, name
        super().__init__(name)
        self.name = name


@dataclass(frozen=True)
class OracleConfig:
    """Manager parameters.

    [LB-PERF] "Minimal Streaming Inference Setup" constructs the manager from
    num_blocks, tokens_per_frame, num_heads, head_dim, num_special_tokens,
    scale_frames, sliding_window and max_total_frames; [LB-KV] "How is memory
    bounded in streaming mode?" sizes the patch pool as scale_frames +
    sliding_window + headroom pages.  ``patch_tokens`` is tokens_per_frame
    minus the special tokens; it may be smaller than ``page_size`` (padded
    pages, [LB-PERF] "Page-Size Handling for FA2 vs FA3").
    """

    num_blocks: int
    num_heads: int
    head_dim: int
    page_size: int
    patch_tokens: int
    num_special_tokens: int
    scale_frames: int
    sliding_window: int
    headroom: int
    max_total_frames: int

    @property
    def num_patch_pages(self):
        # [LB-SLOT] "双流分页布局": scale 8 + window 64 + headroom 16 = 88 pages.
        return self.scale_frames + self.sliding_window + self.headroom

    @property
    def frames_per_special_page(self):
        # [LB-SLOT] "特殊 token 流": a special page holds floor(page_size / 6)
        # frames (42 at page_size 256).  Whole frames only (reading R4).
        return self.page_size // self.num_special_tokens

    @property
    def num_special_pages(self):
        # [LB-SLOT] "特殊 token 流": the special pool is preallocated for
        # max_total_frames frames.
        return -(-self.max_total_frames // self.frames_per_special_page)

    @property
    def max_num_pages(self):
        # [LB-KV] "Physical Page Layout and Indexing": pages 0..M-1 are patch
        # pages, the remaining ones special pages.
        return self.num_patch_pages + self.num_special_pages

    @property
    def special_capacity_frames(self):
        # Reading R8: overflow is physical (every slot of every special page).
        return self.num_special_pages * self.frames_per_special_page

    @property
    def tokens_per_frame(self):
        return self.num_special_tokens + self.patch_tokens

    def validate(self):
        c = self
        ok = (
            c.num_blocks >= 1
            and c.num_heads >= 1
            and c.head_dim >= 1
            and c.num_special_tokens >= 1
            and c.page_size >= c.num_special_tokens
            and 1 <= c.patch_tokens <= c.page_size
            and c.scale_frames >= 0
            and c.sliding_window >= 1
            and c.headroom >= 0
            and c.max_total_frames >= 1
        )
        if not ok:
            raise OracleError("INVALID_ARG")


@dataclass
class Plan:
    """What plan() builds once per frame step from block 0.

    [LB-KV] "Kernel-Level Execution Flow" and [LB-PERF] "One-Time Planning
    Pattern": the visible page table in the order scale -> live window ->
    special, and the number of valid tokens in the last special page.
    """

    table: list
    n_patch: int
    last_page_len: int
    # Snapshot of block 0's state the plan was built from (reading R14).
    scale: tuple = field(default=())
    live: tuple = field(default=())
    nsf: int = 0
    # Per committed frame, how many of its special tokens are visible
    # (reading R13); all of them unless an eviction flag removed some.
    spec_vis: tuple = field(default=())

    def page_lengths(self, cfg):
        """Valid tokens of each table entry, derived from its position.

        Patch pages hold the frame's patch tokens; special pages before the
        last hold num_special_tokens * frames_per_special_page tokens
        (reading R4); the last one holds last_page_len.
        """
        n = len(self.table)
        full = cfg.num_special_tokens * cfg.frames_per_special_page
        out = []
        for i in range(n):
            if i < self.n_patch:
                out.append(cfg.patch_tokens)
            elif i < n - 1:
                out.append(full)
            else:
                out.append(self.last_page_len)
        return out

    def visible_slots(self, cfg):
        """For each table entry, the list of its valid slots that are visible.

        Patch pages: all of their valid slots.  Special pages: slot o of
        special page p holds token o % num_special of frame
        (p - M) * frames_per_special_page + o // num_special ([LB-SLOT]
        "特殊 token 流"), and it is visible when that token's index is below the
        frame's count in spec_vis (reading R13: the camera token is the first).
        """
        ns, fpp, m = cfg.num_special_tokens, cfg.frames_per_special_page, cfg.num_patch_pages
        out = []
        for i, (page, n) in enumerate(zip(self.table, self.page_lengths(cfg))):
            if i < self.n_patch:
                out.append(list(range(n)))
                continue
            keep = []
            for o in range(n):
                frame = (page - m) * fpp + o // ns
                if o % ns < self.spec_vis[frame]:
                    keep.append(o)
            out.append(keep)
        return out

    def num_visible_tokens(self, cfg):
        return int(sum(len(x) for x in self.visible_slots(cfg)))


class _Block:
    def __init__(self, m):
        self.free = deque(range(m))     # reading R1: initial order 0..M-1
        self.scale = []
        self.live = deque()
        self.nsf = 0
        self.last = None
        self.frame_of = {}
        self.spec_vis = []
        self.flags = (1, 0)             # reading R13: the pages' defaults


def special_tokens_kept(cfg, cross_frame_special, camera_only):
    """How many of an evicted frame's special tokens stay visible (reading
    R13).  [LB-KV] "Append and Evict API": eviction recycles the oldest patch
    pages "while optionally preserving special tokens"; [LB-SLOT] "特殊 token
    流": kept specials are where cross-frame context comes from, the camera
    tokens of any earlier frame in particular.  cross_frame_special=1 keeps
    them (all of them, or with camera_only=1 the camera token, the first of
    the frame's specials); cross_frame_special=0 keeps none."""
    if not cross_frame_special:
        return 0
    return 1 if camera_only else cfg.num_special_tokens


class PagePoolOracle:
    """The manager: per-block page-pool states plus the shared plan.

    ``track_pool`` selects the blocks whose pool bytes are kept (a numpy array
    per tracked block, zero-initialised like the device pools).
    """

    def __init__(self, cfg, track_pool=()):
        cfg.validate()
        self.cfg = cfg
        self.defer = False
        self.blocks = [_Block(cfg.num_patch_pages) for _ in range(cfg.num_blocks)]
        self.plan_state = None
        self.pools = {}
        for b in track_pool:
            self._check_block(b)
            self.pools[b] = np.zeros(
                (cfg.max_num_pages, 2, cfg.page_size, cfg.num_heads, cfg.head_dim),
                dtype=np.uint16,
            )

    # ------------------------------------------------------------------ utils
    def _check_block(self, b):
        if not (0 <= b < self.cfg.num_blocks):
            raise OracleError("BAD_BLOCK")

    def _check_evict_args(self, scale_frames, sliding_window):
        # Reading R12: routing happens at append time with the manager's S, so
        # the call must name the same S; the window must leave room for the
        # scale pages inside the patch pool.
        c = self.cfg
        if scale_frames != c.scale_frames:
            raise OracleError("INVALID_ARG")
        if not (1 <= sliding_window <= c.num_patch_pages - c.scale_frames):
            raise OracleError("INVALID_ARG")

    def special_slot(self, frame_index):
        """(page, first slot) of a frame's special tokens in the special stream.

        [LB-SLOT] "特殊 token 流": frames are packed contiguously,
        floor(page_size/6) whole frames per page, after the patch pages.
        """
        c = self.cfg
        fpp = c.frames_per_special_page
        return (
            c.num_patch_pages + frame_index // fpp,
            c.num_special_tokens * (frame_index % fpp),
        )

    # -------------------------------------------------------------- the steps
    def append_frame(self, b, k=None, v=None):
        """append_frame(block_idx, K, V).

        [LB-KV] "Append and Evict API"; [LB-SLOT] "scale frames：永不驱逐的前 8
        个 slot": the new patch page goes to the scale pages while fewer than
        scale_frames are held, else to the live window; [LB-SLOT] "特殊 token
        流": the frame's special tokens join the append-only special stream.
        K and V are [num_special + patch_tokens, H, D] bf16 patterns in token
        order [camera, register x4, scale, patch...] ([LB-SLOT] "为什么流式 3D
        重建离不开 KV 缓存").  Returns (page, special_page, special_slot).
        """
        self._check_block(b)
        c = self.cfg
        blk = self.blocks[b]
        if not blk.free:
            raise OracleError("POOL_EXHAUSTED")
        if blk.nsf >= c.special_capacity_frames:
            raise OracleError("SPECIAL_OVERFLOW")
        if b in self.pools:
            shape = (c.tokens_per_frame, c.num_heads, c.head_dim)
            if k is None or v is None or k.shape != shape or v.shape != shape:
                raise OracleError("INVALID_ARG")

        p = blk.free.popleft()          # reading R1: allocate from the head
        if len(blk.scale) < c.scale_frames:
            blk.scale.append(p)
            where = "scale"
        else:
            blk.live.append(p)
            where = "live"
        s_page, s_slot = self.special_slot(blk.nsf)

        if b in self.pools:
            pool = self.pools[b]
            ns, pt = c.num_special_tokens, c.patch_tokens
            # [LB-KV] "Physical Page Layout and Indexing": index 0 = K, 1 = V.
            pool[p, 0, 0:pt] = k[ns:ns + pt]
            pool[p, 1, 0:pt] = v[ns:ns + pt]
            pool[s_page, 0, s_slot:s_slot + ns] = k[0:ns]
            pool[s_page, 1, s_slot:s_slot + ns] = v[0:ns]

        blk.frame_of[p] = blk.nsf
        blk.spec_vis.append(c.num_special_tokens)   # a resident frame: all visible
        blk.nsf += 1
        blk.last = (p, where)
        return p, s_page, s_slot

    def _evict_to(self, blk, sliding_window):
        """Pop the oldest live pages to the tail of the free list while the
        window is over its limit ([LB-SLOT] "keyframes：滑动窗口 slot 的进出规则";
        [LB-KV] "How is memory bounded in streaming mode?").  The frame a page
        held keeps as many visible special tokens as the block's eviction
        flags say (reading R13); its bytes stay in the special stream."""
        moved = 0
        kept = special_tokens_kept(self.cfg, *blk.flags)
        while len(blk.live) > sliding_window:
            p = blk.live.popleft()
            blk.spec_vis[blk.frame_of.pop(p)] = kept
            blk.free.append(p)                     # reading R1: return to tail
            moved += 1
        if moved:
            blk.last = None                        # reading R11
        return moved

    def evict_frames(self, b, scale_frames, sliding_window,
                     cross_frame_special=1, camera_only=0):
        """evict_frames(block_idx, scale_frames, sliding_window, ...).

        [LB-KV] "Append and Evict API" / "Streaming Forward Pass".  Scale pages
        and the special stream's bytes are never evicted ([LB-SLOT] "scale
        frames" and "特殊 token 流").  While eviction is deferred this moves
        nothing ([LB-PERF] "Deferred Eviction Strategy").  The flags (each 0
        or 1) say what of an evicted frame's special tokens stays visible
        (special_tokens_kept); the block records them, and a later
        execute_deferred_eviction, which takes none, uses them (reading R13).
        Returns the number of pages moved.
        """
        self._check_block(b)
        if cross_frame_special not in (0, 1) or camera_only not in (0, 1):
            raise OracleError("INVALID_ARG")
        self._check_evict_args(scale_frames, sliding_window)
        blk = self.blocks[b]
        blk.flags = (cross_frame_special, camera_only)
        if self.defer:
            return 0
        return self._evict_to(blk, sliding_window)

    def set_defer_eviction(self, enable):
        """_set_defer_eviction(True/False) ([LB-SLOT] "进阶：光流关键帧与回滚机制";
        [LB-PERF] "Deferred Eviction for Keyframe Decisions")."""
        self.defer = bool(enable)

    def execute_deferred_eviction(self, b, scale_frames, sliding_window):
        """execute_deferred_eviction(block_idx, scale_frames, sliding_window):
        perform the eviction that deferral held back, whatever the flag says
        ([LB-SLOT] "进阶：光流关键帧与回滚机制"), with the special-token flags of
        the block's last evict_frames call (reading R13)."""
        self._check_block(b)
        self._check_evict_args(scale_frames, sliding_window)
        return self._evict_to(self.blocks[b], sliding_window)

    def rollback_last_frame(self, b):
        """rollback_last_frame(block_idx): undo the last append exactly.

        [LB-SLOT] "进阶：光流关键帧与回滚机制": the patch page goes back to the
        free list, the special count and the frame count drop by one, and the
        slot is restored.  Legal only while nothing has moved since that append
        (reading R11).  Pool bytes are left as written (reading R16).
        """
        self._check_block(b)
        blk = self.blocks[b]
        if blk.last is None:
            raise OracleError("NOTHING_TO_ROLLBACK")
        p, where = blk.last
        lst = blk.scale if where == "scale" else blk.live
        assert lst[-1] == p
        lst.pop()
        blk.free.appendleft(p)          # reading R1: back to the head
        del blk.frame_of[p]
        blk.spec_vis.pop()
        blk.nsf -= 1
        blk.last = None
        return p

    def reset(self):
        """clean_kv_cache(): every block back to its initial state, deferral off
        and no plan ([LB-SLOT] "窗口模式：window_size 数的是 slot 不是帧").
        Pool bytes are not touched."""
        m = self.cfg.num_patch_pages
        self.blocks = [_Block(m) for _ in range(self.cfg.num_blocks)]
        self.defer = False
        self.plan_state = None

    def plan(self):
        """plan() on block 0 for this frame step.

        [LB-KV] "Patch Pages vs. Special Pages": visible order scale -> live
        window -> special, specials last.  [LB-KV] "Physical Page Layout and
        Indexing": last_page_len is the number of valid tokens in the final,
        possibly partly filled, special page.  [LB-PERF] "One-Time Planning
        Pattern": built once on block 0 and reused by every block.
        Special pages none of whose tokens is visible any more (reading R13)
        are left out of the table; the newest frame is always resident, so the
        stream's last page, the one last_page_len describes, always stays.
        """
        c = self.cfg
        blk = self.blocks[0]
        if blk.nsf == 0:
            raise OracleError("EMPTY")
        fpp = c.frames_per_special_page
        n_sp = -(-blk.nsf // fpp)
        specials = [c.num_patch_pages + i for i in range(n_sp)
                    if any(blk.spec_vis[i * fpp:(i + 1) * fpp])]
        assert specials[-1] == c.num_patch_pages + n_sp - 1
        table = list(blk.scale) + list(blk.live) + specials
        last_page_len = c.num_special_tokens * (blk.nsf - fpp * (n_sp - 1))
        self.plan_state = Plan(
            table=table,
            n_patch=len(blk.scale) + len(blk.live),
            last_page_len=last_page_len,
            scale=tuple(blk.scale),
            live=tuple(blk.live),
            nsf=blk.nsf,
            spec_vis=tuple(blk.spec_vis),
        )
        return self.plan_state

    def check_run(self, b):
        """The preconditions of run(block): a plan exists and block b holds the
        state the plan was built from (reading R14)."""
        self._check_block(b)
        pl = self.plan_state
        if pl is None:
            raise OracleError("NOT_PLANNED")
        blk = self.blocks[b]
        if (tuple(blk.scale) != pl.scale or tuple(blk.live) != pl.live
                or blk.nsf != pl.nsf or tuple(blk.spec_vis) != pl.spec_vis):
            raise OracleError("STALE_PLAN")
        return pl

    def get_cache_stats(self, b):
        """get_cache_stats(block_idx) -> (frame_count, scale_pages, live_pages,
        free_pages, special_tokens) ([LB-SLOT] "动手验证：查看你的 KV 缓存占用")."""
        self._check_block(b)
        blk = self.blocks[b]
        return (blk.nsf, len(blk.scale), len(blk.live), len(blk.free),
                self.cfg.num_special_tokens * blk.nsf)

    def block_state(self, b):
        """(scale, live, free, nsf) as plain lists, for comparisons."""
        self._check_block(b)
        blk = self.blocks[b]
        return list(blk.scale), list(blk.live), list(blk.free), blk.nsf

    def special_visibility(self, b):
        """Block b's spec_vis as runs [first frame, frames, visible tokens per
        frame] of equal counts, frames with none left out."""
        self._check_block(b)
        return special_runs(self.blocks[b].spec_vis)


def special_runs(spec_vis):
    """A per-frame visible-special count list as runs of equal counts:
    [first frame, number of frames, count], runs with count 0 omitted."""
    runs = []
    for f, n in enumerate(spec_vis):
        if runs and runs[-1][2] == n and runs[-1][0] + runs[-1][1] == f:
            runs[-1][1] += 1
        elif n:
            runs.append([f, 1, n])
    return runs


def visible_tokens_closed_form(cfg, committed, own=False, kept=None):
    """Visible valid tokens after `committed` frames are in the cache and
    evicted to the window, plus an optional own (pending) frame.

    Follows from the routing and window rules: the first S frames stay, at
    most W later ones are live; a frame whose patch page is held keeps its
    special tokens, an evicted one keeps ``kept`` of them (all by default,
    reading R13).
    """
    s, w = cfg.scale_frames, cfg.sliding_window
    k = committed
    if kept is None:
        kept = cfg.num_special_tokens
    n_patch_frames = min(k, s) + min(max(k - s, 0), w)
    n = (cfg.patch_tokens + cfg.num_special_tokens) * n_patch_frames
    n += kept * (k - n_patch_frames)
    if own:
        n += cfg.patch_tokens + cfg.num_special_tokens
    return n


def window_mode_frames(window_size, scale_frames, keyframe_interval):
    """Frames covered by one window in window mode: scale slots hold one frame
    each, every other slot stands for keyframe_interval frames ([LB-SLOT]
    "窗口模式": 128 slots = 8 scale + 120 keyframes, interval 13 -> 1568)."""
    return scale_frames + (window_size - scale_frames) * keyframe_interval


def ceil_div(a, b):
    return -(-a // b)


__all__ = [
    "ERRORS", "OracleError", "OracleConfig", "Plan", "PagePoolOracle",
    "special_tokens_kept", "special_runs", "visible_tokens_closed_form",
    "window_mode_frames", "ceil_div",
]
