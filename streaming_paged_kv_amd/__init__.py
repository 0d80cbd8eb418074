"""Streaming two-stream paged-KV attention for MI355X (gfx950).

A thin ctypes binding over libspkv.so (C ABI in include/spkv.h).  Every step
of the hot path -- page allocation, the append copy, the plan and the
attention -- runs in the library; this module only marshals arguments and
uses torch for device memory (the pools and the workspace) and streams.

The methods mirror the KV-cache manager the pages describe ("How LingBot-Map
Implements the KV Cache Mechanism for Streaming Inference with FlashInfer
Integration", sections "Append and Evict API" and "Kernel-Level Execution
Flow"; "How to Improve Streaming Inference Performance with FlashInfer KV
Cache Backend", "Deferred Eviction Strategy"; "LingBot-Map KV缓存机制深度揭秘",
sections on rollback, window mode and get_cache_stats):

    cache = PagedKVCache(num_blocks=24, num_heads=16, head_dim=64,
                         page_size=999, patch_tokens=999, ...)
    for b in range(24):
        cache.append_frame(b, k[b], v[b])
        cache.evict_frames(b, 8, 64)
        if b == 0:
            cache.plan()
        out[b] = cache.run(b, q[b])

Set SPKV_DEBUG_KV=N to print every block's page occupancy every N plans.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspkv.so")

ERROR_NAMES = {
    0: "OK",
    -1: "INVALID_ARG",
    -2: "BAD_BLOCK",
    -3: "POOL_EXHAUSTED",
    -4: "SPECIAL_OVERFLOW",
    -5: "NOTHING_TO_ROLLBACK",
    -6: "EMPTY",
    -7: "NOT_PLANNED",
    -8: "STALE_PLAN",
    -9: "UNSUPPORTED",
    -10: "HIP",
    -11: "WORKSPACE",
}

# Symbols the header declares (checked by the CPU tests).
EXPORTED = (
    "spkv_query_sizes", "spkv_query_workspace", "spkv_create", "spkv_destroy", "spkv_append_frame",
    "spkv_append_frame_in_run",
    "spkv_evict_frames", "spkv_set_defer_eviction",
    "spkv_execute_deferred_eviction", "spkv_rollback_last_frame", "spkv_reset",
    "spkv_plan", "spkv_run", "spkv_run_noalloc", "spkv_run_own", "spkv_run_batch", "spkv_set_num_splits",
    "spkv_get_cache_stats",
    "spkv_get_plan", "spkv_get_plan_specials", "spkv_get_block_specials",
    "spkv_get_block_state", "spkv_error_string",
)


class SpkvError(RuntimeError):
    def __init__(self, code, call):
        self.code = code
        self.name = ERROR_NAMES.get(code, str(code))
        super().__init__(f"{call}: SPKV_ERR_{self.name} ({code})")


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_blocks", "num_heads", "head_dim", "page_size", "patch_tokens",
        "num_special_tokens", "scale_frames", "sliding_window", "headroom",
        "max_total_frames")]


class Request(ctypes.Structure):
    """spkv_request: one stream's run (or run_own) inside spkv_run_batch."""
    _fields_ = [("handle", ctypes.c_void_p), ("block", ctypes.c_int32),
                ("nq", ctypes.c_int32), ("q", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("own_k", ctypes.c_void_p), ("own_v", ctypes.c_void_p),
                ("sm_scale", ctypes.c_float)]


MAX_BATCH = 16


class Stats(ctypes.Structure):
    _fields_ = [("frame_count", ctypes.c_int64), ("scale_pages", ctypes.c_int32),
                ("live_pages", ctypes.c_int32), ("free_pages", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("special_tokens", ctypes.c_int64)]


_lib = None


def load_library(path=None):
    """Load libspkv.so.  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(
            f"{p} is missing: build it with `python -m streaming_paged_kv_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    pi32, pi64 = ctypes.POINTER(i32), ctypes.POINTER(i64)
    sig = {
        "spkv_query_sizes": [ctypes.POINTER(Config), pi64, pi64, pi64],
        "spkv_query_workspace": [ctypes.POINTER(Config), i32, i32, pi64],
        "spkv_create": [ctypes.POINTER(Config), ctypes.POINTER(vp), vp, i64,
                        ctypes.POINTER(vp)],
        "spkv_destroy": [vp],
        "spkv_append_frame": [vp, i32, vp, vp, vp],
        "spkv_append_frame_in_run": [vp, i32, vp, vp, vp],
        "spkv_evict_frames": [vp, i32, i32, i32, i32, i32],
        "spkv_set_defer_eviction": [vp, i32],
        "spkv_execute_deferred_eviction": [vp, i32, i32, i32],
        "spkv_rollback_last_frame": [vp, i32],
        "spkv_reset": [vp],
        "spkv_plan": [vp, vp],
        "spkv_run": [vp, i32, vp, vp, i32, ctypes.c_float, vp],
        "spkv_run_noalloc": [vp, i32, vp, vp, i32, ctypes.c_float, vp],
        "spkv_run_own": [vp, i32, vp, vp, i32, ctypes.c_float, vp, vp, vp],
        "spkv_run_batch": [ctypes.POINTER(Request), i32, vp],
        "spkv_set_num_splits": [vp, i32],
        "spkv_get_cache_stats": [vp, i32, ctypes.POINTER(Stats)],
        "spkv_get_plan": [vp, pi32, i32, pi32, pi32, pi32],
        "spkv_get_plan_specials": [vp, pi32, i32, pi32],
        "spkv_get_block_specials": [vp, i32, pi32, i32, pi32],
        "spkv_get_block_state": [vp, i32, pi32, pi32, pi32, i32, pi32, pi32,
                                 pi32, pi64],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.spkv_error_string.argtypes = [ctypes.c_int]
    lib.spkv_error_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(code, call):
    if code != 0:
        raise SpkvError(code, call)


def _stream_ptr(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def make_config(**kw):
    c = Config()
    for name, _ in Config._fields_:
        setattr(c, name, int(kw[name]))
    return c


MAX_SPLITS = 32


def query_workspace(nq, num_splits, **cfg):
    """Workspace bytes that let run() split nq query rows num_splits ways."""
    lib = load_library()
    c = make_config(**cfg)
    out = ctypes.c_int64()
    _check(lib.spkv_query_workspace(ctypes.byref(c), int(nq), int(num_splits),
                                    ctypes.byref(out)), "spkv_query_workspace")
    return out.value


def query_sizes(**cfg):
    """(max_num_pages, pool_bytes_per_block, min_workspace_bytes,
    full_workspace_bytes) of a configuration; the last is the workspace that
    lets run() split one frame's queries the most ways it does (32)."""
    lib = load_library()
    c = make_config(**cfg)
    out = [ctypes.c_int64() for _ in range(3)]
    _check(lib.spkv_query_sizes(ctypes.byref(c), *[ctypes.byref(x) for x in out]),
           "spkv_query_sizes")
    tpf = int(cfg["num_special_tokens"]) + int(cfg["patch_tokens"])
    return tuple(x.value for x in out) + (query_workspace(tpf, MAX_SPLITS, **cfg),)


class PagedKVCache:
    """One manager: per-block pools, the host page-pool state and the plan.

    host_only=True builds the bookkeeping alone (no GPU, no kernels): append
    takes no tensors and run() reports UNSUPPORTED after its checks.
    """

    def __init__(self, *, num_blocks, num_heads, head_dim, page_size,
                 patch_tokens, num_special_tokens=6, scale_frames=8,
                 sliding_window=64, headroom=16, max_total_frames=2048,
                 device=None, host_only=False, workspace_bytes=None):
        self.lib = load_library()
        self.cfg = dict(num_blocks=num_blocks, num_heads=num_heads,
                        head_dim=head_dim, page_size=page_size,
                        patch_tokens=patch_tokens,
                        num_special_tokens=num_special_tokens,
                        scale_frames=scale_frames, sliding_window=sliding_window,
                        headroom=headroom, max_total_frames=max_total_frames)
        self._c = make_config(**self.cfg)
        (self.max_num_pages, self.pool_bytes, self.min_workspace_bytes,
         self.full_workspace_bytes) = query_sizes(**self.cfg)
        self.host_only = host_only
        self.tokens_per_frame = num_special_tokens + patch_tokens
        self.pools = []
        self.workspace = None
        self._h = ctypes.c_void_p()
        if host_only:
            _check(self.lib.spkv_create(ctypes.byref(self._c), None, None, 0,
                                        ctypes.byref(self._h)), "spkv_create")
        else:
            if not torch.cuda.is_available():
                raise RuntimeError("PagedKVCache needs a GPU (or host_only=True)")
            self.device = torch.device(device) if device is not None else \
                torch.device("cuda", torch.cuda.current_device())
            shape = (self.max_num_pages, 2, page_size, num_heads, head_dim)
            self.pools = [torch.zeros(shape, dtype=torch.bfloat16, device=self.device)
                          for _ in range(num_blocks)]
            ws = self.full_workspace_bytes if workspace_bytes is None else workspace_bytes
            self.workspace = torch.empty(ws, dtype=torch.uint8, device=self.device)
            ptrs = (ctypes.c_void_p * num_blocks)(*[p.data_ptr() for p in self.pools])
            with torch.cuda.device(self.device):
                _check(self.lib.spkv_create(ctypes.byref(self._c), ptrs,
                                            ctypes.c_void_p(self.workspace.data_ptr()),
                                            ws, ctypes.byref(self._h)), "spkv_create")
        self._held = {}   # frames whose copy append_frame_in_run left to a later call
        dbg = os.environ.get("SPKV_DEBUG_KV", "")
        self._debug_every = int(dbg) if dbg.isdigit() and int(dbg) > 0 else 0
        self._plans = 0

    # ----------------------------------------------------------- lifecycle
    def close(self):
        if self._h:
            _check(self.lib.spkv_destroy(self._h), "spkv_destroy")
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # --------------------------------------------------------------- checks
    def _frame_tensor(self, t, name, rows):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 \
                or not t.is_contiguous() or t.device != self.device:
            raise ValueError(f"{name} must be a contiguous bf16 tensor on {self.device}")
        if tuple(t.shape) != (rows, self.cfg["num_heads"], self.cfg["head_dim"]):
            raise ValueError(f"{name} has shape {tuple(t.shape)}")
        return ctypes.c_void_p(t.data_ptr())

    # ------------------------------------------------------------ the calls
    def append_frame(self, block, k=None, v=None, stream=None):
        if self.host_only:
            _check(self.lib.spkv_append_frame(self._h, block, None, None, None),
                   "spkv_append_frame")
            return
        kp = self._frame_tensor(k, "k", self.tokens_per_frame)
        vp = self._frame_tensor(v, "v", self.tokens_per_frame)
        _check(self.lib.spkv_append_frame(self._h, block, kp, vp, _stream_ptr(stream)),
               "spkv_append_frame")

    def append_frame_in_run(self, block, k=None, v=None, stream=None):
        """append_frame whose copy into the pool is done by this block's next
        run() (inside the attention launch), or earlier by a plain copy when
        another call needs the bytes first.  k and v are kept referenced here
        until the block's next append, so they stay valid for that copy."""
        if self.host_only:
            _check(self.lib.spkv_append_frame_in_run(self._h, block, None, None, None),
                   "spkv_append_frame_in_run")
            return
        kp = self._frame_tensor(k, "k", self.tokens_per_frame)
        vp = self._frame_tensor(v, "v", self.tokens_per_frame)
        _check(self.lib.spkv_append_frame_in_run(self._h, block, kp, vp,
                                                 _stream_ptr(stream)),
               "spkv_append_frame_in_run")
        self._held[block] = (k, v)

    def evict_frames(self, block, scale_frames, sliding_window,
                     cross_frame_special=1, camera_only=0):
        _check(self.lib.spkv_evict_frames(self._h, block, scale_frames, sliding_window,
                                          int(cross_frame_special), int(camera_only)),
               "spkv_evict_frames")

    def set_defer_eviction(self, enable):
        _check(self.lib.spkv_set_defer_eviction(self._h, 1 if enable else 0),
               "spkv_set_defer_eviction")

    def execute_deferred_eviction(self, block, scale_frames, sliding_window):
        _check(self.lib.spkv_execute_deferred_eviction(self._h, block, scale_frames,
                                                       sliding_window),
               "spkv_execute_deferred_eviction")

    def rollback_last_frame(self, block):
        _check(self.lib.spkv_rollback_last_frame(self._h, block),
               "spkv_rollback_last_frame")

    def reset(self):
        _check(self.lib.spkv_reset(self._h), "spkv_reset")

    clean_kv_cache = reset

    def plan(self, stream=None):
        s = None if self.host_only else _stream_ptr(stream)
        _check(self.lib.spkv_plan(self._h, s), "spkv_plan")
        self._plans += 1
        if self._debug_every and self._plans % self._debug_every == 0:
            for b in range(self.cfg["num_blocks"]):
                st = self.get_cache_stats(b)
                print(f"[spkv] plan {self._plans} block {b}: scale_pg={st[1]} "
                      f"live_pg={st[2]} free_pg={st[3]} special={st[4]}", flush=True)

    def run(self, block, q=None, out=None, sm_scale=None, nq=None, stream=None):
        if sm_scale is None:
            sm_scale = self.cfg["head_dim"] ** -0.5
        if self.host_only:
            n = self.tokens_per_frame if nq is None else nq
            _check(self.lib.spkv_run(self._h, block, None, None, n, sm_scale, None),
                   "spkv_run")
            return None
        n = q.shape[0] if nq is None else nq
        qp = self._frame_tensor(q, "q", n)
        if out is None:
            out = torch.empty_like(q)
        op = self._frame_tensor(out, "out", n)
        _check(self.lib.spkv_run(self._h, block, qp, op, n, float(sm_scale),
                                 _stream_ptr(stream)), "spkv_run")
        return out

    def run_noalloc(self, block, q=None, out=None, sm_scale=None, nq=None, stream=None):
        """run() with the split partials in the library's own device memory
        (spkv_run_noalloc): nothing is allocated, and the handle's workspace
        need only be the minimum.  Calls on one GPU share that memory."""
        if sm_scale is None:
            sm_scale = self.cfg["head_dim"] ** -0.5
        if self.host_only:
            n = self.tokens_per_frame if nq is None else nq
            _check(self.lib.spkv_run_noalloc(self._h, block, None, None, n, sm_scale, None),
                   "spkv_run_noalloc")
            return None
        n = q.shape[0] if nq is None else nq
        qp = self._frame_tensor(q, "q", n)
        if out is None:
            out = torch.empty_like(q)
        op = self._frame_tensor(out, "out", n)
        _check(self.lib.spkv_run_noalloc(self._h, block, qp, op, n, float(sm_scale),
                                         _stream_ptr(stream)), "spkv_run_noalloc")
        return out

    def run_own(self, block, q=None, k=None, v=None, out=None, sm_scale=None, nq=None,
                stream=None):
        """Attention over the planned pages plus the caller's own frame k, v
        (the layout append_frame takes), without storing them: a non-keyframe
        that skips the append."""
        if sm_scale is None:
            sm_scale = self.cfg["head_dim"] ** -0.5
        if self.host_only:
            n = self.tokens_per_frame if nq is None else nq
            _check(self.lib.spkv_run_own(self._h, block, None, None, n, sm_scale, None,
                                         None, None), "spkv_run_own")
            return None
        n = q.shape[0] if nq is None else nq
        qp = self._frame_tensor(q, "q", n)
        kp = self._frame_tensor(k, "k", self.tokens_per_frame)
        vp = self._frame_tensor(v, "v", self.tokens_per_frame)
        if out is None:
            out = torch.empty_like(q)
        op = self._frame_tensor(out, "out", n)
        _check(self.lib.spkv_run_own(self._h, block, qp, op, n, float(sm_scale), kp, vp,
                                     _stream_ptr(stream)), "spkv_run_own")
        return out

    def set_num_splits(self, n):
        _check(self.lib.spkv_set_num_splits(self._h, n), "spkv_set_num_splits")

    # ---------------------------------------------------------- inspection
    def get_cache_stats(self, block):
        s = Stats()
        _check(self.lib.spkv_get_cache_stats(self._h, block, ctypes.byref(s)),
               "spkv_get_cache_stats")
        return (s.frame_count, s.scale_pages, s.live_pages, s.free_pages,
                s.special_tokens)

    def get_plan(self):
        cap = self.max_num_pages
        tab = (ctypes.c_int32 * cap)()
        n, npatch, lpl = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(self.lib.spkv_get_plan(self._h, tab, cap, ctypes.byref(n),
                                      ctypes.byref(npatch), ctypes.byref(lpl)),
               "spkv_get_plan")
        return list(tab[:n.value]), npatch.value, lpl.value

    def _specials(self, fn, name, *args):
        n = ctypes.c_int32()
        _check(fn(self._h, *args, None, 0, ctypes.byref(n)), name)
        buf = (ctypes.c_int32 * max(1, 3 * n.value))()
        _check(fn(self._h, *args, buf, n.value, ctypes.byref(n)), name)
        return [list(buf[3 * i:3 * i + 3]) for i in range(n.value)]

    def get_plan_specials(self):
        """The plan's visible special tokens: [first frame, frames, tokens
        per frame] runs in stream order."""
        return self._specials(self.lib.spkv_get_plan_specials, "spkv_get_plan_specials")

    def get_block_specials(self, block):
        """The same runs for a block's current state."""
        return self._specials(self.lib.spkv_get_block_specials, "spkv_get_block_specials",
                              block)

    def get_block_state(self, block):
        cap = self.max_num_pages
        sc, lv, fr = ((ctypes.c_int32 * cap)() for _ in range(3))
        ns, nl, nf = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        nsf = ctypes.c_int64()
        _check(self.lib.spkv_get_block_state(self._h, block, sc, lv, fr, cap,
                                             ctypes.byref(ns), ctypes.byref(nl),
                                             ctypes.byref(nf), ctypes.byref(nsf)),
               "spkv_get_block_state")
        return list(sc[:ns.value]), list(lv[:nl.value]), list(fr[:nf.value]), nsf.value


class Batch:
    """The marshalled requests of one spkv_run_batch call; launch() makes it.

    requests: sequence of dicts with keys cache (a PagedKVCache), block, q and
    optionally out, k and v (the caller's own frame, as for run_own), sm_scale
    and nq.  Host-only caches pass no tensors.  outs holds the output tensors,
    in order (None for host-only caches).
    """

    def __init__(self, requests):
        requests = list(requests)
        self.lib = load_library()
        self.n = len(requests)
        self.arr = (Request * max(1, self.n))()
        self.outs = []
        self.host_only = not requests or requests[0]["cache"].host_only
        self._keep = requests
        for i, r in enumerate(requests):
            c = r["cache"]
            sm = r.get("sm_scale")
            if sm is None:
                sm = c.cfg["head_dim"] ** -0.5
            a = self.arr[i]
            a.handle = c._h
            a.block = r["block"]
            a.sm_scale = float(sm)
            if c.host_only:
                a.nq = c.tokens_per_frame if r.get("nq") is None else r["nq"]
                self.outs.append(None)
                continue
            q = r["q"]
            n = q.shape[0] if r.get("nq") is None else r["nq"]
            a.nq = n
            a.q = c._frame_tensor(q, "q", n)
            out = r.get("out")
            if out is None:
                out = torch.empty_like(q)
            a.out = c._frame_tensor(out, "out", n)
            if r.get("k") is not None or r.get("v") is not None:
                a.own_k = c._frame_tensor(r.get("k"), "k", c.tokens_per_frame)
                a.own_v = c._frame_tensor(r.get("v"), "v", c.tokens_per_frame)
            self.outs.append(out)

    def launch(self, stream=None):
        s = None if self.host_only else _stream_ptr(stream)
        _check(self.lib.spkv_run_batch(self.arr, self.n, s), "spkv_run_batch")
        return self.outs


def run_batch(requests, stream=None):
    """Several streams' runs in one launch (spkv_run_batch); see Batch.
    Returns the outputs, in order (None for host-only caches)."""
    return Batch(requests).launch(stream)
