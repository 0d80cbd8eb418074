"""spkv_run_noalloc, through the C ABI, against spkv_run on the same handle
state: the same attention with the key-range split's partials in the
library's own device array instead of the handle's workspace.

Two calls in a row, the second with fewer query rows.  With the same split
count the two entry points launch the same kernels on the same inputs, so
their outputs are bit-identical; a handle holding only the minimum workspace
cannot split in run() but still splits in run_noalloc(), and both stay
within the tolerance of the float64 oracle.  A query count beyond the
array's limit is refused with nothing written."""

import numpy as np
import pytest
import torch

import harness as H
import synth
from oracle import OracleConfig, PagePoolOracle
from oracle.attention import paged_attention

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _stream(wl, caches, o):
    for f in range(wl.frames):
        q, k, v = synth.frame_qkv(wl, f, 0, device=DEV)
        for c in caches:
            c.append_frame(0, k, v)
            c.evict_frames(0, wl.scale_frames, wl.sliding_window)
        o.append_frame(0, synth.bf16_bits(k), synth.bf16_bits(v))
        o.evict_frames(0, wl.scale_frames, wl.sliding_window)
    for c in caches:
        c.plan()
    return o.plan()


def test_run_noalloc_matches_run():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import streaming_paged_kv_amd as spkv
    wl = synth.WORKLOADS["518x378"].with_(name="noalloc", num_blocks=1, keyframe_interval=1,
                                          frames=24)
    cfg = OracleConfig(**wl.cfg_kwargs())
    o = PagePoolOracle(cfg, track_pool=[0])
    full = spkv.PagedKVCache(**wl.cfg_kwargs())
    lean = spkv.PagedKVCache(**wl.cfg_kwargs(),
                             workspace_bytes=spkv.query_sizes(**wl.cfg_kwargs())[2])
    pl = _stream(wl, (full, lean), o)
    sm = 0.125
    # the second call has fewer rows: one query tile instead of two
    for call, nq in enumerate((wl.tokens_per_frame, 300)):
        q = synth.frame_qkv(wl, 100 + call, 0, device=DEV)[0][:nq].contiguous()
        print(f"  run_noalloc call {call}: nq {nq}", flush=True)
        ref = paged_attention(o.pools[0], pl, cfg, synth.bf16_bits(q), sm)
        out_run = full.run(0, q, sm_scale=sm)
        out_na = full.run_noalloc(0, q, sm_scale=sm)
        out_lean_na = lean.run_noalloc(0, q, sm_scale=sm)
        out_lean_run = lean.run(0, q, sm_scale=sm)       # no room to split
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_run), call
        assert torch.equal(out_lean_na, out_run), call
        for out in (out_run, out_na, out_lean_na, out_lean_run):
            H.compare(out, ref, ("noalloc", call, nq))
        # forced splits: both entry points honour them alike
        for sp in (3, 11):
            full.set_num_splits(sp)
            a = full.run(0, q, sm_scale=sm)
            b = full.run_noalloc(0, q, sm_scale=sm)
            torch.cuda.synchronize()
            assert torch.equal(a, b), (call, sp)
            H.compare(b, ref, ("noalloc forced", call, sp))
        full.set_num_splits(0)
    # beyond the array's limit (two splits of 16-head rows, each row's
    # partial a bf16 O of 64 dims and an fp32 (m, l)): refused, nothing written
    limit = (48 << 20) // (2 * 16 * (64 * 2 + 8))
    assert limit == 11565
    q = torch.zeros((limit + 1, 16, 64), dtype=torch.bfloat16, device=DEV)
    out = torch.full_like(q, 7.0)
    with pytest.raises(spkv.SpkvError) as ei:
        full.run_noalloc(0, q, out=out)
    assert ei.value.name == "WORKSPACE"
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    q = synth.frame_qkv(wl, 200, 0, device=DEV, nq=limit)[0]
    out = full.run_noalloc(0, q, sm_scale=sm)
    torch.cuda.synchronize()
    rows = H.sample_rows(limit, seed=4)
    ref = paged_attention(o.pools[0], pl, cfg, synth.bf16_bits(q[rows]), sm)
    H.compare(out[rows], ref, ("noalloc at the limit", limit))
    full.close()
    lean.close()
