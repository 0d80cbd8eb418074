"""Part 3 of the oracle: a page-free model of what a frame attends to.

TEST INFRASTRUCTURE ONLY (see the package docstring for the page tags).

This model keeps whole frames, not pages, and states the visibility rule in
terms of frames only, so it checks Part 1 (routing, eviction, packing, the
plan) and Part 2 (the gather) together:

* the first S committed frames are anchors whose patch tokens stay forever
  ([LB-SLOT] "scale frames：永不驱逐的前 8 个 slot");
* of the later committed frames, the most recent W keep their patch tokens
  ([LB-SLOT] "keyframes：滑动窗口 slot 的进出规则");
* every committed frame keeps its special tokens, and they come after all
  patch tokens ([LB-SLOT] "特殊 token 流"; [LB-KV] "Patch Pages vs. Special
  Pages") -- except that a frame whose patch tokens have left keeps only the
  first ``kept`` of them when the stream's eviction flags say so ([LB-KV]
  "Append and Evict API", specials optionally preserved; reading R13);
* a frame that is not (yet) committed -- a non-keyframe, or a frame whose
  keyframe decision is pending under deferred eviction -- attends to the cache
  plus its own K/V ([LB-SLOT] "keyframes" table, non-keyframe row; reading R6):
  its patch tokens follow the committed patch tokens and its special tokens
  follow the committed special tokens.

Frames are [num_special + patch_tokens, H, D] float64 arrays in token order
[camera, register x4, scale, patch...].
"""

import numpy as np

from .attention import dense_attention


class BruteForceStream:
    def __init__(self, scale_frames, sliding_window, num_special_tokens, kept=None):
        self.s = scale_frames
        self.w = sliding_window
        self.ns = num_special_tokens
        self.kept = num_special_tokens if kept is None else kept
        self.committed_k = []
        self.committed_v = []

    def commit(self, k, v):
        """The frame becomes part of the cache (a keyframe, or an accepted
        pending frame)."""
        self.committed_k.append(np.asarray(k, dtype=np.float64))
        self.committed_v.append(np.asarray(v, dtype=np.float64))

    def reset(self):
        self.committed_k.clear()
        self.committed_v.clear()

    def _visible_frames(self):
        n = len(self.committed_k)
        anchors = list(range(min(n, self.s)))
        n_recent = min(self.w, max(n - self.s, 0))
        recent = list(range(n - n_recent, n))
        return anchors + recent

    def visible(self, own_k=None, own_v=None):
        """Visible K, V as float64 [Nk, H, D] in attention order."""
        ns = self.ns
        patch_frames = self._visible_frames()
        ks = [self.committed_k[i][ns:] for i in patch_frames]
        vs = [self.committed_v[i][ns:] for i in patch_frames]
        if own_k is not None:
            ks.append(np.asarray(own_k, dtype=np.float64)[ns:])
            vs.append(np.asarray(own_v, dtype=np.float64)[ns:])
        held = set(patch_frames)
        for i in range(len(self.committed_k)):
            n = ns if i in held else self.kept
            ks.append(self.committed_k[i][:n])
            vs.append(self.committed_v[i][:n])
        if own_k is not None:
            ks.append(np.asarray(own_k, dtype=np.float64)[:ns])
            vs.append(np.asarray(own_v, dtype=np.float64)[:ns])
        return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)

    def attend(self, q, sm_scale, own_k=None, own_v=None):
        k, v = self.visible(own_k, own_v)
        return dense_attention(q, k, v, sm_scale), k.shape[0]
