"""Seeded synthetic inputs shared by the tests, the smoke run and the benchmark.

This package holds none of the method's arithmetic: it only draws Q, K and V
for a (stream, frame, block) triple and the keyframe-acceptance coin flips of
the dynamic-keyframe stream.  Both the HIP path and the CPU oracle are fed the
very same tensors.

Workload recipes (synthetic stand-ins for the unnamed video streams the pages
measure on):

========  =====================================================================
tiny      1 block, H=4, D=64, 16 patch + 6 special tokens, page 16, S/W/R 2/4/2,
          special pool for 32 frames; 12 frames, all keyframes
224x224   24 blocks, H=16, D=64, 256 patch tokens, page 256, S/W/R 8/64/16,
          special pool for 2048 frames; 200 frames, all keyframes
518x378   24 blocks, H=16, D=64, 999 patch tokens, page 999 (exact) or 1024
          (padded), S/W/R 8/64/16, special pool for 2048 frames; keyframe
          interval 2; K drawn at half scale
dynamic   as 518x378 exact but S/W/R 8/120/16; every frame is appended under
          deferred eviction, then accepted or rolled back by a Bernoulli(0.4)
          draw, forced accept after 12 rejects in a row
========  =====================================================================

Values are N(0, 1) drawn in float32 and rounded to bf16 by torch.
"""

from dataclasses import dataclass, replace

import numpy as np
import torch

_MASK64 = (1 << 64) - 1


def _mix64(x):
    """splitmix64 finaliser (Steele, Lea, Flood 2014): spreads a counter into
    an unrelated 64-bit seed."""
    x = (x + 0x9E3779B97F4A7C15) & _MASK64
    x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & _MASK64
    return x ^ (x >> 31)


def seed_for(*parts):
    """Deterministic 63-bit seed from a tuple of small non-negative ints."""
    h = 0x2545F4914F6CDD1D
    for p in parts:
        h = _mix64(h ^ (int(p) & _MASK64))
    return h & ((1 << 63) - 1)


TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    name: str
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
    frames: int
    keyframe_interval: int = 1     # 1: every frame is a keyframe
    dynamic: bool = False          # deferred append + Bernoulli accept/rollback
    accept_prob: float = 0.4
    max_rejects: int = 12
    reset_every: int = 0           # 0: never reset
    k_scale: float = 1.0
    seed: int = 0

    @property
    def tokens_per_frame(self):
        return self.num_special_tokens + self.patch_tokens

    def cfg_kwargs(self):
        return dict(
            num_blocks=self.num_blocks, num_heads=self.num_heads,
            head_dim=self.head_dim, page_size=self.page_size,
            patch_tokens=self.patch_tokens,
            num_special_tokens=self.num_special_tokens,
            scale_frames=self.scale_frames, sliding_window=self.sliding_window,
            headroom=self.headroom, max_total_frames=self.max_total_frames)

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 4, 64, 16, 16, 6, 2, 4, 2, 32, 12, seed=1),
    "224x224": Workload("224x224", 24, 16, 64, 256, 256, 6, 8, 64, 16, 2048,
                        200, seed=2),
    "518x378": Workload("518x378", 24, 16, 64, 999, 999, 6, 8, 64, 16, 2048,
                        600, keyframe_interval=2, k_scale=0.5, seed=3),
    "518x378-padded": Workload("518x378-padded", 24, 16, 64, 1024, 999, 6, 8,
                               64, 16, 2048, 4096, keyframe_interval=2,
                               k_scale=0.5, seed=4),
    "dynamic": Workload("dynamic", 24, 16, 64, 999, 999, 6, 8, 120, 16, 2048,
                        1000, dynamic=True, reset_every=1568, seed=5),
}


def frame_qkv(wl, frame, block, device="cpu", which=(TENSOR_Q, TENSOR_K, TENSOR_V),
              nq=None):
    """Q, K, V of one (frame, block): bf16 [tokens_per_frame, H, D] each.

    Drawn with a torch generator on ``device`` seeded from (workload seed,
    frame, block, tensor id); the same call gives the same tensors.
    """
    n = wl.tokens_per_frame if nq is None else nq
    shape = (n, wl.num_heads, wl.head_dim)
    out = []
    for t in which:
        g = torch.Generator(device=device)
        g.manual_seed(seed_for(wl.seed, frame, block, t))
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if t == TENSOR_K and wl.k_scale != 1.0:
            x = x * wl.k_scale
        out.append(x.to(torch.bfloat16))
    return tuple(out)


def bf16_bits(t):
    """A bf16 torch tensor as a numpy uint16 array of its bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def is_keyframe(wl, frame):
    """Fixed-interval schedule: frame i is a keyframe iff i % interval == 0."""
    return frame % wl.keyframe_interval == 0


def accept_decisions(wl, frames=None):
    """Accept/reject coin flips of the dynamic stream.

    numpy default_rng(seed); a frame is accepted when 12 rejects in a row came
    before it, else iff the draw is below accept_prob (every frame draws).
    """
    n = wl.frames if frames is None else frames
    rng = np.random.default_rng(wl.seed)
    out, rejects = [], 0
    for _ in range(n):
        u = rng.random()
        if rejects >= wl.max_rejects:
            acc = True
        else:
            acc = bool(u < wl.accept_prob)
        rejects = 0 if acc else rejects + 1
        out.append(acc)
    return out
