"""CPU oracle for streaming two-stream paged-KV attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (no headers, helpers, tables or constants); both sides only see
the same seeded inputs, produced by the separate ``synth`` package.

What it computes, and where the pages say so
--------------------------------------------
The pages are cited by title and section:

* [LB-KV]   "How LingBot-Map Implements the KV Cache Mechanism for Streaming
            Inference with FlashInfer Integration" (instagit.com)
* [LB-PERF] "How to Improve Streaming Inference Performance with FlashInfer KV
            Cache Backend" (instagit.com)
* [LB-SLOT] "LingBot-Map KV缓存机制深度揭秘：scale frames与keyframes如何占用slot"
            (mhpq.cn) -- a Chinese deep dive on how scale frames and keyframes
            occupy cache slots.

Modules
-------
``pagepool``   Part 1: the page-pool state machine (scale list, live-window
               deque, free list, append-only special stream, deferred
               eviction, rollback, reset, plan, stats) and the byte-level pool.
``attention``  Part 2: gather of the visible K/V through a plan, then the plain
               definition of softmax attention in float64.
``brute``      Part 3: an independent page-free model of which tokens a frame
               sees, used to pin Parts 1 and 2 on small streams.
``bf16``       exact bf16 <-> float64 conversion of stored bit patterns.

Pins (see tests/test_oracle_*.py): the constants the pages print (6 special
tokens in the order camera, 4 registers, scale; 8 + 64 + 16 = 88 patch pages;
42 frames per 256-token special page; 8 + 120 x 13 = 1568 frames per window;
healthy stats), closed forms for the visible token count and special-page
packing, state invariants, the brute-force model, attention special cases and a
library cross-check of the dense attention.  No function here is "parity
unpinned".
"""

from .pagepool import (  # noqa: F401
    OracleConfig,
    OracleError,
    PagePoolOracle,
    Plan,
)
from .attention import (  # noqa: F401
    gather_visible, dense_attention, paged_attention, paged_attention_with_own)
from .brute import BruteForceStream  # noqa: F401
from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits  # noqa: F401
