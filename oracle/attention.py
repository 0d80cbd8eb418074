"""Part 2 of the oracle: attention over the visible pages, by definition.

TEST INFRASTRUCTURE ONLY (see the package docstring for the page tags).

[LB-KV] "Kernel-Level Execution Flow": every block runs scaled dot-product
attention of the frame's queries over the K/V pages the plan lists, with
causal=False, no positional encoding and as many query heads as K/V heads.
The paged kernel reaches the plain definition

    O[i, h, :] = sum_j softmax_j( s * Q[i, h, :] . K[j, h, :] ) V[j, h, :]

over the visible tokens j in table order.  This module gathers those tokens
explicitly (page by page, with the valid length of each page) and evaluates
the definition densely in float64.  The result is exact up to float64 rounding
order; the row chunking only bounds memory and does not change any sum.
"""

import numpy as np

from .bf16 import bf16_bits_to_f64


def gather_visible(pool, plan, cfg):
    """Visible K and V of one block, in table order, as float64 [Nk, H, D].

    ``pool`` is the block's uint16 [max_num_pages, 2, page_size, H, D] array.
    Only the valid slots of each page are read (reading R4/R5): the tail of a
    padded patch page and the unused tail of a special page are never part of
    the sequence ([LB-KV] "Physical Page Layout and Indexing").  Of a special
    page's slots, those of special tokens that eviction took out of view
    (reading R13) are skipped.
    """
    ks, vs = [], []
    for page, slots in zip(plan.table, plan.visible_slots(cfg)):
        ks.append(pool[page, 0, slots])
        vs.append(pool[page, 1, slots])
    k = bf16_bits_to_f64(np.concatenate(ks, axis=0))
    v = bf16_bits_to_f64(np.concatenate(vs, axis=0))
    return k, v


def dense_attention(q, k, v, sm_scale, row_chunk=128):
    """Plain softmax attention in float64.

    q: [Nq, H, D], k and v: [Nk, H, D] (float64).  Returns [Nq, H, D] float64.
    For each head: scores = sm_scale * q_h k_h^T, subtract the row maximum,
    exponentiate, divide by the row sum, multiply by v_h.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nh, _ = q.shape
    out = np.empty((nq, nh, v.shape[2]), dtype=np.float64)
    for h in range(nh):
        kh = k[:, h, :]
        vh = v[:, h, :]
        for r0 in range(0, nq, row_chunk):
            qh = q[r0:r0 + row_chunk, h, :]
            scores = sm_scale * (qh @ kh.T)
            scores -= scores.max(axis=1, keepdims=True)
            p = np.exp(scores)
            p /= p.sum(axis=1, keepdims=True)
            out[r0:r0 + row_chunk, h, :] = p @ vh
    return out


def paged_attention(pool, plan, cfg, q_bits, sm_scale, rows=None):
    """What run(block) computes for one block: gather through the plan, then
    dense attention.  ``q_bits`` is the uint16 [Nq, H, D] query; ``rows``
    optionally selects query rows (each row's result does not depend on the
    others, so a subset is exactly the same rows of the full result)."""
    k, v = gather_visible(pool, plan, cfg)
    q = bf16_bits_to_f64(q_bits)
    if rows is not None:
        q = q[np.asarray(rows)]
    return dense_attention(q, k, v, sm_scale)


def paged_attention_with_own(pool, plan, cfg, q_bits, own_k_bits, own_v_bits, sm_scale,
                             rows=None):
    """What run_own(block) computes: a frame that attends to the cache plus
    its own K/V without joining the cache ([LB-SLOT] "进阶：光流关键帧与回滚机制":
    a non-keyframe attends to the cache and to its own K/V, which are then
    discarded).  The visible set is the plan's tokens followed by every row of
    the frame's own K/V (its specials, then its patches, as the frame is laid
    out); the order does not change the softmax, only float64 rounding."""
    k, v = gather_visible(pool, plan, cfg)
    k = np.concatenate([k, bf16_bits_to_f64(own_k_bits)], axis=0)
    v = np.concatenate([v, bf16_bits_to_f64(own_v_bits)], axis=0)
    q = bf16_bits_to_f64(q_bits)
    if rows is not None:
        q = q[np.asarray(rows)]
    return dense_attention(q, k, v, sm_scale)
