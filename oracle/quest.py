"""Query-aware block selection (QUEST) for decode (test infrastructure only).

What the page fixes (tencent cloud article 2526001, section "QUEST:
Query-Aware Sparsity for Efficient Long-Context LLM Inference", the paragraph on
its top-K procedure and figure):

* For every block, the channel-wise minimum and maximum of its keys.
* For a query, each channel's product with the minimum and with the maximum;
  the larger of the two (the minimum wins where the query is negative) summed
  over channels bounds from above the query's score with any key of the block.
* Only the K blocks with the largest bounds take part in attention; K is a
  hyperparameter (the page cites a budget of 4096).

Readings where the page is silent:

* Min / max run over the block's valid tokens only (the sequence's last block
  may be partly filled), on dequantised keys.
* The budget is given in blocks here (4096 tokens = 256 blocks of 16).  A
  context of no more blocks than the budget is attended in full.
* Grouped-query attention: one selection per (sequence, KV head), shared by its
  query heads, scored with the largest bound over those heads.
* Ranking is by bound, then by lower logical block index for equal bounds; the
  selected blocks are attended in logical order, and the softmax runs over
  their tokens only.
"""
from __future__ import annotations

import numpy as np

from . import attention as oattn


def block_minmax(k_pool, table, ctx: int, kv_head: int, kv_dtype: str, k_scale: float = 1.0):
    """(min, max) [nblocks, D] of the dequantised keys of one (sequence, KV head)."""
    K = oattn.dequant(oattn.gather_keys(k_pool, table, ctx, kv_head), kv_dtype, k_scale)
    B = k_pool.shape[2]
    nb = -(-ctx // B)
    mins = np.stack([K[b * B:min(ctx, (b + 1) * B)].min(axis=0) for b in range(nb)]) if nb else \
        np.zeros((0, K.shape[1]))
    maxs = np.stack([K[b * B:min(ctx, (b + 1) * B)].max(axis=0) for b in range(nb)]) if nb else \
        np.zeros((0, K.shape[1]))
    return mins, maxs


def bounds(q, mins, maxs):
    """Upper bounds [heads, nblocks] of q . k over each block: sum_d max(q_d min_d, q_d max_d)."""
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    lo = q[:, None, :] * mins[None, :, :]
    hi = q[:, None, :] * maxs[None, :, :]
    return np.maximum(lo, hi).sum(axis=2)


def select(scores, budget: int):
    """Indices (ascending) of the `budget` blocks with the largest scores, lower index first
    among equal scores; every block when there are no more than `budget`."""
    scores = np.asarray(scores, dtype=np.float64)
    n = len(scores)
    if n <= budget:
        return np.arange(n)
    order = sorted(range(n), key=lambda b: (-scores[b], b))
    return np.sort(np.asarray(order[:budget]))


def selected_blocks(q, k_pool, tables, ctx, num_kv_heads: int, budget: int, kv_dtype: str,
                    k_scale: float = 1.0):
    """Per (sequence, KV head): the logical indices of the blocks QUEST keeps."""
    S, Hq, _ = q.shape
    g = Hq // num_kv_heads
    out = {}
    for s in range(S):
        for kvh in range(num_kv_heads):
            mins, maxs = block_minmax(k_pool, tables[s], int(ctx[s]), kvh, kv_dtype, k_scale)
            u = bounds(q[s, kvh * g:(kvh + 1) * g], mins, maxs).max(axis=0) if len(mins) else \
                np.zeros(0)
            out[(s, kvh)] = select(u, budget)
    return out


def quest_decode(q, k_pool, v_pool, tables, ctx, scale: float, num_kv_heads: int, budget: int,
                 kv_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0, chosen=None):
    """Decode attention over the QUEST-selected blocks (or over `chosen`, if given)."""
    S, Hq, D = q.shape
    g = Hq // num_kv_heads
    B = k_pool.shape[2]
    if chosen is None:
        chosen = selected_blocks(q, k_pool, tables, ctx, num_kv_heads, budget, kv_dtype, k_scale)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        n = int(ctx[s])
        for kvh in range(num_kv_heads):
            K = oattn.dequant(oattn.gather_keys(k_pool, tables[s], n, kvh), kv_dtype, k_scale)
            V = oattn.dequant(oattn.gather_values(v_pool, tables[s], n, kvh), kv_dtype, v_scale)
            keep = np.concatenate([np.arange(b * B, min(n, (b + 1) * B))
                                   for b in chosen[(s, kvh)]]).astype(np.int64) \
                if len(chosen[(s, kvh)]) else np.zeros(0, dtype=np.int64)
            for h in range(kvh * g, (kvh + 1) * g):
                out[s, h] = oattn.attend(q[s, h], K[keep], V[keep], scale)
    return out
