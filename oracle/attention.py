"""Paged decode attention of the oracle: naive gather + textbook softmax, float64.

Test infrastructure only.

What it follows:

* The attention kernel reads a request's keys and values back block by block
  through its block table, so the cache need not be contiguous (ultralytics
  glossary "PagedAttention", section "How paging works", whose code example
  reads the keys back by indexing the pool with the whole table, flattening
  the blocks and keeping the first ctx rows; optiverse article, "Block table
  and non-contiguous allocation").  Paging changes only
  where the bytes live: the result is plain softmax attention of the query over
  the sequence's cached keys and values.  FlashAttention-style tiling (glossary,
  "Related techniques") reorders the same sum and gives the same result.
* Grouped-query attention lets several query heads share one key/value head
  (glossary, "Related techniques"; Tencent article 2526001, "Compressed
  attention").  Reading: query heads are grouped contiguously, head h uses KV
  head ``h // (Hq / Hkv)``.
* An fp8 cache value is ``e4m3(code) * scale`` (per-tensor scale).

Readings where the pages are silent: the context of a sequence includes the
token being decoded (its K/V are written first); ``scale`` is given by the
caller (1/sqrt(head_dim) in every workload); a sequence with an empty context
returns zeros.
"""
from __future__ import annotations

import numpy as np

from . import codec


def dequant(values: np.ndarray, kv_dtype: str, scale: float = 1.0) -> np.ndarray:
    """Pool storage values -> float64 values."""
    if kv_dtype == "f32":
        return np.asarray(values, dtype=np.float32).astype(np.float64)
    if kv_dtype == "bf16":
        return codec.bf16_to_f64(values)
    if kv_dtype == "fp8":
        return codec.e4m3_to_f64(values) * np.float64(np.float32(scale))
    raise ValueError(kv_dtype)


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head h (contiguous groups)."""
    return h // (num_q_heads // num_kv_heads)


def gather_keys(k_pool, table, ctx: int, kv_head: int) -> np.ndarray:
    """Keys of positions 0..ctx-1, in logical order: ``k_pool[table[t // B], kv_head, t % B, :]``."""
    B = k_pool.shape[2]
    t = np.arange(ctx)
    return k_pool[np.asarray(table)[t // B], kv_head, t % B, :]


def gather_values(v_pool, table, ctx: int, kv_head: int) -> np.ndarray:
    """Values of positions 0..ctx-1, in logical order: ``v_pool[table[t // B], kv_head, :, t % B]``."""
    B = v_pool.shape[3]
    t = np.arange(ctx)
    return v_pool[np.asarray(table)[t // B], kv_head, :, t % B]


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query over K, V (float64); zeros for an empty context."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    z = scale * (K @ q)
    p = np.exp(z - z.max())
    p /= p.sum()
    return p @ V


def paged_decode(q, k_pool, v_pool, block_tables, context_lens, scale: float,
                 kv_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0,
                 seqs=None) -> np.ndarray:
    """Decode attention for every sequence (or the batch rows in ``seqs``).

    ``q``: float64 [S, Hq, D]; pools in storage format; ``block_tables`` [S, *]
    int; ``context_lens`` [S].  Returns float64 [S, Hq, D] (rows not in
    ``seqs`` are zero).
    """
    q = np.asarray(q, dtype=np.float64)
    S, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    out = np.zeros((S, Hq, D), dtype=np.float64)
    rows = range(S) if seqs is None else seqs
    for s in rows:
        ctx = int(context_lens[s])
        for kvh in range(Hkv):
            K = dequant(gather_keys(k_pool, block_tables[s], ctx, kvh), kv_dtype, k_scale)
            V = dequant(gather_values(v_pool, block_tables[s], ctx, kvh), kv_dtype, v_scale)
            for h in range(Hq):
                if kv_head_of(h, Hq, Hkv) == kvh:
                    out[s, h] = attend(q[s, h], K, V, scale)
    return out
