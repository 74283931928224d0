"""Oracle side of a workload: allocator replay, cache writes, decode-step inputs.

Runs only ``oracle/`` code on the seeded draws of ``workloads``; nothing here
touches the HIP library.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

from oracle import allocator as oalloc
from oracle import attention as oattn
from oracle import prefix_cache as oprefix
from oracle import cache as ocache
from oracle import codec


@dataclasses.dataclass
class OracleState:
    wl: object
    alloc: oalloc.BlockAllocator
    k_pool: Optional[np.ndarray]
    v_pool: Optional[np.ndarray]
    setup_events: list
    step_slots: List[int]
    step_pairs: list
    tables: np.ndarray
    ctx: np.ndarray
    k_scale: float
    v_scale: float

    def q64(self) -> np.ndarray:
        q = self.wl.q_input()
        return codec.bf16_to_f64(q) if self.wl.in_dtype == "bf16" else q.astype(np.float64)


def kv_by_seq(wl):
    index = wl.seq_index()

    def get(seq):
        seq = int(seq)
        if seq not in index:
            return wl.extra_kv_input(seq)
        return wl.seq_kv_input(index[seq])
    return get


def new_allocator(wl):
    cls = oprefix.PrefixCachingAllocator if wl.prefix_caching else oalloc.BlockAllocator
    return cls(wl.num_blocks, wl.block_size, wl.free_order)


def _encoded_source(wl, get, seqs, k_scale, v_scale, workers):
    """Every sequence's K, V already in pool storage: the oracle's own encode, run for many
    sequences at once on threads (numpy releases the GIL inside it), so that a full-size
    fp8 workload fills in seconds instead of minutes.  The arithmetic is unchanged."""
    from concurrent.futures import ThreadPoolExecutor

    def enc(seq):
        k, v = get(seq)
        return (ocache.encode(k, wl.in_dtype, wl.kv_dtype, k_scale),
                ocache.encode(v, wl.in_dtype, wl.kv_dtype, v_scale))

    seqs = sorted(int(s) for s in seqs)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        done = dict(zip(seqs, ex.map(enc, seqs)))
    return lambda seq: done[int(seq)]


def run(wl, fill: bool = True, encode_workers: int = 1) -> OracleState:
    """Replay the allocator script, then the decode step's append; optionally fill pools.

    ``encode_workers`` > 1 encodes an fp8 workload's inputs on that many threads first."""
    alloc = new_allocator(wl)
    # the churn dummies own no data: their writes are dropped
    events = oalloc.run_ops(alloc, wl.setup_ops)
    seqs = [int(s) for s in wl.decode_seqs]
    starts = [alloc.lens[s] for s in seqs]
    slots, pairs = alloc.append_batch(seqs)
    assert [alloc.lens[s] for s in seqs] == [int(c) for c in wl.ctx_lens]
    tables, ctx = alloc.block_tables(seqs, wl.max_blocks_per_seq)
    k_scale, v_scale = wl.kv_scales()
    st = OracleState(wl, alloc, None, None, events, slots, pairs, tables, ctx, k_scale, v_scale)
    if fill:
        st.k_pool, st.v_pool = ocache.new_pools(wl.num_blocks, wl.num_kv_heads, wl.block_size,
                                                wl.head_dim, wl.kv_dtype)
        get = kv_by_seq(wl)
        live = wl.data_seqs()
        in_dtype = wl.in_dtype
        if wl.kv_dtype == "fp8" and in_dtype != "fp8" and encode_workers > 1:
            get = _encoded_source(wl, get, live, k_scale, v_scale, encode_workers)
            in_dtype = "fp8"                       # inputs already encoded: stored as they are
        ev = [e for e in events if e[0] == "copy" or e[1] in live]
        ocache.apply_events(st.k_pool, st.v_pool, ev, get, in_dtype, wl.kv_dtype,
                            k_scale, v_scale)
        if pairs:
            ocache.copy_blocks(st.k_pool, st.v_pool, pairs)
        kn, vn = new_token_inputs(wl, starts, get)
        ocache.reshape_and_cache(st.k_pool, st.v_pool, kn, vn, slots, in_dtype,
                                 wl.kv_dtype, k_scale, v_scale)
    return st


def new_token_inputs(wl, positions, get=None):
    """K, V [S, Hkv, D] of the token each sequence decodes this step (input format, or
    what ``get`` serves)."""
    get = kv_by_seq(wl) if get is None else get
    ks, vs = [], []
    for seq, pos in zip(wl.decode_seqs, positions):
        k, v = get(int(seq))
        ks.append(k[pos])
        vs.append(v[pos])
    return np.stack(ks), np.stack(vs)


def decode(st: OracleState, seqs=None, scale=None) -> np.ndarray:
    wl = st.wl
    return oattn.paged_decode(st.q64(), st.k_pool, st.v_pool, st.tables, st.ctx,
                              wl.scale if scale is None else scale, wl.kv_dtype, st.k_scale,
                              st.v_scale, seqs=seqs)
