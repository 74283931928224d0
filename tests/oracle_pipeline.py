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


def run(wl, fill: bool = True) -> OracleState:
    """Replay the allocator script, then the decode step's append; optionally fill pools."""
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
        ev = [e for e in events if e[0] == "copy" or e[1] in live]
        ocache.apply_events(st.k_pool, st.v_pool, ev, get, wl.in_dtype, wl.kv_dtype,
                            k_scale, v_scale)
        if pairs:
            ocache.copy_blocks(st.k_pool, st.v_pool, pairs)
        kn, vn = new_token_inputs(wl, starts)
        ocache.reshape_and_cache(st.k_pool, st.v_pool, kn, vn, slots, wl.in_dtype,
                                 wl.kv_dtype, k_scale, v_scale)
    return st


def new_token_inputs(wl, positions):
    """K, V [S, Hkv, D] of the token each sequence decodes this step (input format)."""
    ks, vs = [], []
    for i, pos in enumerate(positions):
        k, v = wl.seq_kv_input(i)
        ks.append(k[pos])
        vs.append(v[pos])
    return np.stack(ks), np.stack(vs)


def decode(st: OracleState, seqs=None) -> np.ndarray:
    wl = st.wl
    return oattn.paged_decode(st.q64(), st.k_pool, st.v_pool, st.tables, st.ctx, wl.scale,
                              wl.kv_dtype, st.k_scale, st.v_scale, seqs=seqs)
