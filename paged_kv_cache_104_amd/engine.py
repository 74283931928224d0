"""One layer's paged KV cache on the GPU: pools + block manager + decode step.

The serving-engine side of the hot path, reduced to what one decode step
needs: the C++ block manager decides block tables, slots and copy-on-write
pairs on the host; the HIP kernels copy blocks, write new tokens and run the
decode attention on the device.

Allocator scripts are lists of operations:
``('add', seq, n)``, ``('fork', parent, child)``, ``('extend', seq, n)``,
``('append_batch', [seqs])``, ``('free', seq)``, and with prefix caching
``('add_tokens', seq, token_ids)`` and ``('extend_tokens', seq, token_ids)``
(tokens found cached are not written again).  Copy-on-write pairs are copied
on the device before any later token write, since the last holder of a shared
block writes into it in place.
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence

import numpy as np

from . import (IMPL_AUTO, IMPL_SHARED_BLOCKS, BlockManager, CacheDesc, alloc_host_pools,
               alloc_pools, alloc_quest_meta, append_tokens, copy_blocks, decode_workspace_bytes,
               paged_attn_decode, prefix_rows, quest_blocks_of_slots, quest_decode,
               quest_update_blocks, quest_update_tails, reshape_and_cache, swap_blocks)


def to_device(x: np.ndarray, in_dtype: str, device):
    """Host array in input format (float32, or bf16 bit patterns) -> device tensor."""
    import torch

    if in_dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device)


class PagedKVCache:
    def __init__(self, desc: CacheDesc, free_order: Optional[Sequence[int]] = None,
                 device="cuda", poison: bool = True, prefix_caching: bool = False):
        self.desc = desc
        self.device = device
        self.bm = BlockManager(desc.num_blocks, desc.block_size, free_order)
        if prefix_caching:
            self.bm.set_prefix_caching(True)
        self.k_pool, self.v_pool = alloc_pools(desc, device, poison)
        self.quest_meta = None

    # -- device work ------------------------------------------------------------
    def write(self, k, v, slots) -> None:
        import torch

        slot_t = torch.as_tensor(np.ascontiguousarray(slots, dtype=np.int64)).to(self.device)
        reshape_and_cache(k, v, slot_t, self.k_pool, self.v_pool, self.desc)
        if self.quest_meta is not None:
            blocks, counts = quest_blocks_of_slots(slots, self.desc.block_size)
            quest_update_blocks(self.k_pool, self.quest_meta, blocks, counts, self.desc)

    def copy(self, pairs) -> None:
        if len(pairs):
            copy_blocks(self.k_pool, self.v_pool, np.asarray(pairs, dtype=np.int64), self.desc)

    # -- swapping ------------------------------------------------------------
    def enable_swap(self, num_host_blocks: int) -> None:
        """A pinned host pool of ``num_host_blocks`` blocks for swapped-out sequences."""
        self.bm.set_host_pool(num_host_blocks)
        self.host_k, self.host_v = alloc_host_pools(self.desc, num_host_blocks)

    def swap_out(self, seqs, method: str = "kernel"):
        """Move a set of sequences (with all their forks) to the host pool; their device
        blocks are free for others once the copy, queued on the stream, has run."""
        pairs = self.bm.swap_out(seqs)
        swap_blocks(self.k_pool, self.v_pool, self.host_k, self.host_v, pairs, self.desc, method)
        return pairs

    def swap_in(self, seqs, method: str = "kernel"):
        pairs = self.bm.swap_in(seqs)
        swap_blocks(self.host_k, self.host_v, self.k_pool, self.v_pool, pairs, self.desc, method)
        if self.quest_meta is not None and len(pairs):
            self.quest_refresh(seqs)          # the set holds every sharer of its blocks
        return pairs

    # -- query-aware block selection -----------------------------------------
    def enable_quest(self, live_seqs: Sequence[int] = ()) -> None:
        """Keep per-block key minimum / maximum metadata from now on (computed now for the
        blocks of ``live_seqs``; later writes, appends and swap-ins keep it current)."""
        self.quest_meta = alloc_quest_meta(self.desc, self.device)
        self.quest_refresh(live_seqs)

    def quest_refresh(self, seqs) -> None:
        """Recompute the metadata of every block of ``seqs`` from the key pool."""
        blocks, counts = self.bm.block_fills(seqs)
        keep = counts > 0
        if keep.any():
            quest_update_blocks(self.k_pool, self.quest_meta, blocks[keep], counts[keep],
                                self.desc)

    def quest_decode(self, q, out, tables, lens, scale: float, max_context_len: int,
                     budget_blocks: int, partition_size: int = 0, workspace=None,
                     impl: int = IMPL_AUTO):
        if self.quest_meta is None:
            raise RuntimeError("enable_quest() first")
        return quest_decode(q, self.k_pool, self.v_pool, self.quest_meta, self.desc, tables,
                            lens, scale, out, max_context_len, budget_blocks, partition_size,
                            workspace, impl)

    # -- allocator script ----------------------------------------------------
    def run_script(self, ops, kv_input: Callable[[int], tuple], in_dtype: str,
                   keep: Optional[Callable[[int], bool]] = None) -> None:
        """Replay ``ops``; ``kv_input(seq)`` gives that sequence's (K, V) by position.

        Token writes of sequences for which ``keep(seq)`` is false are skipped
        (their blocks are still allocated).
        """
        keep = keep or (lambda s: True)
        bm = self.bm

        def put(seq, positions, slots):
            if not keep(seq) or len(positions) == 0:
                return
            k, v = kv_input(seq)
            self.write(to_device(k[positions], in_dtype, self.device),
                       to_device(v[positions], in_dtype, self.device), slots)

        for op in ops:
            kind = op[0]
            if kind == "add":
                _, seq, n = op
                bm.add_seq(seq, n)
                if n:
                    put(seq, np.arange(n), bm.slots(seq, 0, n))
            elif kind == "fork":
                bm.fork(op[1], op[2])
            elif kind == "free":
                bm.free_seq(op[1])
            elif kind == "extend":
                _, seq, n = op
                start = bm.seq_len(seq)
                slots, pairs = bm.extend(seq, n)
                self.copy(pairs)
                put(seq, np.arange(start, start + n), slots)
            elif kind == "append_batch":
                seqs = list(op[1])
                starts = [bm.seq_len(s) for s in seqs]
                slots, pairs = bm.append_batch(seqs)
                self.copy(pairs)
                for s, p, sl in zip(seqs, starts, slots):
                    put(s, np.array([p]), np.array([sl]))
            elif kind == "add_tokens":
                _, seq, toks = op
                n = len(toks)
                cached = bm.add_seq_tokens(seq, toks)
                if n > cached:
                    put(seq, np.arange(cached, n), bm.slots(seq, cached, n - cached))
            elif kind == "extend_tokens":
                _, seq, toks = op
                start = bm.seq_len(seq)
                slots, pairs = bm.extend_tokens(seq, toks)
                self.copy(pairs)
                put(seq, np.arange(start, start + len(toks)), slots)
            else:
                raise ValueError(f"unknown op {kind}")

    # -- decode step ---------------------------------------------------------
    def append_and_write(self, seqs, k_new, v_new):
        """Reserve one slot per sequence, copy shared partial blocks, write the new tokens.

        Returns (slots, pairs) as host arrays.
        """
        slots, pairs = self.bm.append_batch(seqs)
        self.copy(pairs)
        self.write(k_new, v_new, slots)
        return slots, pairs

    def tables(self, seqs, max_blocks: int):
        import torch

        t, lens = self.bm.block_tables(seqs, max_blocks)
        return torch.from_numpy(t).to(self.device), torch.from_numpy(lens).to(self.device)

    def shares_blocks(self) -> bool:
        """True when some physical block is held by more than one sequence."""
        st = self.bm.stats()
        return st["logical_blocks"] > st["physical_blocks"]

    def decode(self, q, out, tables, lens, scale: float, max_context_len: int,
               partition_size: int = 0, workspace=None, impl: int = IMPL_AUTO,
               hint_sharing: bool = False):
        """Decode over the cache's pools.  ``hint_sharing``: when some block is held by
        several sequences, read K/V with ordinary cached loads (PKV_IMPL_SHARED_BLOCKS)
        instead of streaming them.  Off by default: the cached loads gain only when the last
        level cache holds no dirty lines of other work when the decode starts; after a large
        write they pay for writing those lines back."""
        if hint_sharing and self.shares_blocks():
            impl |= IMPL_SHARED_BLOCKS
        return paged_attn_decode(q, self.k_pool, self.v_pool, tables, lens, scale, out, self.desc,
                                 max_context_len, partition_size, workspace, impl)

    def workspace(self, num_seqs: int, num_q_heads: int, max_context_len: int,
                  partition_size: int):
        import torch

        n = decode_workspace_bytes(num_seqs, num_q_heads, self.desc.head_dim, max_context_len,
                                   partition_size)
        return torch.empty(max(n, 16), dtype=torch.uint8, device=self.device) if n else None


class DecodeBatch:
    """A fixed batch of sequences whose block tables and context lengths live on the device.

    They are uploaded once; each decode step's append then writes the new tokens and
    brings the device tables up to date in the same launch (``append_tokens``), so a
    step moves nothing from the host but the kernel arguments.
    """

    def __init__(self, cache: PagedKVCache, seqs: Sequence[int], max_blocks: int):
        import torch

        self.cache = cache
        self.seqs = [int(s) for s in seqs]
        self.max_blocks = max_blocks
        t, lens = cache.bm.block_tables(self.seqs, max_blocks)
        self.tables = torch.from_numpy(t).to(cache.device)
        self.lens = torch.from_numpy(lens).to(cache.device)
        self.host_lens = lens.astype(np.int64)

    def append(self, k_new, v_new):
        """One token per sequence: block manager, copy-on-write copies, write + table update.

        Returns (slots, pairs) as host arrays."""
        c = self.cache
        slots, pairs = c.bm.append_batch(self.seqs)
        c.copy(pairs)
        append_tokens(k_new, v_new, slots, self.host_lens, c.k_pool, c.v_pool, c.desc,
                      self.tables, self.lens)
        if c.quest_meta is not None:
            quest_update_tails(c.k_pool, c.quest_meta, self.tables, self.lens, c.desc)
        self.host_lens += 1
        return slots, pairs

    def max_context_len(self) -> int:
        return int(self.host_lens.max()) if len(self.host_lens) else 0

    def shared_prefix_rows(self, group: int, min_shared_blocks: int = 1):
        """Units of the shared-prefix decode for the batch as it stands, uploaded:
        ``(rows, seq_rows, reread)``, device int32 tensors and whether some unit's shared
        blocks are read by other units too (then ``shared_blocks=True`` for the decode can
        pay, when the last-level cache holds no dirty lines of other work).
        Sequences that share leading blocks must be consecutive in the batch.  The units
        stay valid while no shared block is replaced (appends only grow the contexts after
        the shared part)."""
        import torch

        t, lens = self.cache.bm.block_tables(self.seqs, self.max_blocks)
        rows, seq_rows = prefix_rows(t, lens, self.cache.desc.block_size, group,
                                     min_shared_blocks)
        dev = self.cache.device
        return (torch.from_numpy(rows).to(dev), torch.from_numpy(seq_rows).to(dev),
                bool(rows[:, 3].any()))
