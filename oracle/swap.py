"""Swapping sequences between the device pool and a host pool (test infrastructure only).

What the pages fix, and where (review of the vLLM paper on cayang0802.github.io,
the preemption paragraphs after the scheduling section): when a new token needs
device memory that is not there, a sequence that is not needed for now can be
swapped out -- its KV cache moved to host memory, which is slower -- and moved
back when device memory frees up.  The same page notes that small blocks make
this slower, many small transfers leaving the host link underused.

Readings where the pages are silent:

* The host pool has its own blocks with the device pool's block shape, its own
  free list (head out, tail in) and its own counts.
* Swapping moves a set of sequences at once: every block one of them holds must
  be held only by sequences of the set (forked samples move together), so a
  shared block moves once and keeps its count.  A set that shares a block with a
  sequence outside it is refused.
* Swap-out maps the set's distinct device blocks, in order of first appearance
  (sequences in the order given, blocks in logical order), to host blocks taken
  from the host free list; the device blocks return to the device free list in
  that order (without a prefix-cache key, if they had one).  Swap-in maps host
  blocks to device blocks the same way and returns the host blocks.  Each
  returns the (source, destination) pairs the device must copy, before any later
  write reuses a block.
* A swapped-out sequence can only be swapped in or released; releasing returns
  its host blocks.
* Running out of blocks on the receiving side fails the whole swap and changes
  nothing.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, List, Sequence, Tuple

from .allocator import BlockAllocator, NoMemory
from .prefix_cache import PrefixCachingAllocator


class SwapMixin:
    def init_host_pool(self, num_host_blocks: int) -> None:
        if num_host_blocks < 0:
            raise ValueError("negative host pool")
        self.num_host_blocks = num_host_blocks
        self.host_free: deque = deque(range(num_host_blocks))
        self.host_ref: List[int] = [0] * num_host_blocks
        self.swapped: set = set()

    def _resident(self, seq: int) -> None:
        if seq not in self.tables or seq in getattr(self, "swapped", ()):
            raise ValueError("unknown or swapped-out sequence")

    # -- the moves ------------------------------------------------------------------
    def _distinct(self, seqs: Sequence[int], counts: List[int]) -> List[int]:
        order, seen = [], {}
        for s in seqs:
            for b in self.tables[s]:
                if b not in seen:
                    seen[b] = 0
                    order.append(b)
                seen[b] += 1
        for b in order:
            if seen[b] != counts[b]:
                raise ValueError("a block is shared with a sequence outside the set")
        return order

    def swap_out(self, seqs: Sequence[int]) -> List[Tuple[int, int]]:
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs):
            raise ValueError("repeated sequence")
        for s in seqs:
            self._resident(s)
        blocks = self._distinct(seqs, self.ref)
        if len(blocks) > len(self.host_free):
            raise NoMemory(seqs)
        to = {}
        for b in blocks:
            h = self.host_free.popleft()
            self.host_ref[h] = self.ref[b]
            to[b] = h
        for s in seqs:
            self.tables[s] = [to[b] for b in self.tables[s]]
            self.swapped.add(s)
        for b in blocks:
            self.ref[b] = 0
            key_of = getattr(self, "key_of", None)
            if key_of is not None and key_of[b] is not None:
                del self.cache[key_of[b]]
                key_of[b] = None
            self.free.append(b)
        return [(b, to[b]) for b in blocks]

    def swap_in(self, seqs: Sequence[int]) -> List[Tuple[int, int]]:
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs) or any(s not in self.swapped for s in seqs):
            raise ValueError("repeated or resident sequence")
        hosts = self._distinct(seqs, self.host_ref)
        if len(hosts) > self.available():
            raise NoMemory(seqs)
        to = {}
        for h in hosts:
            d = self._pop()
            self.ref[d] = self.host_ref[h]
            to[h] = d
        for s in seqs:
            self.tables[s] = [to[h] for h in self.tables[s]]
            self.swapped.discard(s)
        for h in hosts:
            self.host_ref[h] = 0
            self.host_free.append(h)
        return [(h, to[h]) for h in hosts]

    # -- operations on resident sequences only ---------------------------------------
    def fork(self, parent, child):
        self._resident(parent)
        return super().fork(parent, child)

    def append(self, seq):
        self._resident(seq)
        return super().append(seq)

    def append_batch(self, seqs):
        for s in seqs:
            self._resident(int(s))
        return super().append_batch(seqs)

    def extend(self, seq, n):
        self._resident(seq)
        return super().extend(seq, n)

    def slots(self, seq, start, n):
        self._resident(seq)
        return super().slots(seq, start, n)

    def block_tables(self, seqs, max_blocks):
        for s in seqs:
            self._resident(int(s))
        return super().block_tables(seqs, max_blocks)

    def free_seq(self, seq):
        if seq in self.swapped:
            for h in self.tables.pop(seq):
                self.host_ref[h] -= 1
                if self.host_ref[h] == 0:
                    self.host_free.append(h)
            del self.lens[seq]
            self.swapped.discard(seq)
            getattr(self, "tokens", {}).pop(seq, None)
            return
        super().free_seq(seq)

    def stats(self) -> Dict[str, int]:
        st = super().stats()
        # swapped sequences' tables hold host blocks: count device figures over residents
        res = {s: t for s, t in self.tables.items() if s not in self.swapped}
        st["tokens"] = sum(self.lens[s] for s in res)
        st["logical_blocks"] = sum(len(t) for t in res.values())
        st["slots_allocated"] = st["logical_blocks"] * self.block_size
        st["host_free_blocks"] = len(self.host_free)
        st["swapped_seqs"] = len(self.swapped)
        return st


class SwappingAllocator(SwapMixin, BlockAllocator):
    def __init__(self, num_blocks: int, block_size: int, free_order=None,
                 num_host_blocks: int = 0):
        super().__init__(num_blocks, block_size, free_order)
        self.init_host_pool(num_host_blocks)


class SwappingPrefixCachingAllocator(SwapMixin, PrefixCachingAllocator):
    def __init__(self, num_blocks: int, block_size: int, free_order=None,
                 num_host_blocks: int = 0):
        super().__init__(num_blocks, block_size, free_order)
        self.init_host_pool(num_host_blocks)
