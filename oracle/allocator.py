"""Block allocator model of the oracle (test infrastructure only).

What the pages fix, and where:

* The KV cache is cut into fixed-size physical blocks of B tokens held in one
  pool shared by every request; a per-request block table maps logical block j
  to a physical block, in order (ithome article 10417389, section 3
  "PagedAttention"; ultralytics glossary, section "How paging works").
* A request takes only the blocks that hold its tokens, and a new block only
  when its last block is full (same passages).  The glossary's code example
  takes blocks from the head of the free list, ``free_blocks.pop(0)``.
* Token ``pos`` lives at ``pool[table[pos // B], pos % B]`` (glossary code
  example); the optiverse block-table table shows fills 16/16/9 for 41 tokens
  and token 41 landing in the 10th position of the third block.
* When a request ends, all its blocks go back to the pool (optiverse,
  "Block table and non-contiguous allocation"; glossary, continuous batching).
* Forked samples point at the same physical blocks with reference count 2;
  full shared blocks stay shared; a write into a shared, partly filled last
  block gives the writer a new block holding a copy and drops the old block's
  count by one (ithome, section 4 "Physical block sharing" and "Copy-on-Write").

Readings where the pages are silent:

* Freed blocks are appended to the tail of the free list, in the freed
  sequence's logical order; allocation always pops the head.
* A batch of appends is applied in the order given; callers pass ascending
  sequence ids, so with n holders of a shared partial block the first n-1 copy
  and the last writes in place (the ithome figure: sample A1 writes first and
  gets new block 3, block 1's count goes 2 -> 1, A2 then writes into block 1).
* The copy-on-write copy covers the whole block (all slots, all heads, K and V).
* Running out of free blocks fails the whole operation and changes nothing.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, Iterable, List, Optional, Sequence, Tuple


class NoMemory(Exception):
    """Not enough free blocks; the allocator state is unchanged."""


class BlockAllocator:
    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if len(set(order)) != len(order) or any(b < 0 or b >= num_blocks for b in order):
            raise ValueError("free_order must hold distinct block ids in [0, num_blocks)")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: deque = deque(order)
        self.ref: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}

    # -- helpers -------------------------------------------------------------
    def _pop(self) -> int:
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def blocks_needed(self, n_tokens: int) -> int:
        return -(-n_tokens // self.block_size)

    def available(self) -> int:
        """Blocks an allocation may take (the free list here)."""
        return len(self.free)

    # -- operations ----------------------------------------------------------
    def add_seq(self, seq: int, n_tokens: int) -> List[int]:
        """Admit a sequence holding ``n_tokens`` tokens; returns its block table."""
        if seq in self.tables or n_tokens < 0:
            raise ValueError("bad add_seq")
        need = self.blocks_needed(n_tokens)
        if need > self.available():
            raise NoMemory(seq)
        self.tables[seq] = [self._pop() for _ in range(need)]
        self.lens[seq] = n_tokens
        return list(self.tables[seq])

    def fork(self, parent: int, child: int) -> None:
        """The child shares every block of the parent; each block's count goes up by one."""
        if parent not in self.tables or child in self.tables:
            raise ValueError("bad fork")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def append(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot of the next token; returns (slot, copy pair or None)."""
        if seq not in self.tables:
            raise ValueError("bad append")
        pos = self.lens[seq]
        table = self.tables[seq]
        pair = None
        if pos % self.block_size == 0:                   # last block full (or none yet)
            if not self.available():
                raise NoMemory(seq)
            table.append(self._pop())
        elif self.ref[table[-1]] > 1:                    # shared, partly filled: copy on write
            if not self.available():
                raise NoMemory(seq)
            old = table[-1]
            new = self._pop()
            self.ref[old] -= 1
            table[-1] = new
            pair = (old, new)
        slot = table[pos // self.block_size] * self.block_size + pos % self.block_size
        self.lens[seq] = pos + 1
        return slot, pair

    def append_batch(self, seqs: Iterable[int]) -> Tuple[List[int], List[Tuple[int, int]]]:
        """One token for each sequence, in the order given; all-or-nothing."""
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs) or any(s not in self.tables for s in seqs):
            raise ValueError("bad append_batch")
        # dry run on counts: a block is needed for a full last block, or for a
        # shared partial last block whose count (after earlier copies in this
        # batch) is still above one
        drop: Dict[int, int] = {}
        need = 0
        for s in seqs:
            pos = self.lens[s]
            if pos % self.block_size == 0:
                need += 1
                continue
            last = self.tables[s][-1]
            if self.ref[last] - drop.get(last, 0) > 1:
                need += 1
                drop[last] = drop.get(last, 0) + 1
        if need > self.available():
            raise NoMemory(seqs)
        slots, pairs = [], []
        for s in seqs:
            slot, pair = self.append(s)
            slots.append(slot)
            if pair is not None:
                pairs.append(pair)
        return slots, pairs

    def extend(self, seq: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """``n`` tokens for one sequence; all-or-nothing."""
        if seq not in self.tables or n < 0:
            raise ValueError("bad extend")
        pos = self.lens[seq]
        have = len(self.tables[seq]) * self.block_size - pos      # free slots in the last block
        need = self.blocks_needed(max(0, n - have))
        if n > 0 and have > 0 and self.ref[self.tables[seq][-1]] > 1:
            need += 1
        if need > self.available():
            raise NoMemory(seq)
        slots, pairs = [], []
        for _ in range(n):
            slot, pair = self.append(seq)
            slots.append(slot)
            if pair is not None:
                pairs.append(pair)
        return slots, pairs

    def free_seq(self, seq: int) -> None:
        """Drop one reference to every block of the sequence; blocks at zero go to the tail."""
        if seq not in self.tables:
            raise ValueError("bad free")
        for b in self.tables.pop(seq):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.lens[seq]

    # -- queries -------------------------------------------------------------
    def slot(self, seq: int, pos: int) -> int:
        table = self.tables[seq]
        return table[pos // self.block_size] * self.block_size + pos % self.block_size

    def slots(self, seq: int, start: int, n: int) -> List[int]:
        if start < 0 or start + n > self.lens[seq]:
            raise ValueError("bad slots")
        return [self.slot(seq, p) for p in range(start, start + n)]

    def block_tables(self, seqs: Sequence[int], max_blocks: int):
        """Packed tables [n, max_blocks] (padding -1) and context lengths [n]."""
        import numpy as np

        out = np.full((len(seqs), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for i, s in enumerate(seqs):
            t = self.tables[int(s)]
            if len(t) > max_blocks:
                raise ValueError("table longer than max_blocks")
            out[i, :len(t)] = t
            lens[i] = self.lens[int(s)]
        return out, lens

    def stats(self) -> Dict[str, int]:
        tokens = sum(self.lens.values())
        logical = sum(len(t) for t in self.tables.values())
        return {
            "free_blocks": len(self.free),
            "used_blocks": self.num_blocks - len(self.free),
            "tokens": tokens,
            "slots_allocated": logical * self.block_size,
            "logical_blocks": logical,
            "physical_blocks": sum(1 for r in self.ref if r > 0),
        }


def run_ops(alloc: BlockAllocator, ops) -> List[tuple]:
    """Replay a workload's allocator script.

    Returns the device work the script implies, in the order it must happen:
    ``('copy', [(src, dst), ...])`` for copy-on-write pairs (which must run
    before any later write, since the last holder of a shared block writes in
    place) and ``('write', seq, positions, slots)`` for token writes.
    """
    events: List[tuple] = []
    for op in ops:
        kind = op[0]
        if kind == "add":
            _, seq, n = op
            alloc.add_seq(seq, n)
            if n:
                events.append(("write", seq, list(range(n)), alloc.slots(seq, 0, n)))
        elif kind == "fork":
            alloc.fork(op[1], op[2])
        elif kind == "free":
            alloc.free_seq(op[1])
        elif kind == "extend":
            _, seq, n = op
            start = alloc.lens[seq]
            slots, pairs = alloc.extend(seq, n)
            if pairs:
                events.append(("copy", pairs))
            events.append(("write", seq, list(range(start, start + n)), slots))
        elif kind == "append_batch":
            seqs = op[1]
            starts = [alloc.lens[s] for s in seqs]
            slots, pairs = alloc.append_batch(seqs)
            if pairs:
                events.append(("copy", pairs))
            for s, p, sl in zip(seqs, starts, slots):
                events.append(("write", s, [p], [sl]))
        elif kind == "add_tokens":                  # prefix caching: cached tokens are not written
            _, seq, toks = op
            _, cached = alloc.add_seq_tokens(seq, toks)
            n = len(toks)
            if n > cached:
                events.append(("write", seq, list(range(cached, n)), alloc.slots(seq, cached, n - cached)))
        elif kind == "extend_tokens":
            _, seq, toks = op
            start = alloc.lens[seq]
            slots, pairs = alloc.extend_tokens(seq, toks)
            if pairs:
                events.append(("copy", pairs))
            events.append(("write", seq, list(range(start, start + len(toks))), slots))
        else:
            raise ValueError(kind)
    return events
