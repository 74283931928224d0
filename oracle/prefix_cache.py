"""Prefix caching on top of the block allocator (test infrastructure only).

What the pages fix, and where:

* A full KV block can be found again through a key made of its own tokens and
  every token before it; equal keys mean the same KV block, so a request whose
  prompt starts with the same full blocks as an earlier one reuses them instead
  of computing them again -- multi-turn dialogue being the example (review of
  the vLLM paper on cayang0802.github.io, the paragraphs on prefix caching after
  the preemption section).
* Hashing full blocks is how the block sharing of forked sequences extends to
  different requests (ultralytics glossary, "Sharing blocks between
  sequences"); shared blocks are reference counted (same section; ithome
  article 10417389, section 4).

Readings where the pages are silent:

* Only full blocks are cached.  The key of logical block i of a sequence with
  tokens t is the tuple t[0 : (i+1)*B] itself -- the prefix, not a hash of it,
  so two keys are equal exactly when the token prefixes are.
* A lookup takes the longest run of cached full blocks from the start of the
  prompt and stops at the first block that is not cached.
* A block whose count falls to zero keeps its key and becomes evictable; a
  later lookup that finds it revives it (count 0 -> 1).  New blocks come from
  the free list first; when it is empty, the evictable block released longest
  ago is evicted (its key forgotten) and reused.
* A released sequence's cached blocks join the evictable queue last block
  first, so a prefix outlives the blocks that extend it.  Its uncached blocks
  return to the free list's tail in logical order, as without caching.
* A block that becomes full takes its key unless the key already names another
  block; the first block keeps it.
* Sequences admitted by count alone (no tokens) never hit and never register.
"""
from __future__ import annotations

from collections import OrderedDict
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

from .allocator import BlockAllocator, NoMemory


class PrefixCachingAllocator(BlockAllocator):
    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        super().__init__(num_blocks, block_size, free_order)
        self.cache: Dict[tuple, int] = {}
        self.key_of: List[Optional[tuple]] = [None] * num_blocks
        self.evictable: "OrderedDict[int, None]" = OrderedDict()   # released longest ago first
        self.tokens: Dict[int, List[int]] = {}
        self.hit_tokens = 0
        self.query_tokens = 0

    # -- block supply ----------------------------------------------------------
    def available(self) -> int:
        return len(self.free) + len(self.evictable)

    def _pop(self) -> int:
        if self.free:
            b = self.free.popleft()
        else:
            b, _ = self.evictable.popitem(last=False)
            del self.cache[self.key_of[b]]
            self.key_of[b] = None
        self.ref[b] = 1
        return b

    def key(self, toks: Sequence[int], i: int) -> tuple:
        """Key of full logical block i: every token up to the end of that block."""
        return tuple(int(t) for t in toks[: (i + 1) * self.block_size])

    def _register(self, seq: int, i: int) -> None:
        k = self.key(self.tokens[seq], i)
        b = self.tables[seq][i]
        if k not in self.cache and self.key_of[b] is None:
            self.cache[k] = b
            self.key_of[b] = k

    def _note_tokens(self, seq: int, new_tokens: Sequence[int]) -> None:
        """Record tokens appended to a tracked sequence; register the blocks they filled."""
        if seq not in self.tokens:
            return
        before = len(self.tokens[seq])
        self.tokens[seq].extend(int(t) for t in new_tokens)
        for i in range(before // self.block_size, len(self.tokens[seq]) // self.block_size):
            self._register(seq, i)

    # -- operations --------------------------------------------------------------
    def lookup(self, toks: Sequence[int]) -> List[int]:
        """Cached blocks of the longest run of full blocks from the start."""
        hits = []
        for i in range(len(toks) // self.block_size):
            b = self.cache.get(self.key(toks, i))
            if b is None:
                break
            hits.append(b)
        return hits

    def add_seq_tokens(self, seq: int, toks: Sequence[int]) -> Tuple[List[int], int]:
        """Admit a sequence with these tokens; returns (block table, tokens already cached)."""
        if seq in self.tables:
            raise ValueError("bad add_seq_tokens")
        toks = [int(t) for t in toks]
        hits = self.lookup(toks)
        need = self.blocks_needed(len(toks)) - len(hits)
        revived = sum(1 for b in hits if self.ref[b] == 0)
        if need > self.available() - revived:
            raise NoMemory(seq)
        for b in hits:
            if self.ref[b] == 0:
                del self.evictable[b]
            self.ref[b] += 1
        self.tables[seq] = hits + [self._pop() for _ in range(need)]
        self.lens[seq] = len(toks)
        self.tokens[seq] = []
        self._note_tokens(seq, toks)
        self.query_tokens += len(toks)
        self.hit_tokens += len(hits) * self.block_size
        return list(self.tables[seq]), len(hits) * self.block_size

    def fork(self, parent: int, child: int) -> None:
        super().fork(parent, child)
        if parent in self.tokens:
            self.tokens[child] = list(self.tokens[parent])

    def append_token(self, seq: int, tok: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        slot, pair = self.append(seq)
        self._note_tokens(seq, [tok])
        return slot, pair

    def append_batch_tokens(self, seqs: Iterable[int], toks: Sequence[int]):
        """One token per sequence in the order given (all-or-nothing); blocks that fill
        register in that order."""
        seqs = [int(s) for s in seqs]
        if len(toks) != len(seqs):
            raise ValueError("one token per sequence")
        slots, pairs = self.append_batch(seqs)
        for s, t in zip(seqs, toks):
            self._note_tokens(s, [t])
        return slots, pairs

    def extend_tokens(self, seq: int, toks: Sequence[int]):
        slots, pairs = self.extend(seq, len(toks))
        self._note_tokens(seq, toks)
        return slots, pairs

    def free_seq(self, seq: int) -> None:
        if seq not in self.tables:
            raise ValueError("bad free")
        zero = []
        for b in self.tables.pop(seq):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                zero.append(b)
        del self.lens[seq]
        self.tokens.pop(seq, None)
        for b in zero:
            if self.key_of[b] is None:
                self.free.append(b)
        for b in reversed(zero):
            if self.key_of[b] is not None:
                self.evictable[b] = None

    # -- queries -------------------------------------------------------------------
    def stats(self) -> Dict[str, int]:
        st = super().stats()
        st["cached_blocks"] = sum(1 for k in self.key_of if k is not None)
        st["evictable_blocks"] = len(self.evictable)
        st["hit_tokens"] = self.hit_tokens
        st["query_tokens"] = self.query_tokens
        return st
