"""Pins of the oracle's prefix caching (CPU).

The pages fix what a cached block is (the KV of its tokens given every earlier
token) and that equal keys mean equal blocks; the pins check the worked cases
that follow from that, and a brute-force shadow of what every physical slot
holds checks the one property prefix caching must keep: every position a live
sequence reads holds the KV computed for that sequence's own token prefix.
"""
import random

import pytest

from oracle.allocator import NoMemory
from oracle.prefix_cache import PrefixCachingAllocator


class Shadow:
    """What each physical slot holds: the token prefix whose last token's KV was
    written there (KV at position p depends on tokens 0..p)."""

    def __init__(self, alloc):
        self.a = alloc
        self.B = alloc.block_size
        self.content = {}

    def write(self, seq, start, stop):
        t = self.a.tokens[seq]
        table = self.a.tables[seq]
        for p in range(start, stop):
            self.content[(table[p // self.B], p % self.B)] = tuple(t[: p + 1])

    def copy(self, pairs):
        for src, dst in pairs:
            for o in range(self.B):
                if (src, o) in self.content:
                    self.content[(dst, o)] = self.content[(src, o)]

    def check(self):
        for seq, t in self.a.tokens.items():
            table = self.a.tables[seq]
            for p in range(len(t)):
                got = self.content.get((table[p // self.B], p % self.B))
                assert got == tuple(t[: p + 1]), (seq, p)

    # operations that mirror the allocator and write what a real engine would
    def add(self, seq, toks):
        table, cached = self.a.add_seq_tokens(seq, toks)
        self.write(seq, cached, len(toks))
        return table, cached

    def append_batch(self, seqs, toks):
        starts = [self.a.lens[s] for s in seqs]
        slots, pairs = self.a.append_batch_tokens(seqs, toks)
        self.copy(pairs)
        for s, p in zip(seqs, starts):
            self.write(s, p, p + 1)
        return slots, pairs


def test_identical_prompts_share_every_full_block():
    """Same prompt twice: the full blocks are the first request's; the partial last
    block is not shared (only full blocks have keys)."""
    a = PrefixCachingAllocator(16, 4)
    sh = Shadow(a)
    prompt = [5, 1, 8, 2, 9, 9, 3, 7, 4, 6]          # 2 full blocks + 2 tokens
    t1, c1 = sh.add(1, prompt)
    t2, c2 = sh.add(2, prompt)
    assert c1 == 0 and c2 == 8
    assert t2[:2] == t1[:2] and t2[2] != t1[2]
    assert [a.ref[b] for b in t1] == [2, 2, 1]
    assert a.stats()["hit_tokens"] == 8 and a.stats()["query_tokens"] == 20
    sh.check()


def test_multi_turn_reuses_the_previous_round():
    """Round 2's prompt is round 1's prompt + reply + a new turn: every full block of
    round 1 comes back from the cache, even after round 1 was released."""
    a = PrefixCachingAllocator(32, 4)
    sh = Shadow(a)
    prompt = list(range(100, 110))                    # 10 tokens
    sh.add(1, prompt)
    reply = [7, 7, 3, 1, 2, 8]                        # decode fills blocks 2 and 3
    for t in reply:
        sh.append_batch([1], [t])
    sh.check()
    conv = a.tokens[1]
    assert len(conv) == 16
    t1 = list(a.tables[1])
    a.free_seq(1)
    assert all(a.ref[b] == 0 for b in t1)
    assert list(a.evictable) == t1[::-1]              # last block first
    t2, cached = sh.add(2, conv + [42, 43, 44])
    assert cached == 16 and t2[:4] == t1
    assert all(a.ref[b] == 1 for b in t1) and not a.evictable
    sh.check()


def test_a_differing_token_ends_the_shared_prefix():
    """A token that differs inside block i changes the key of block i and of every later
    block (they include it): blocks before i are shared, none after."""
    a = PrefixCachingAllocator(32, 4)
    sh = Shadow(a)
    base = list(range(16))
    t1, _ = sh.add(1, base)
    other = list(base)
    other[9] = 99                                      # inside block 2
    t2, cached = sh.add(2, other)
    assert cached == 8 and t2[:2] == t1[:2]
    assert set(t2[2:]).isdisjoint(t1)
    # block 3 holds the same tokens as in `base` but a different prefix: not shared
    assert other[12:16] == base[12:16] and t2[3] != t1[3]
    sh.check()


def test_lookup_stops_at_the_first_miss():
    """A cached block is reachable only through its whole chain of prefixes: when block
    0's key is gone, a still-cached block 1 with the right key is not used.

    (Releases put a sequence's last blocks first in the queue, so an ancestor loses its
    key before a descendant only through a duplicate: here C's first block repeats A's
    key, stays uncached, and C's second block is cached under it.)"""
    a = PrefixCachingAllocator(8, 2, free_order=range(8))
    a.add_seq_tokens(1, [1])                           # A: block 0
    a.add_seq_tokens(2, [1])                           # C: block 1
    a.append_batch_tokens([1, 2], [2, 2])              # block 0 takes (1, 2); block 1 does not
    assert a.cache[(1, 2)] == 0 and a.key_of[1] is None
    a.append_batch_tokens([2], [3])
    a.append_batch_tokens([2], [4])                    # block 2 takes (1, 2, 3, 4)
    assert a.cache[(1, 2, 3, 4)] == 2
    a.free_seq(1)
    a.free_seq(2)
    assert list(a.evictable) == [0, 2] and list(a.free)[-1] == 1
    a.add_seq_tokens(3, [9] * 14)                      # six free blocks, then evicts block 0
    assert (1, 2) not in a.cache and a.cache[(1, 2, 3, 4)] == 2
    assert a.lookup([1, 2, 3, 4]) == []
    assert a.lookup([9] * 6) == a.tables[3][:3]


def test_eviction_takes_the_block_released_longest_ago():
    a = PrefixCachingAllocator(6, 2, free_order=range(6))
    sh = Shadow(a)
    sh.add(1, [1, 1, 2, 2])                            # blocks 0, 1
    sh.add(2, [3, 3, 4, 4])                            # blocks 2, 3
    a.free_seq(1)                                      # evictable [1, 0]
    a.free_seq(2)                                      # evictable [1, 0, 3, 2]
    assert list(a.evictable) == [1, 0, 3, 2]
    t3, cached = sh.add(3, [9, 9, 8, 8, 7, 7])         # free 4, 5, then evict 1
    assert cached == 0 and t3 == [4, 5, 1]
    # block 1 lost request 1's key and now holds request 3's full last block
    assert (1, 1, 2, 2) not in a.cache and a.key_of[1] == (9, 9, 8, 8, 7, 7)
    # request 1's first block survived (it outlives the block that extends it)
    t4, cached = sh.add(4, [1, 1, 2, 2])
    assert cached == 2 and t4[0] == 0
    sh.check()
    # no room: nothing changes
    before = (dict(a.tables), list(a.evictable), list(a.free), list(a.ref))
    with pytest.raises(NoMemory):
        a.add_seq_tokens(5, list(range(100, 110)))
    assert before == (dict(a.tables), list(a.evictable), list(a.free), list(a.ref))


def test_first_block_keeps_its_key():
    """Two sequences filling blocks with equal keys in one batch: the first keeps the key."""
    a = PrefixCachingAllocator(8, 2)
    a.add_seq_tokens(1, [4])
    a.add_seq_tokens(2, [4])                            # partial blocks are never shared
    t1, t2 = a.tables[1][0], a.tables[2][0]
    assert t1 != t2
    a.append_batch_tokens([1, 2], [5, 5])
    assert a.cache[(4, 5)] == t1 and a.key_of[t2] is None
    a.free_seq(2)
    assert t2 in a.free and t2 not in a.evictable


def test_forks_and_copy_on_write_keep_prefixes_right():
    a = PrefixCachingAllocator(32, 4)
    sh = Shadow(a)
    sh.add(1, [1, 2, 3, 4, 5, 6])                      # 1 full block + 2 tokens
    a.fork(1, 2)
    a.fork(1, 3)
    sh.append_batch([1, 2, 3], [10, 20, 30])           # partial shared block: 2 copies
    sh.append_batch([1, 2, 3], [11, 21, 31])           # blocks fill: three distinct keys
    sh.check()
    keys = {a.key_of[a.tables[s][1]] for s in (1, 2, 3)}
    assert keys == {(1, 2, 3, 4, 5, 6, 10, 11), (1, 2, 3, 4, 5, 6, 20, 21),
                    (1, 2, 3, 4, 5, 6, 30, 31)}
    _, cached = sh.add(4, [1, 2, 3, 4, 5, 6, 20, 21, 0])
    assert cached == 8 and a.tables[4][:2] == a.tables[2][:2]
    sh.check()


@pytest.mark.parametrize("seed", range(40))
def test_random_operations_keep_every_prefix_right(seed):
    """Random prompts built from a few shared stems, decode appends, forks and releases
    in a pool small enough to evict: every live position always holds its own prefix's
    KV, counts match the tables, and the free, evictable and live sets partition the pool."""
    rng = random.Random(seed)
    B = rng.choice([2, 4, 8])
    N = rng.randint(12, 40)
    a = PrefixCachingAllocator(N, B, free_order=rng.sample(range(N), N))
    sh = Shadow(a)
    stems = [[rng.randint(0, 3) for _ in range(rng.randint(0, 3 * B))] for _ in range(4)]
    live, next_id = [], 0
    for _ in range(300):
        op = rng.random()
        try:
            if op < 0.3 or not live:
                toks = rng.choice(stems) + [rng.randint(0, 3) for _ in range(rng.randint(0, 2 * B))]
                sh.add(next_id, toks)
                live.append(next_id)
                next_id += 1
            elif op < 0.6:
                k = rng.randint(1, len(live))
                seqs = sorted(rng.sample(live, k))
                sh.append_batch(seqs, [rng.randint(0, 3) for _ in seqs])
            elif op < 0.7:
                p = rng.choice(live)
                a.fork(p, next_id)
                live.append(next_id)
                next_id += 1
            else:
                s = rng.choice(live)
                a.free_seq(s)
                live.remove(s)
        except NoMemory:
            pass
        sh.check()
        ref = [0] * N
        for t in a.tables.values():
            for b in t:
                ref[b] += 1
        assert ref == a.ref
        used = {b for b in range(N) if ref[b] > 0}
        assert set(a.free).isdisjoint(used) and set(a.evictable).isdisjoint(used)
        assert set(a.free).isdisjoint(a.evictable)
        assert len(a.free) + len(a.evictable) + len(used) == N
        assert all(a.key_of[b] is not None for b in a.evictable)
        assert all(a.cache[k] == b for b, k in enumerate(a.key_of) if k is not None)
        assert len(a.cache) == sum(1 for k in a.key_of if k is not None)


# --------------------------------------------------------------------------- mutations
# Plausible mistakes planted in the prefix-caching oracle (on the CPU); each must make
# at least one of the pins above fail.

def _key_block_only(self, toks, i):
    B = self.block_size
    return tuple(int(t) for t in toks[i * B:(i + 1) * B])


def _lookup_skips_misses(self, toks):
    hits = []
    for i in range(len(toks) // self.block_size):
        b = self.cache.get(self.key(toks, i))
        if b is not None:
            hits.append(b)
    return hits


def _pop_most_recent(self):
    if self.free:
        b = self.free.popleft()
    else:
        b, _ = self.evictable.popitem(last=True)
        del self.cache[self.key_of[b]]
        self.key_of[b] = None
    self.ref[b] = 1
    return b


def _note_partial_too(self, seq, new_tokens):
    if seq not in self.tokens:
        return
    self.tokens[seq].extend(int(t) for t in new_tokens)
    n = len(self.tokens[seq])
    for i in range(-(-n // self.block_size)):
        k = tuple(self.tokens[seq][: min(n, (i + 1) * self.block_size)])
        b = self.tables[seq][i]
        if k not in self.cache and self.key_of[b] is None:
            self.cache[k] = b
            self.key_of[b] = k


def _free_in_logical_order(self, seq):
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
        else:
            self.evictable[b] = None


def _free_forgets_keys(self, seq):
    for b in self.tables.pop(seq):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if self.key_of[b] is not None:
                del self.cache[self.key_of[b]]
                self.key_of[b] = None
            self.free.append(b)
    del self.lens[seq]
    self.tokens.pop(seq, None)


_PINS = [test_identical_prompts_share_every_full_block, test_multi_turn_reuses_the_previous_round,
         test_a_differing_token_ends_the_shared_prefix, test_lookup_stops_at_the_first_miss,
         test_eviction_takes_the_block_released_longest_ago, test_first_block_keeps_its_key,
         test_forks_and_copy_on_write_keep_prefixes_right]
_PINS += [lambda s=s: test_random_operations_keep_every_prefix_right(s) for s in range(10)]

MUTATIONS = {
    "key without the earlier tokens": ("key", _key_block_only),
    "lookup skips over misses": ("lookup", _lookup_skips_misses),
    "evicts the most recently released block": ("_pop", _pop_most_recent),
    "partial blocks get keys": ("_note_tokens", _note_partial_too),
    "released blocks queued first block first": ("free_seq", _free_in_logical_order),
    "released blocks lose their keys": ("free_seq", _free_forgets_keys),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_prefix_cache_mutation_is_caught(name, monkeypatch):
    attr, value = MUTATIONS[name]
    monkeypatch.setattr(PrefixCachingAllocator, attr, value)
    caught = False
    for pin in _PINS:
        try:
            pin()
        except Exception:
            caught = True
            break
    assert caught, name
