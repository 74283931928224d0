"""Pins of the oracle's swapping (CPU).

What the page fixes is the round trip: a swapped-out sequence's KV leaves the
device (its blocks become free there) and comes back intact.  A shadow of what
every device and host slot holds, driven through random operation sequences
with the copies each operation returns applied in order, checks that every
position of every sequence -- resident or swapped out -- still holds what was
written for it, and that the decode of a swapped-in batch equals the decode
before it left.
"""
import random

import numpy as np
import pytest

from oracle import attention as oattn
from oracle import cache as ocache
from oracle.allocator import NoMemory
from oracle.swap import SwappingAllocator, SwappingPrefixCachingAllocator


class Shadow:
    """Value held by every slot of the device ('d') and host ('h') pools; a sequence's
    expected values follow it through forks."""

    def __init__(self, a):
        self.a, self.B = a, a.block_size
        self.slot = {}
        self.want = {}
        self.n = 0

    def _fresh(self):
        self.n += 1
        return self.n

    def write(self, seq, start, stop):
        t = self.a.tables[seq]
        for p in range(start, stop):
            v = self._fresh()
            self.slot[("d", t[p // self.B], p % self.B)] = v
            self.want[seq][p] = v

    def move(self, pairs, src, dst):
        for s, d in pairs:
            for o in range(self.B):
                if (src, s, o) in self.slot:
                    self.slot[(dst, d, o)] = self.slot[(src, s, o)]

    def check(self):
        for seq, w in self.want.items():
            where = "h" if seq in self.a.swapped else "d"
            t = self.a.tables[seq]
            for p, v in w.items():
                assert self.slot.get((where, t[p // self.B], p % self.B)) == v, (seq, p)

    # mirrored operations
    def add(self, seq, n):
        self.a.add_seq(seq, n)
        self.want[seq] = {}
        self.write(seq, 0, n)

    def fork(self, p, c):
        self.a.fork(p, c)
        self.want[c] = dict(self.want[p])

    def append_batch(self, seqs):
        starts = [self.a.lens[s] for s in seqs]
        _, pairs = self.a.append_batch(seqs)
        self.move(pairs, "d", "d")
        for s, p in zip(seqs, starts):
            self.write(s, p, p + 1)

    def swap_out(self, seqs):
        self.move(self.a.swap_out(seqs), "d", "h")

    def swap_in(self, seqs):
        self.move(self.a.swap_in(seqs), "h", "d")

    def free(self, seq):
        self.a.free_seq(seq)
        del self.want[seq]


def test_round_trip_frees_device_blocks_and_restores_the_data():
    a = SwappingAllocator(12, 4, num_host_blocks=8)
    sh = Shadow(a)
    sh.add(1, 10)
    sh.add(2, 5)
    before = len(a.free)
    sh.swap_out([1])
    assert len(a.free) == before + 3 and len(a.host_free) == 5
    assert a.stats()["swapped_seqs"] == 1 and a.stats()["tokens"] == 5
    sh.add(3, 20)                                    # the freed device blocks serve another request
    sh.check()
    sh.swap_in([1])
    sh.check()
    assert len(a.host_free) == 8 and not a.swapped


def test_forked_samples_move_together_once():
    a = SwappingAllocator(16, 4, num_host_blocks=16)
    sh = Shadow(a)
    sh.add(1, 6)
    sh.fork(1, 2)
    sh.fork(1, 3)
    sh.append_batch([1, 2, 3])                       # copy-on-write: 2 copies of block 1
    shared = a.tables[1][0]
    assert a.ref[shared] == 3
    sh.swap_out([1, 2, 3])
    h = a.tables[1][0]
    assert a.tables[2][0] == a.tables[3][0] == h and a.host_ref[h] == 3
    assert len(a.host_free) == 16 - 4                # 1 shared + 1 in place + 2 copies
    sh.swap_in([3, 1, 2])
    d = a.tables[1][0]
    assert a.tables[2][0] == a.tables[3][0] == d and a.ref[d] == 3
    sh.check()
    sh.append_batch([1, 2, 3])                       # sharing still behaves
    sh.check()


def test_a_set_must_own_its_blocks():
    a = SwappingAllocator(16, 4, num_host_blocks=16)
    a.add_seq(1, 6)
    a.fork(1, 2)
    with pytest.raises(ValueError):
        a.swap_out([1])                              # block 0 is also sample 2's
    with pytest.raises(ValueError):
        a.swap_in([1])                               # resident
    a.swap_out([1, 2])
    for op in (lambda: a.append(1), lambda: a.fork(1, 5), lambda: a.slots(1, 0, 1),
               lambda: a.block_tables([2], 4), lambda: a.append_batch([2])):
        with pytest.raises(ValueError):
            op()
    a.free_seq(1)                                    # releasing a swapped-out sequence
    assert a.host_ref[a.tables[2][0]] == 1
    a.free_seq(2)
    assert len(a.host_free) == 16 and a.stats()["swapped_seqs"] == 0


def test_no_room_changes_nothing():
    a = SwappingAllocator(6, 4, num_host_blocks=2)
    a.add_seq(1, 12)                                 # 3 blocks
    snap = lambda: (dict(a.tables), list(a.free), list(a.ref), list(a.host_free),
                    list(a.host_ref), set(a.swapped))
    s0 = snap()
    with pytest.raises(NoMemory):
        a.swap_out([1])
    assert snap() == s0
    b = SwappingAllocator(4, 4, num_host_blocks=4)
    b.add_seq(1, 12)
    b.swap_out([1])
    b.add_seq(2, 8)                                  # device now too full for 1 to return
    s1 = (dict(b.tables), list(b.free), list(b.host_free))
    with pytest.raises(NoMemory):
        b.swap_in([1])
    assert (dict(b.tables), list(b.free), list(b.host_free)) == s1


def test_decode_after_a_round_trip_is_unchanged():
    """The attention of a swapped-in sequence over its new blocks equals the attention
    before it left (same values in the same logical order)."""
    rng = np.random.default_rng(0)
    B, H, D = 4, 2, 8
    a = SwappingAllocator(10, B, free_order=rng.permutation(10), num_host_blocks=10)
    kp, vp = ocache.new_pools(10, H, B, D, "f32")
    hk, hv = ocache.new_pools(10, H, B, D, "f32")
    a.add_seq(1, 11)
    k = rng.standard_normal((11, H, D)).astype(np.float32)
    v = rng.standard_normal((11, H, D)).astype(np.float32)
    ocache.reshape_and_cache(kp, vp, k, v, a.slots(1, 0, 11), "f32", "f32")
    q = rng.standard_normal((1, 4, D))
    t, n = a.block_tables([1], 3)
    ref = oattn.paged_decode(q, kp, vp, t, n, 0.3, "f32", 1.0, 1.0)
    ocache.swap_blocks(kp, vp, hk, hv, a.swap_out([1]))
    kp[:] = np.nan                                   # the device blocks are reused by others
    vp[:] = np.nan
    ocache.swap_blocks(hk, hv, kp, vp, a.swap_in([1]))
    t2, n2 = a.block_tables([1], 3)
    assert np.array_equal(oattn.paged_decode(q, kp, vp, t2, n2, 0.3, "f32", 1.0, 1.0), ref)


def test_swap_blocks_checks_pairs():
    kp, vp = ocache.new_pools(4, 1, 2, 4, "bf16")
    hk, hv = ocache.new_pools(2, 1, 2, 4, "bf16")
    for bad in ([[4, 0]], [[0, 2]], [[0, 1], [1, 1]], [[-1, 0]]):
        with pytest.raises(ValueError):
            ocache.swap_blocks(kp, vp, hk, hv, bad)
    kp[:] = 7
    ocache.swap_blocks(kp, vp, hk, hv, [[3, 0]])
    assert (hk[0] == 7).all() and np.isnan(ocache.codec.bf16_to_f64(hk[1])).all()


def test_prefix_cached_blocks_lose_their_keys():
    a = SwappingPrefixCachingAllocator(16, 2, num_host_blocks=8)
    a.add_seq_tokens(1, [1, 2, 3, 4, 5])
    assert len(a.cache) == 2
    a.swap_out([1])
    assert not a.cache and all(k is None for k in a.key_of)
    assert a.lookup([1, 2, 3, 4]) == []
    a.swap_in([1])
    assert not a.cache
    a.append_batch_tokens([1], [6])                  # the block it fills registers again
    assert a.cache == {(1, 2, 3, 4, 5, 6): a.tables[1][2]}


@pytest.mark.parametrize("seed", range(30))
def test_random_operations_keep_every_sequence_intact(seed):
    rng = random.Random(seed)
    B = rng.choice([1, 2, 4])
    N, Nh = rng.randint(6, 30), rng.randint(2, 30)
    a = SwappingAllocator(N, B, free_order=rng.sample(range(N), N), num_host_blocks=Nh)
    sh = Shadow(a)
    families = {}                                   # root -> members (forks move together)
    nxt = 0
    for _ in range(250):
        op = rng.random()
        resident = [r for r, m in families.items() if not (set(m) & a.swapped)]
        out = [r for r, m in families.items() if set(m) <= a.swapped]
        try:
            if op < 0.25 or not families:
                sh.add(nxt, rng.randint(0, 4 * B))
                families[nxt] = [nxt]
                nxt += 1
            elif op < 0.35 and resident:
                r = rng.choice(resident)
                sh.fork(rng.choice(families[r]), nxt)
                families[r].append(nxt)
                nxt += 1
            elif op < 0.6 and resident:
                rs = rng.sample(resident, rng.randint(1, len(resident)))
                sh.append_batch(sorted(s for r in rs for s in families[r]))
            elif op < 0.75 and resident:
                rs = rng.sample(resident, rng.randint(1, len(resident)))
                sh.swap_out([s for r in rs for s in families[r]])
            elif op < 0.88 and out:
                rs = rng.sample(out, rng.randint(1, len(out)))
                sh.swap_in([s for r in rs for s in families[r]])
            else:
                r = rng.choice(list(families))
                for s in families.pop(r):
                    sh.free(s)
        except NoMemory:
            pass
        sh.check()
        dev = [0] * N
        host = [0] * Nh
        for s, t in a.tables.items():
            for b in t:
                (host if s in a.swapped else dev)[b] += 1
        assert dev == a.ref and host == a.host_ref
        assert len(a.free) + sum(1 for r in dev if r) == N
        assert len(a.host_free) + sum(1 for r in host if r) == Nh


# --------------------------------------------------------------------------- mutations

def _out_maps_every_holder(self, seqs):
    """Mistake: a shared block gets a host block per holder."""
    seqs = [int(s) for s in seqs]
    pairs = []
    for s in seqs:
        self._resident(s)
    need = sum(len(self.tables[s]) for s in seqs)
    if need > len(self.host_free):
        raise NoMemory(seqs)
    freed = []
    for s in seqs:
        new = []
        for b in self.tables[s]:
            h = self.host_free.popleft()
            self.host_ref[h] = 1
            pairs.append((b, h))
            new.append(h)
            if b not in freed:
                freed.append(b)
        self.tables[s] = new
        self.swapped.add(s)
    for b in freed:
        self.ref[b] = 0
        self.free.append(b)
    return pairs


def _in_forgets_counts(self, seqs):
    pairs = type(self).__mro__[1].swap_in(self, seqs)
    for _, d in pairs:
        self.ref[d] = 1
    return pairs


def _out_keeps_device_blocks(self, seqs):
    free_before = list(self.free)
    pairs = type(self).__mro__[1].swap_out(self, seqs)
    self.free.clear()
    self.free.extend(free_before)
    return pairs


def _in_reversed_pairs(self, seqs):
    return [(d, h) for h, d in type(self).__mro__[1].swap_in(self, seqs)]


_PINS = [test_round_trip_frees_device_blocks_and_restores_the_data,
         test_forked_samples_move_together_once, test_a_set_must_own_its_blocks,
         test_no_room_changes_nothing, test_decode_after_a_round_trip_is_unchanged]
_PINS += [lambda s=s: test_random_operations_keep_every_sequence_intact(s) for s in range(8)]

MUTATIONS = {
    "a shared block moves once per holder": ("swap_out", _out_maps_every_holder),
    "swap-in drops the counts of shared blocks": ("swap_in", _in_forgets_counts),
    "swap-out does not free the device blocks": ("swap_out", _out_keeps_device_blocks),
    "swap-in copies the wrong way": ("swap_in", _in_reversed_pairs),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_swap_mutation_is_caught(name, monkeypatch):
    attr, value = MUTATIONS[name]
    monkeypatch.setattr(SwappingAllocator, attr, value)
    caught = False
    for pin in _PINS:
        try:
            pin()
        except Exception:
            caught = True
            break
    assert caught, name
