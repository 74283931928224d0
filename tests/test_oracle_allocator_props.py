"""Invariants of the oracle's block allocator under random operation sequences.

What the pages fix, checked as properties: a block is counted once per table
that holds it; a free block is held by nobody; a sequence holds exactly
ceil(len / B) blocks; a token is always written into a block nobody else holds
(copy-on-write); two sequences share a slot only at the same position of a
shared block; running out of blocks changes nothing.
"""
import copy

from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import allocator as oalloc

OPS = st.lists(
    st.tuples(st.sampled_from(["add", "fork", "append", "batch", "extend", "free"]),
              st.integers(0, 7), st.integers(0, 7), st.integers(0, 40)),
    min_size=1, max_size=60)


def _state(a):
    return (list(a.free), list(a.ref), {k: list(v) for k, v in a.tables.items()}, dict(a.lens))


def _check(a):
    B = a.block_size
    count = [0] * a.num_blocks
    for t in a.tables.values():
        for b in t:
            count[b] += 1
    assert count == a.ref
    assert len(set(a.free)) == len(a.free)
    assert all(a.ref[b] == 0 for b in a.free)
    assert len(a.free) + sum(1 for r in a.ref if r > 0) == a.num_blocks
    for s, t in a.tables.items():
        assert len(t) == -(-a.lens[s] // B)
    owner = {}
    for s, t in a.tables.items():
        for p in range(a.lens[s]):
            sl = a.slot(s, p)
            if sl in owner:
                s2, p2 = owner[sl]
                assert p2 == p and a.ref[sl // B] >= 2
            owner[sl] = (s, p)


@settings(max_examples=300, deadline=None)
@given(OPS, st.integers(1, 5), st.integers(4, 40))
def test_allocator_invariants(ops, B, N):
    a = oalloc.BlockAllocator(N, B)
    for kind, x, y, n in ops:
        before = _state(a)
        try:
            if kind == "add":
                a.add_seq(x, n)
            elif kind == "fork":
                a.fork(x, y)
            elif kind == "append":
                slot, _ = a.append(x)
                assert a.ref[slot // B] == 1            # written block is private
            elif kind == "batch":
                seqs = sorted({x, y})
                slots, _ = a.append_batch(seqs)
                for sl in slots:
                    assert a.ref[sl // B] == 1
            elif kind == "extend":
                slots, pairs = a.extend(x, n % 9)
                assert len(pairs) <= 1
                for sl in slots:
                    assert a.ref[sl // B] == 1
            else:
                a.free_seq(x)
        except ValueError:
            assert _state(a) == before
        except oalloc.NoMemory:
            assert _state(a) == before                  # all-or-nothing
        _check(a)
