"""CPU checks of the library's shared-prefix row builder (pkv_prefix_rows): runs of
consecutive sequences whose tables start with the same block ids become one prefix row
plus a row per member for the rest; every context is covered exactly once."""
import numpy as np
import pytest


def _rows(tables, lens, B, g, min_blocks=1):
    import paged_kv_cache_104_amd as pkv

    return pkv.prefix_rows(np.asarray(tables), np.asarray(lens), B, g, min_blocks)


def _check_cover(tables, lens, B, g, min_blocks, rows, seq_rows):
    """Every sequence's tokens [0, len) are its prefix row's [0, te) (when it has one) and
    its own row's [tb, len), with te == tb; prefix rows hold the same block ids for all
    their members; member counts and shared sizes obey the limits."""
    tables = np.asarray(tables)
    S = len(lens)
    assert seq_rows.shape == (S, 4)
    owned = np.zeros(len(rows), dtype=int)
    for s in range(S):
        own, pre, member, _ = seq_rows[s]
        seq, tb, te, m = rows[own]
        assert seq == s and te == -1 and m == 1
        owned[own] += 1
        if pre < 0:
            assert tb == 0
            continue
        ps, ptb, pte, pm = rows[pre]
        assert ptb == 0 and pte == tb and tb % B == 0
        assert 0 <= member < pm and ps + member == s
        assert tb // B >= max(1, min_blocks) and tb < lens[s]       # own row is never empty
        assert np.array_equal(tables[s, :tb // B], tables[ps, :tb // B])
        assert (tables[s, :tb // B] >= 0).all()
        assert 2 <= pm <= 16 // g
    prefix = [r for r in range(len(rows)) if rows[r][3] > 1]
    assert all(owned[r] == 0 for r in prefix)
    assert sorted(np.flatnonzero(owned).tolist() + prefix) == list(range(len(rows)))


def test_families_singletons_and_order():
    B = 4
    t = np.array([[7, 8, 9, -1], [7, 8, 10, -1], [7, 8, 11, 12], [3, 4, -1, -1],
                  [5, 6, -1, -1], [5, 6, 2, -1]], dtype=np.int32)
    lens = np.array([10, 12, 14, 6, 7, 9], dtype=np.int32)
    rows, sr = _rows(t, lens, B, 2)
    assert rows.tolist() == [[0, 0, 8, 3], [0, 8, -1, 1], [1, 8, -1, 1], [2, 8, -1, 1],
                             [3, 0, -1, 1],
                             [4, 0, 4, 2], [4, 4, -1, 1], [5, 4, -1, 1]]
    assert sr.tolist() == [[1, 0, 0, 0], [2, 0, 1, 0], [3, 0, 2, 0], [4, -1, 0, 0],
                           [6, 5, 0, 0], [7, 5, 1, 0]]
    _check_cover(t, lens, B, 2, 1, rows, sr)


def test_shared_part_stays_below_every_members_last_block():
    """Sequence 4 holds blocks 5, 6 and its 7th token sits in block 6: it can share block 5
    only, and so does its partner, whose third block would otherwise also match."""
    B = 4
    t = np.array([[5, 6, 1], [5, 6, 2]], dtype=np.int32)
    rows, sr = _rows(t, [7, 10], B, 1)
    assert rows.tolist() == [[0, 0, 4, 2], [0, 4, -1, 1], [1, 4, -1, 1]]
    # a context ending on a block boundary shares all its full blocks but the last
    rows, _ = _rows(t, [8, 10], B, 1)
    assert rows[0].tolist() == [0, 0, 4, 2]
    rows, _ = _rows(t, [9, 10], B, 1)
    assert rows[0].tolist() == [0, 0, 8, 2]


def test_member_limit_splits_large_families():
    B, g = 16, 4                                   # 16 / 4 = 4 members per prefix row
    S = 10
    t = np.full((S, 4), -1, dtype=np.int32)
    t[:, :2] = [40, 41]
    t[:, 2] = np.arange(S)
    lens = np.full(S, 40, dtype=np.int32)
    rows, sr = _rows(t, lens, B, g)
    pre = rows[rows[:, 3] > 1]
    assert pre[:, 3].tolist() == [4, 4, 2] and pre[:, 0].tolist() == [0, 4, 8]
    _check_cover(t, lens, B, g, 1, rows, sr)
    # groups of 16 heads leave one column per member: no sharing at all
    rows, sr = _rows(t, lens, B, 16)
    assert len(rows) == S and (sr[:, 1] == -1).all()


def test_minimum_shared_blocks():
    B = 8
    t = np.array([[1, 2, 3, 9], [1, 2, 4, 9]], dtype=np.int32)
    lens = np.array([30, 30], dtype=np.int32)
    assert _rows(t, lens, B, 2, 2)[0][0].tolist() == [0, 0, 16, 2]
    rows, sr = _rows(t, lens, B, 2, 3)
    assert len(rows) == 2 and (rows[:, 1] == 0).all()


def test_unused_table_entries_are_not_shared():
    t = np.array([[-1, -1], [-1, -1]], dtype=np.int32)
    rows, sr = _rows(t, [0, 0], 16, 1)
    assert rows.tolist() == [[0, 0, -1, 1], [1, 0, -1, 1]]


@pytest.mark.parametrize("seed", range(6))
def test_random_batches_cover_every_context(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([8, 16, 32]))
    g = int(rng.choice([1, 2, 4, 8]))
    S = int(rng.integers(1, 60))
    maxb = 12
    t = np.full((S, maxb), -1, dtype=np.int32)
    lens = np.zeros(S, dtype=np.int32)
    nxt = 0
    s = 0
    while s < S:
        fam = int(rng.integers(1, 7))
        shared = int(rng.integers(0, 6))
        ids = np.arange(nxt, nxt + shared)
        nxt += shared
        for _ in range(min(fam, S - s)):
            n = int(rng.integers(max(shared, 1), maxb + 1))
            t[s, :shared] = ids[:n]
            t[s, shared:n] = np.arange(nxt, nxt + n - shared)
            nxt += n - shared
            lens[s] = int(rng.integers((n - 1) * B + 1, n * B + 1))
            s += 1
    mb = int(rng.integers(1, 3))
    rows, sr = _rows(t, lens, B, g, mb)
    _check_cover(t, lens, B, g, mb, rows, sr)


def test_argument_validation():
    import paged_kv_cache_104_amd as pkv

    t = np.zeros((2, 2), dtype=np.int32)
    for bad in (dict(group=0), dict(group=17), dict(block_size=0)):
        kw = dict(block_size=16, group=2)
        kw.update(bad)
        with pytest.raises(Exception):
            pkv.prefix_rows(t, np.array([3, 3]), kw["block_size"], kw["group"], 1)
