"""Pins of the oracle's QUEST block selection (CPU).

The page fixes the bound (channel-wise min / max keys, the larger product per
channel, summed) and that the top-K blocks by it are attended.  The pins check
it against what the mathematics fixes: the bound is never below the best score
in its block and equals it for a one-token block; the sign rule on a worked
two-channel example; a budget that covers the context gives plain attention; a
block the query points at is the one kept.
"""
import numpy as np
import pytest

from oracle import allocator as oalloc
from oracle import attention as oattn
from oracle import cache as ocache
from oracle import quest


def _setup(rng, lens, H=2, D=8, B=4, N=80, k=None, order=None):
    a = oalloc.BlockAllocator(N, B, order)
    kp, vp = ocache.new_pools(N, H, B, D, "f32")
    for s, n in enumerate(lens):
        a.add_seq(s, n)
        kk = rng.standard_normal((n, H, D)).astype(np.float32) if k is None else k[s]
        vv = rng.standard_normal((n, H, D)).astype(np.float32)
        ocache.reshape_and_cache(kp, vp, kk, vv, a.slots(s, 0, n), "f32", "f32")
    t, l = a.block_tables(list(range(len(lens))), max(-(-n // B) for n in lens))
    return a, kp, vp, t, l


def test_bound_never_below_the_best_score_and_tight_for_one_token():
    rng = np.random.default_rng(0)
    for trial in range(200):
        n = int(rng.integers(1, 9))
        D = int(rng.integers(1, 6))
        K = rng.standard_normal((n, D))
        q = rng.standard_normal(D) * rng.choice([-3, 1, 3])
        u = quest.bounds(q, K.min(0)[None], K.max(0)[None])[0, 0]
        assert u >= (K @ q).max() - 1e-12
        if n == 1:
            assert u == pytest.approx(float(K[0] @ q), abs=1e-12)


def test_sign_rule_worked_example():
    """q = (2, -3); keys (1, 5) and (4, -1): min = (1, -1), max = (4, 5).  Channel 0 takes
    2 * 4 = 8 (max), channel 1 takes -3 * -1 = 3 (min, the query being negative): 11, which is
    exactly the second key's score 2 * 4 + 3 = 11."""
    K = np.array([[1.0, 5.0], [4.0, -1.0]])
    u = quest.bounds([2.0, -3.0], K.min(0)[None], K.max(0)[None])
    assert u.tolist() == [[11.0]]
    assert (K @ np.array([2.0, -3.0])).tolist() == [-13.0, 11.0]


def test_budget_covering_the_context_is_plain_attention():
    rng = np.random.default_rng(1)
    a, kp, vp, t, l = _setup(rng, [37, 9, 16])
    q = rng.standard_normal((3, 4, 8))
    dense = oattn.paged_decode(q, kp, vp, t, l, 0.3, "f32")
    assert np.array_equal(quest.quest_decode(q, kp, vp, t, l, 0.3, 2, 10, "f32"), dense)
    assert not np.allclose(quest.quest_decode(q, kp, vp, t, l, 0.3, 2, 2, "f32"), dense)


def test_the_block_the_query_points_at_is_kept():
    """The page's intuition ("A is B. C is D. A is" -> B): one block holds a key aligned with the
    query; with a budget of one block it is the one kept, and the output is its value."""
    rng = np.random.default_rng(2)
    D, B, n = 8, 4, 40
    q = rng.standard_normal(D)
    k = rng.standard_normal((n, 1, D)).astype(np.float32) * 0.1
    k[22, 0] = (5.0 * q).astype(np.float32)                # block 5, position 2
    a, kp, vp, t, l = _setup(rng, [n], H=1, D=D, B=B, k=[k])
    chosen = quest.selected_blocks(q[None, None], kp, t, l, 1, 1, "f32")
    assert chosen[(0, 0)].tolist() == [5]
    out = quest.quest_decode(q[None, None], kp, vp, t, l, 1.0, 1, 1, "f32")
    V = oattn.gather_values(vp, t[0], n, 0)
    assert np.allclose(out[0, 0], V[22], atol=1e-3)


def test_group_selection_takes_the_largest_bound_over_its_heads():
    """Block 1's keys are (40, -30), block 2's (0, 30).  Head 0 (query (1, 0)) bounds them by
    40 and 0, head 1 (query (0, 1)) by -30 and 30: the group keeps block 1 (largest bound 40),
    where an average over the heads would keep block 2 (5 against 15)."""
    B, D = 2, 2
    k = np.zeros((6, 1, D), dtype=np.float32)
    k[2:4, 0] = [40.0, -30.0]
    k[4:6, 0] = [0.0, 30.0]
    rng = np.random.default_rng(3)
    a, kp, vp, t, l = _setup(rng, [6], H=1, D=D, B=B, k=[k])
    q = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    assert quest.selected_blocks(q, kp, t, l, 1, 1, "f32")[(0, 0)].tolist() == [1]
    assert quest.selected_blocks(q[:, 1:], kp, t, l, 1, 1, "f32")[(0, 0)].tolist() == [2]


def test_ties_keep_the_lower_index_and_output_is_in_logical_order():
    assert quest.select([1.0, 3.0, 3.0, 0.5, 3.0], 2).tolist() == [1, 2]
    assert quest.select([2.0, 1.0], 5).tolist() == [0, 1]
    assert quest.select([], 3).tolist() == []


def test_placement_does_not_matter():
    rng = np.random.default_rng(4)
    lens = [45, 23]
    k = [rng.standard_normal((n, 2, 8)).astype(np.float32) for n in lens]
    q = rng.standard_normal((2, 4, 8))
    outs = []
    for order in (None, rng.permutation(80)):
        a, kp, vp, t, l = _setup(np.random.default_rng(5), lens, k=k, order=order)
        outs.append((quest.selected_blocks(q, kp, t, l, 2, 3, "f32"),
                     quest.quest_decode(q, kp, vp, t, l, 0.3, 2, 3, "f32")))
    assert all(np.array_equal(outs[0][0][key], outs[1][0][key]) for key in outs[0][0])
    assert np.array_equal(outs[0][1], outs[1][1])


def test_partial_last_block_ignores_unused_slots():
    rng = np.random.default_rng(6)
    a, kp, vp, t, l = _setup(rng, [10], H=1, D=4, B=4)
    last = t[0][2]
    kp[last, 0, 2:] = 1e30                                   # two unused slots of the last block
    mins, maxs = quest.block_minmax(kp, t[0], 10, 0, "f32")
    K = oattn.gather_keys(kp, t[0], 10, 0).astype(np.float64)
    assert np.array_equal(maxs[2], K[8:10].max(0)) and np.array_equal(mins[2], K[8:10].min(0))


# --------------------------------------------------------------------------- mutations

def _bounds_ignore_sign(q, mins, maxs):
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    return (q[:, None, :] * maxs[None, :, :]).sum(axis=2)


def _bounds_min_only(q, mins, maxs):
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    return np.minimum(q[:, None, :] * mins[None, :, :], q[:, None, :] * maxs[None, :, :]).sum(axis=2)


def _select_smallest(scores, budget):
    scores = np.asarray(scores, dtype=np.float64)
    if len(scores) <= budget:
        return np.arange(len(scores))
    return np.sort(np.argsort(scores, kind="stable")[:budget])


def _select_ties_high(scores, budget):
    scores = np.asarray(scores, dtype=np.float64)
    n = len(scores)
    if n <= budget:
        return np.arange(n)
    return np.sort(np.asarray(sorted(range(n), key=lambda b: (-scores[b], -b))[:budget]))


def _minmax_whole_block(k_pool, table, ctx, kv_head, kv_dtype, k_scale=1.0):
    B = k_pool.shape[2]
    nb = -(-ctx // B)
    full = nb * B
    K = oattn.dequant(k_pool[np.asarray(table)[np.arange(full) // B], kv_head, np.arange(full) % B],
                      kv_dtype, k_scale)
    return (np.stack([K[b * B:(b + 1) * B].min(0) for b in range(nb)]),
            np.stack([K[b * B:(b + 1) * B].max(0) for b in range(nb)]))


def _group_mean(q, k_pool, tables, ctx, num_kv_heads, budget, kv_dtype, k_scale=1.0):
    S, Hq, _ = q.shape
    g = Hq // num_kv_heads
    out = {}
    for s in range(S):
        for kvh in range(num_kv_heads):
            mins, maxs = quest.block_minmax(k_pool, tables[s], int(ctx[s]), kvh, kv_dtype, k_scale)
            u = quest.bounds(q[s, kvh * g:(kvh + 1) * g], mins, maxs).mean(axis=0)
            out[(s, kvh)] = quest.select(u, budget)
    return out


_PINS = [test_bound_never_below_the_best_score_and_tight_for_one_token,
         test_sign_rule_worked_example, test_budget_covering_the_context_is_plain_attention,
         test_the_block_the_query_points_at_is_kept,
         test_group_selection_takes_the_largest_bound_over_its_heads,
         test_ties_keep_the_lower_index_and_output_is_in_logical_order,
         test_partial_last_block_ignores_unused_slots]

MUTATIONS = {
    "bound ignores the query's sign": ("bounds", _bounds_ignore_sign),
    "bound takes the smaller product": ("bounds", _bounds_min_only),
    "keeps the smallest bounds": ("select", _select_smallest),
    "ties keep the higher index": ("select", _select_ties_high),
    "min / max over unused slots too": ("block_minmax", _minmax_whole_block),
    "group score is the mean over heads": ("selected_blocks", _group_mean),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_quest_mutation_is_caught(name, monkeypatch):
    attr, value = MUTATIONS[name]
    monkeypatch.setattr(quest, attr, value)
    caught = False
    for pin in _PINS:
        try:
            pin()
        except Exception:
            caught = True
            break
    assert caught, name
