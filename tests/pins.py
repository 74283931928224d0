"""Pins of the oracle: checks against what the pages and the mathematics fix.

Each ``check_*`` raises AssertionError (or any exception) when the oracle
disagrees with the pages' worked examples, a library routine on a special
case, a closed form, or an invariant.  ``test_oracle_pins`` runs them as they
are; ``test_oracle_mutations`` plants mistakes in the oracle and checks that at
least one of them fails.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import workloads
from oracle import allocator as oalloc
from oracle import attention as oattn
from oracle import cache as ocache
from oracle import codec

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ allocator / cache

def check_glossary_example():
    """The glossary's code example: 40 keys through a block table (printed output)."""
    g = _golden("glossary_code_example.json")
    B, D, N = g["block_size"], g["head_dim"], g["pool_blocks"]
    a = oalloc.BlockAllocator(N, B, g["free_blocks"])
    table = a.add_seq(0, g["num_keys"])
    e = g["expected"]
    assert len(table) == e["num_blocks"]
    assert table == e["block_table"]
    assert list(a.free) == e["free_blocks_after"]
    keys = np.random.default_rng(0).standard_normal((g["num_keys"], 1, D)).astype(np.float32)
    k_pool, v_pool = ocache.new_pools(N, 1, B, D, "f32")
    slots = a.slots(0, 0, g["num_keys"])
    ocache.reshape_and_cache(k_pool, v_pool, keys, keys, slots, "f32", "f32")
    # position pos sits in row pos mod B of the block listed at table entry pos div B
    for pos in range(g["num_keys"]):
        assert np.array_equal(k_pool[table[pos // B], 0, pos % B], keys[pos, 0])
    gathered = oattn.gather_keys(k_pool, table, g["num_keys"], 0)
    assert np.array_equal(gathered, keys[:, 0]) == e["keys_intact"]
    assert len(table) * B - g["num_keys"] == e["unused_slots_paged"]
    assert e["reservation_tokens"] - g["num_keys"] == e["unused_slots_reserved"]
    st = a.stats()
    assert st["slots_allocated"] - st["tokens"] == e["unused_slots_paged"]


def check_optiverse_block_table():
    """The optiverse block table: 41 tokens -> 7/3/12 filled 16/16/9; token 41 -> 10th slot of 12."""
    g = _golden("optiverse_block_table.json")
    B = g["block_size"]
    e = g["expected"]
    a = oalloc.BlockAllocator(16, B, g["free_blocks"])
    table = a.add_seq(0, g["num_tokens"])
    assert table == e["block_table"]
    fills = [min(B, g["num_tokens"] - j * B) for j in range(len(table))]
    assert fills == e["fills"]
    for j, (lo, hi) in enumerate(e["logical_block_token_ranges"]):
        assert {a.slot(0, t) // B for t in range(lo, min(hi + 1, g["num_tokens"]))} == {table[j]}
    slot, pair = a.append(0)                                   # token 41
    assert pair is None
    assert slot // B == e["next_token_physical_block"]
    assert slot % B + 1 == e["next_token_position_ordinal"]
    for t in range(g["num_tokens"] + 1, e["last_token_filling_block"] + 1):
        s, _ = a.append(0)
        assert s // B == e["next_token_physical_block"]
    assert s % B == B - 1                                      # token 47 fills block 12
    free_before = len(a.free)
    s, _ = a.append(0)                                         # token 48 needs a new block
    assert a.lens[0] - 1 == e["token_after_full_block_needs_new_block"]
    assert s // B not in e["block_table"] and len(a.free) == free_before - 1
    new_block = s // B
    a.free_seq(0)
    assert set(e["blocks_returned_at_end"]) <= set(a.free)
    # reading: freed blocks go to the tail, in logical order
    assert list(a.free)[-4:] == e["blocks_returned_at_end"] + [new_block]


def check_optiverse_worked_example():
    """825 tokens: 52 blocks, 832 slots, 7 wasted; waste <= B-1 for any length."""
    g = _golden("optiverse_worked_example.json")
    B, n, e = g["block_size"], g["num_tokens"], g["expected"]
    a = oalloc.BlockAllocator(200, B)
    table = a.add_seq(0, n)
    st = a.stats()
    assert len(table) == e["paged_blocks"]
    assert st["slots_allocated"] == e["paged_slots"]
    assert n - (len(table) - 1) * B == e["paged_filled_in_last_block"]
    assert st["slots_allocated"] - st["tokens"] == e["paged_wasted_slots"]
    assert 100.0 * e["paged_wasted_slots"] / st["slots_allocated"] < e["paged_waste_below_percent"]
    assert g["reservation_tokens"] - n == e["contiguous_wasted_slots"]
    assert round(100.0 * e["contiguous_wasted_slots"] / g["reservation_tokens"]) == \
        e["contiguous_waste_percent_rounded"]
    worst = 0
    for m in range(1, 3 * g["reservation_tokens"]):
        b = oalloc.BlockAllocator(400, B)
        b.add_seq(0, m)
        s = b.stats()
        worst = max(worst, s["slots_allocated"] - s["tokens"])
    assert worst == e["max_waste_per_request"]


def check_copy_on_write():
    """The ithome copy-on-write figure: A1 copies block 1 into new block 3, A2 writes in place."""
    g = _golden("ithome_copy_on_write.json")
    B, e = g["block_size"], g["expected"]
    words = g["prompt_tokens"] + [w for _, w in g["writes_in_order"]]
    wid = {w: float(i + 1) for i, w in enumerate(words)}
    a = oalloc.BlockAllocator(8, B, g["free_blocks"])
    A1, A2 = 1, 2
    table = a.add_seq(A1, len(g["prompt_tokens"]))
    a.fork(A1, A2)
    assert table == e["shared_table_before"]
    assert {str(b): a.ref[b] for b in table} == e["refcounts_before"]
    k_pool, v_pool = ocache.new_pools(8, 1, B, 1, "f32")
    kin = np.array([[[wid[w]]] for w in g["prompt_tokens"]], dtype=np.float32)
    ocache.reshape_and_cache(k_pool, v_pool, kin, kin, a.slots(A1, 0, len(kin)), "f32", "f32")
    slots, pairs = a.append_batch([A1, A2])
    assert [list(p) for p in pairs] == e["copy_pairs"]
    assert a.tables[A1] == e["A1_table_after"] and a.tables[A2] == e["A2_table_after"]
    assert {k: a.ref[int(k)] for k in e["refcounts_after"]} == e["refcounts_after"]
    ocache.copy_blocks(k_pool, v_pool, pairs)
    new = np.array([[[wid[w]]] for _, w in g["writes_in_order"]], dtype=np.float32)
    ocache.reshape_and_cache(k_pool, v_pool, new, new, slots, "f32", "f32")
    inv = {v: k for k, v in wid.items()}
    for blk, key in ((1, "block_1_tokens_after"), (3, "block_3_tokens_after")):
        assert [inv[float(x)] for x in k_pool[blk, 0, :, 0]] == e[key]
        assert [inv[float(x)] for x in v_pool[blk, 0, 0, :]] == e[key]


def check_copy_blocks_invariant():
    """copy_blocks: dst == src afterwards, every other byte unchanged; bad pairs rejected."""
    rng = np.random.default_rng(3)
    k = rng.integers(0, 65535, size=(12, 2, 4, 8), dtype=np.uint16)
    v = rng.integers(0, 65535, size=(12, 2, 8, 4), dtype=np.uint16)
    k0, v0 = k.copy(), v.copy()
    pairs = [(3, 7), (5, 0), (3, 9)]
    ocache.copy_blocks(k, v, pairs)
    for s, d in pairs:
        assert np.array_equal(k[d], k0[s]) and np.array_equal(v[d], v0[s])
    untouched = [b for b in range(12) if b not in (7, 0, 9)]
    assert np.array_equal(k[untouched], k0[untouched]) and np.array_equal(v[untouched], v0[untouched])
    for bad in ([(1, 1)], [(1, 2), (3, 2)], [(1, 2), (2, 3)], [(1, 12)], [(-1, 2)]):
        try:
            ocache.copy_blocks(k, v, bad)
        except ValueError:
            continue
        raise AssertionError(f"accepted bad pairs {bad}")


def check_cache_write_only_touches_slots():
    """reshape_and_cache writes exactly the given slots (negative = skip)."""
    B, D, Hkv, N = 16, 8, 3, 6
    k_pool, v_pool = ocache.new_pools(N, Hkv, B, D, "bf16")
    k0, v0 = k_pool.copy(), v_pool.copy()
    rng = np.random.default_rng(5)
    k = rng.integers(0, 0x7F00, size=(4, Hkv, D), dtype=np.uint16)
    v = rng.integers(0, 0x7F00, size=(4, Hkv, D), dtype=np.uint16)
    slots = [17, -1, 95, 40]
    ocache.reshape_and_cache(k_pool, v_pool, k, v, slots, "bf16", "bf16")
    written = set()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        b, p = divmod(s, B)
        written.add((b, p))
        assert np.array_equal(k_pool[b, :, p, :], k[i])
        assert np.array_equal(v_pool[b, :, :, p], v[i])
    for b in range(N):
        for p in range(B):
            if (b, p) not in written:
                assert np.array_equal(k_pool[b, :, p, :], k0[b, :, p, :])
                assert np.array_equal(v_pool[b, :, :, p], v0[b, :, :, p])


# ------------------------------------------------------------------ attention

def _oracle_case(seed, *, S, Hq, Hkv, D, B, max_ctx, kv_dtype, in_dtype, min_ctx=1):
    from oracle_pipeline import run
    wl = workloads.random_small(seed, S=S, Hq=Hq, Hkv=Hkv, D=D, B=B, max_ctx=max_ctx,
                                kv_dtype=kv_dtype, in_dtype=in_dtype, min_ctx=min_ctx)
    return wl, run(wl)


def _sdpa_reference(wl, st):
    """torch SDPA in float64 over each sequence's contiguous K/V, built from the raw draws."""
    q = st.q64()
    out = np.zeros_like(q)
    g = wl.num_q_heads // wl.num_kv_heads
    for i in range(wl.num_seqs):
        k, v = wl.seq_kv_input(i)
        if wl.kv_dtype == "fp8":
            # torch's own widening and fp8 cast of x / scale (within range: no saturation)
            kf = _torch_bf16(k).to(torch.float32) if wl.in_dtype == "bf16" else torch.from_numpy(k)
            vf = _torch_bf16(v).to(torch.float32) if wl.in_dtype == "bf16" else torch.from_numpy(v)
            kq = kf / torch.tensor(st.k_scale, dtype=torch.float32)
            vq = vf / torch.tensor(st.v_scale, dtype=torch.float32)
            K = kq.to(torch.float8_e4m3fn).to(torch.float64) * float(np.float32(st.k_scale))
            V = vq.to(torch.float8_e4m3fn).to(torch.float64) * float(np.float32(st.v_scale))
        elif wl.in_dtype == "bf16":
            K = _torch_bf16(k).to(torch.float64)
            V = _torch_bf16(v).to(torch.float64)
        else:
            K = torch.from_numpy(k).to(torch.float64)
            V = torch.from_numpy(v).to(torch.float64)
        # [ctx, Hkv, D] -> [Hq, ctx, D], query head h reads KV head h // g
        K = K.permute(1, 0, 2).repeat_interleave(g, dim=0).contiguous()
        V = V.permute(1, 0, 2).repeat_interleave(g, dim=0).contiguous()
        qq = torch.from_numpy(q[i]).unsqueeze(1)                      # [Hq, 1, D]
        o = torch.nn.functional.scaled_dot_product_attention(
            qq.unsqueeze(0), K.unsqueeze(0), V.unsqueeze(0), scale=wl.scale)
        out[i] = o[0, :, 0, :].numpy()
    return out


ATTN_CASES = [
    dict(seed=11, S=5, Hq=4, Hkv=2, D=64, B=16, max_ctx=70, kv_dtype="f32", in_dtype="f32"),
    dict(seed=12, S=4, Hq=8, Hkv=2, D=32, B=8, max_ctx=50, kv_dtype="bf16", in_dtype="bf16"),
    dict(seed=13, S=3, Hq=6, Hkv=3, D=16, B=4, max_ctx=30, kv_dtype="fp8", in_dtype="bf16"),
    dict(seed=14, S=3, Hq=3, Hkv=1, D=64, B=16, max_ctx=40, kv_dtype="f32", in_dtype="f32"),
]


def check_attention_vs_sdpa():
    """Paged oracle == torch SDPA (float64) on contiguous K/V: the paging reduces to plain attention."""
    for case in ATTN_CASES:
        wl, st = _oracle_case(**case)
        got = oattn.paged_decode(st.q64(), st.k_pool, st.v_pool, st.tables, st.ctx, wl.scale,
                                 wl.kv_dtype, st.k_scale, st.v_scale)
        ref = _sdpa_reference(wl, st)
        err = np.abs(got - ref).max()
        assert err < 1e-12, (case, err)


def check_single_token_context():
    """ctx = 1: the output is the single cached value, exactly."""
    wl, st = _oracle_case(21, S=3, Hq=4, Hkv=2, D=32, B=16, max_ctx=1, kv_dtype="bf16",
                          in_dtype="bf16")
    got = oattn.paged_decode(st.q64(), st.k_pool, st.v_pool, st.tables, st.ctx, wl.scale, "bf16")
    for i in range(wl.num_seqs):
        _, v = wl.seq_kv_input(i)
        for h in range(wl.num_q_heads):
            assert np.array_equal(got[i, h], codec.bf16_to_f64(v[0, h // 2]))


def check_identical_keys():
    """All keys equal: the weights are uniform and the output is the mean of the values."""
    B, D, ctx = 16, 8, 37
    a = oalloc.BlockAllocator(8, B, [5, 2, 7, 0, 1, 3, 4, 6])
    a.add_seq(0, ctx)
    k_pool, v_pool = ocache.new_pools(8, 1, B, D, "f32")
    rng = np.random.default_rng(9)
    key = rng.standard_normal(D).astype(np.float32)
    vals = rng.standard_normal((ctx, 1, D)).astype(np.float32)
    ocache.reshape_and_cache(k_pool, v_pool, np.broadcast_to(key, (ctx, 1, D)), vals,
                             a.slots(0, 0, ctx), "f32", "f32")
    tables, lens = a.block_tables([0], 4)
    q = rng.standard_normal((1, 1, D))
    got = oattn.paged_decode(q, k_pool, v_pool, tables, lens, 0.3, "f32")
    assert np.allclose(got[0, 0], vals[:, 0].astype(np.float64).mean(axis=0), atol=1e-13, rtol=0)


def check_empty_context():
    """ctx = 0: zeros (our reading)."""
    k_pool, v_pool = ocache.new_pools(4, 1, 16, 8, "f32")
    out = oattn.paged_decode(np.ones((1, 2, 8)), k_pool, v_pool, np.full((1, 1), -1), [0],
                             1.0, "f32")
    assert np.array_equal(out, np.zeros((1, 2, 8)))


def _place(wl, order_seed):
    """Same contents in a different physical placement (a different free list)."""
    import dataclasses

    from oracle_pipeline import run
    rng = np.random.default_rng(order_seed)
    wl2 = dataclasses.replace(wl, free_order=rng.permutation(wl.num_blocks).astype(np.int32),
                              _cache={})
    return wl2, run(wl2)


def check_placement_invariance():
    """Permuting where blocks sit in the pool leaves the output unchanged (bit for bit)."""
    wl, st = _oracle_case(31, S=4, Hq=4, Hkv=2, D=32, B=8, max_ctx=60, kv_dtype="bf16",
                          in_dtype="bf16")
    base = oattn.paged_decode(st.q64(), st.k_pool, st.v_pool, st.tables, st.ctx, wl.scale, "bf16")
    wl2, st2 = _place(wl, 77)
    assert not np.array_equal(st.tables, st2.tables)
    other = oattn.paged_decode(st2.q64(), st2.k_pool, st2.v_pool, st2.tables, st2.ctx,
                               wl2.scale, "bf16")
    assert np.array_equal(base, other)


def check_sharing_invariance():
    """Sequences sharing prefix blocks (fork) == the same sequences stored unshared."""
    B, D, Hkv, N = 4, 8, 2, 32
    rng = np.random.default_rng(41)
    prefix, tails = 10, [3, 0, 5]
    pk = rng.standard_normal((prefix, Hkv, D)).astype(np.float32)
    pv = rng.standard_normal((prefix, Hkv, D)).astype(np.float32)
    tk = [rng.standard_normal((t + 1, Hkv, D)).astype(np.float32) for t in tails]
    tv = [rng.standard_normal((t + 1, Hkv, D)).astype(np.float32) for t in tails]
    q = rng.standard_normal((3, 4, D))

    def build(shared):
        a = oalloc.BlockAllocator(N, B, rng.permutation(N) if not shared else None)
        kp, vp = ocache.new_pools(N, Hkv, B, D, "f32")
        if shared:
            a.add_seq(0, prefix)
            ocache.reshape_and_cache(kp, vp, pk, pv, a.slots(0, 0, prefix), "f32", "f32")
            a.fork(0, 1)
            a.fork(0, 2)
        else:
            for s in range(3):
                a.add_seq(s, prefix)
                ocache.reshape_and_cache(kp, vp, pk, pv, a.slots(s, 0, prefix), "f32", "f32")
        for s in range(3):
            slots, pairs = a.extend(s, tails[s] + 1)
            if pairs:
                ocache.copy_blocks(kp, vp, pairs)
            ocache.reshape_and_cache(kp, vp, tk[s], tv[s], slots, "f32", "f32")
        tables, lens = a.block_tables([0, 1, 2], 8)
        return tables, oattn.paged_decode(q, kp, vp, tables, lens, 0.25, "f32")

    t_shared, shared = build(True)
    t_plain, plain = build(False)
    assert t_shared[0, 0] == t_shared[1, 0] == t_shared[2, 0]      # prefix blocks are shared
    assert np.array_equal(shared, plain)


def check_gqa_is_repeated_mha():
    """GQA with Hq/Hkv = g equals MHA whose KV heads are each repeated g times (contiguously)."""
    wl, st = _oracle_case(51, S=3, Hq=6, Hkv=2, D=16, B=8, max_ctx=40, kv_dtype="f32",
                          in_dtype="f32")
    gqa = oattn.paged_decode(st.q64(), st.k_pool, st.v_pool, st.tables, st.ctx, wl.scale, "f32")
    g = 3
    kp = np.repeat(st.k_pool, g, axis=1)
    vp = np.repeat(st.v_pool, g, axis=1)
    mha = oattn.paged_decode(st.q64(), kp, vp, st.tables, st.ctx, wl.scale, "f32")
    assert np.array_equal(gqa, mha)


# ------------------------------------------------------------------ number formats

def _torch_bf16(bits: np.ndarray):
    """Raw bfloat16 patterns as a torch bfloat16 tensor (a reinterpretation, no arithmetic)."""
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16)


def check_bf16_widening():
    """Both widenings of the oracle against torch's bfloat16 casts, on all 65536 patterns:
    to float64 by value, to float32 bit for bit (torch keeps NaN payloads too)."""
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ref = _torch_bf16(bits).to(torch.float64).numpy()
    got = codec.bf16_to_f64(bits)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    ref32 = _torch_bf16(bits).to(torch.float32).numpy()
    got32 = codec.bf16_to_f32(bits)
    assert got32.dtype == np.float32 and got32.shape == bits.shape
    assert np.array_equal(got32.view(np.uint32), ref32.view(np.uint32))


def check_fp8_cache_encode():
    """The oracle's cache write of bf16 inputs into an fp8 pool (widen, divide by the scale in
    fp32, round) against torch on every finite bf16 pattern: torch widens, divides and casts to
    float8_e4m3fn itself.  Scales are chosen so that |x / scale| stays below 464, where torch's
    cast rounds to nearest-even without overflowing; past that the oracle saturates (a reading
    torch cannot confirm)."""
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    x32 = _torch_bf16(bits).to(torch.float32)
    finite = torch.isfinite(x32).numpy()
    bits, x32 = bits[finite], x32[torch.from_numpy(finite)]
    amax = float(x32.abs().max())
    for scale in (np.float32(amax / 448.0), np.float32(amax / 400.0), np.float32(amax / 300.0)):
        y = x32 / torch.tensor(float(scale), dtype=torch.float32)
        ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert float(y.abs().max()) < 464.0
        got = ocache.encode(bits, "bf16", "fp8", float(scale))
        assert np.array_equal(got, ref), int(np.count_nonzero(got != ref))


def check_e4m3_decode():
    """All 256 codes decode as torch.float8_e4m3fn does."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codec.e4m3_to_f64(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), np.nonzero(~same)
    assert np.nanmax(got) == 448.0 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def _f32_sweep():
    """fp32 values covering every E4M3 rounding interval: a strided sweep of bit patterns
    below 464 (the first value that does not round to 448), both signs, plus midpoints
    and their neighbours."""
    top = np.float32(464.0).view(np.uint32)
    pats = np.arange(0, int(top), 4099, dtype=np.uint32)
    vals = [pats.view(np.float32)]
    mags = codec.E4M3_TABLE[:0x7F]
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    vals += [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
             mags.astype(np.float32)]
    v = np.concatenate(vals).astype(np.float32)
    v = v[np.abs(v) < 464.0]
    return np.concatenate([v, -v])


def check_e4m3_encode():
    """Encoding matches torch's float8_e4m3fn cast (nearest-even) wherever torch does not overflow."""
    x = _f32_sweep()
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = codec.e4m3_encode_f32(x)
    assert np.array_equal(got, ref), np.nonzero(got != ref)
    # reading: saturate beyond 448 (torch would give NaN), NaN -> 0x7F, -0 -> 0x80
    big = np.array([464.0, 1e6, np.inf, -500.0, -np.inf], dtype=np.float32)
    assert codec.e4m3_encode_f32(big).tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert codec.e4m3_encode_f32(np.array([np.nan, -0.0, 0.0], np.float32)).tolist() == \
        [0x7F, 0x80, 0x00]


def check_fp8_pool_is_half_of_bf16():
    """An 8-bit cache takes about half the memory of a 16-bit one (glossary, FP8 cache)."""
    k8, v8 = ocache.new_pools(10, 2, 16, 64, "fp8")
    k16, v16 = ocache.new_pools(10, 2, 16, 64, "bf16")
    assert 2 * (k8.nbytes + v8.nbytes) == k16.nbytes + v16.nbytes


ALL = [
    check_glossary_example, check_optiverse_block_table, check_optiverse_worked_example,
    check_copy_on_write, check_copy_blocks_invariant, check_cache_write_only_touches_slots,
    check_attention_vs_sdpa, check_single_token_context, check_identical_keys,
    check_empty_context, check_placement_invariance, check_sharing_invariance,
    check_gqa_is_repeated_mha, check_bf16_widening, check_e4m3_decode, check_e4m3_encode,
    check_fp8_cache_encode, check_fp8_pool_is_half_of_bf16,
]
