"""GPU parity of the cache operations, bit for bit against the oracle.

reshape_and_cache and copy_blocks are integer / byte work: the whole pools
written by the HIP library must equal the oracle's, including every byte the
operations must not touch (unused slots stay NaN-poisoned).
"""
import numpy as np
import pytest

import workloads
from gpu_util import GpuState, pools_equal_bits, torch_mod
from oracle import cache as ocache
from oracle import codec
from oracle_pipeline import run as oracle_run

pytestmark = pytest.mark.gpu

SMALL = [
    dict(seed=101, S=5, Hq=2, Hkv=2, D=64, B=16, max_ctx=70, kv_dtype="f32", in_dtype="f32"),
    dict(seed=102, S=6, Hq=8, Hkv=2, D=128, B=16, max_ctx=200, kv_dtype="bf16", in_dtype="bf16"),
    dict(seed=103, S=4, Hq=4, Hkv=4, D=64, B=8, max_ctx=90, kv_dtype="bf16", in_dtype="bf16"),
    dict(seed=104, S=4, Hq=16, Hkv=2, D=128, B=32, max_ctx=150, kv_dtype="fp8", in_dtype="bf16"),
    dict(seed=105, S=3, Hq=4, Hkv=1, D=64, B=16, max_ctx=60, kv_dtype="fp8", in_dtype="f32"),
    dict(seed=106, S=3, Hq=3, Hkv=3, D=128, B=8, max_ctx=40, kv_dtype="f32", in_dtype="f32"),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c['kv_dtype']}-D{c['D']}-B{c['B']}")
def test_pools_bitexact_after_script_and_step(case):
    wl = workloads.random_small(**case)
    print(f"case {wl.name} {case}", flush=True)
    st = oracle_run(wl)
    g = GpuState(wl)
    k, v = g.pools_host()
    assert pools_equal_bits(k, st.k_pool)
    assert pools_equal_bits(v, st.v_pool)
    assert g.slots.tolist() == st.step_slots


def test_tiny_config_pools_bitexact():
    wl = workloads.get("tiny-f32")
    st = oracle_run(wl)
    g = GpuState(wl)
    k, v = g.pools_host()
    assert pools_equal_bits(k, st.k_pool) and pools_equal_bits(v, st.v_pool)
    assert np.array_equal(g.tables.cpu().numpy(), st.tables)
    assert np.array_equal(g.lens.cpu().numpy(), st.ctx)


def _shared_prefix_small(seed, prompts=3, n=4, prefix=40, B=16, Hkv=2, D=64, g=2, max_tail=40,
                         kv_dtype="bf16"):
    """A reduced copy of the shared-prefix workload: forks, one copy-on-write batch, tails."""
    import dataclasses
    import math

    base = workloads.shared_prefix_bf16()
    rng = np.random.default_rng(seed)
    tails = rng.integers(0, max_tail, size=prompts * n)
    ids = np.arange(prompts * n, dtype=np.int64)
    ctx = prefix + 1 + tails + 1
    need = sum(prefix // B + sum(-(-(int(ctx[p * n + k]) - (prefix // B) * B) // B)
                                 for k in range(n)) for p in range(prompts))
    N = int(math.ceil(1.25 * need)) + 2
    ops = []
    for p in range(prompts):
        ops.append(("add", p * n, prefix))
        for k in range(1, n):
            ops.append(("fork", p * n, p * n + k))
    ops.append(("append_batch", [int(s) for s in ids]))
    for s in ids:
        if tails[s]:
            ops.append(("extend", int(s), int(tails[s])))

    def seg(i):
        return [((i // n) * n, 0, prefix), (10_000 + i, 0, int(ctx[i]) - prefix)]

    return dataclasses.replace(
        base, name="shared-prefix-small", seed=seed, num_q_heads=g * Hkv, num_kv_heads=Hkv,
        head_dim=D, block_size=B, num_blocks=N, scale=1 / math.sqrt(D), kv_dtype=kv_dtype,
        free_order=rng.permutation(N).astype(np.int32), setup_ops=ops, decode_seqs=ids,
        ctx_lens=ctx, _segments=seg, _cache={})


def test_copy_on_write_flow_bitexact():
    wl = _shared_prefix_small(7)
    st = oracle_run(wl)
    g = GpuState(wl)
    k, v = g.pools_host()
    assert pools_equal_bits(k, st.k_pool) and pools_equal_bits(v, st.v_pool)
    assert np.array_equal(g.tables.cpu().numpy(), st.tables)


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "fp8"])
def test_copy_blocks_bitexact(kv_dtype):
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    N, H, B, D = 40, 3, 16, 64
    desc = pkv.cache_desc(N, H, B, D, kv_dtype, *((0.5, 0.25) if kv_dtype == "fp8" else (1, 1)))
    ks, vs = pkv.pool_shapes(desc)
    rng = np.random.default_rng(3)
    elem = {"f32": 4, "bf16": 2, "fp8": 1}[kv_dtype]
    kb = rng.integers(0, 256, size=int(np.prod(ks)) * elem, dtype=np.uint8)
    vb = rng.integers(0, 256, size=int(np.prod(vs)) * elem, dtype=np.uint8)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[kv_dtype]
    kp = torch.from_numpy(kb).cuda().view(tdt).view(ks)
    vp = torch.from_numpy(vb).cuda().view(tdt).view(vs)
    pairs = np.array([[3, 7], [5, 0], [3, 9], [39, 12], [11, 38]], dtype=np.int64)
    pkv.copy_blocks(kp, vp, pairs, desc)
    torch.cuda.synchronize()
    ko, vo = kb.reshape(N, -1).copy(), vb.reshape(N, -1).copy()
    ocache.copy_blocks(ko, vo, pairs)
    assert np.array_equal(kp.view(torch.uint8).cpu().numpy().reshape(N, -1), ko)
    assert np.array_equal(vp.view(torch.uint8).cpu().numpy().reshape(N, -1), vo)
    with pytest.raises(ValueError):
        pkv.copy_blocks(kp, vp, np.array([[1, 2], [2, 3]]), desc)


def _f32_patterns():
    """Every fp32 sign / exponent / top-16-mantissa pattern, with low bits 0, 1 and all-ones,
    plus the E4M3 midpoints and their neighbours."""
    hi = np.arange(1 << 24, dtype=np.uint32) << np.uint32(8)
    pats = np.concatenate([hi, hi | np.uint32(1), hi | np.uint32(0xFF)])
    vals = pats.view(np.float32)
    mags = codec.E4M3_TABLE[:0x7F]
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    extra = np.concatenate([mids, np.nextafter(mids, np.float32(0)),
                            np.nextafter(mids, np.float32(1e9))])
    extra = np.concatenate([extra, -extra])
    return np.concatenate([vals, extra])


@pytest.mark.parametrize("scale", [1.0, 0.013671875, 3.0])
def test_fp8_encode_sweep_f32_input(scale):
    """reshape_and_cache's E4M3 encode over 50M fp32 inputs equals the oracle's, bit for bit."""
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    x = _f32_patterns()
    H, D, B = 1, 128, 16
    T = -(-x.size // (H * D))
    xin = np.zeros(T * H * D, dtype=np.float32)
    xin[: x.size] = x
    xin = xin.reshape(T, H, D)
    N = -(-T // B)
    desc = pkv.cache_desc(N, H, B, D, "fp8", scale, scale)
    kp, vp = pkv.alloc_pools(desc)
    xt = torch.from_numpy(xin).cuda()
    slots = torch.arange(T, dtype=torch.int64, device="cuda")
    pkv.reshape_and_cache(xt, xt, slots, kp, vp, desc)
    got = kp.cpu().numpy().reshape(-1)[: x.size]
    want = codec.e4m3_quantize(x, scale)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (bad[:10], x[bad[:10]], got[bad[:10]], want[bad[:10]])
    gv = vp.cpu().numpy().transpose(0, 1, 3, 2).reshape(-1)[: x.size]
    assert np.array_equal(gv, want)


@pytest.mark.parametrize("layout", ["in order", "reversed", "small calls"])
def test_fp8_encode_every_bf16_input(layout):
    """Every bf16 input (65536 patterns) through the bf16 -> fp8 cache write, keys and
    values, by each of the write's encode paths: whole value rows (tokens in order, one
    call), single value elements (slots in reverse order, so no two neighbouring tokens
    share a row run) and the per-token kernel (calls of fewer than 512 tokens)."""
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    H, D, B = 2, 64, 16
    T = bits.size // (H * D)
    N = T // B
    order = np.arange(T)[::-1].copy() if layout == "reversed" else np.arange(T)
    calls = [(0, 200), (200, 400), (400, T)] if layout == "small calls" else [(0, T)]
    for scale in (1.0, 0.0078125, 0.37):
        desc = pkv.cache_desc(N, H, B, D, "fp8", scale, scale)
        kp, vp = pkv.alloc_pools(desc)
        xt = torch.from_numpy(bits.view(np.int16).reshape(T, H, D)).view(torch.bfloat16).cuda()
        slots = torch.from_numpy(order.astype(np.int64)).cuda()
        for a, b in calls:
            pkv.reshape_and_cache(xt[a:b], xt[a:b], slots[a:b], kp, vp, desc)
        want = codec.e4m3_quantize(codec.bf16_to_f32(bits), scale).reshape(T, H, D)[np.argsort(order)]
        got_k = kp.cpu().numpy().reshape(N, H, B, D).transpose(0, 2, 1, 3).reshape(T, H, D)
        got_v = vp.cpu().numpy().reshape(N, H, D, B).transpose(0, 3, 1, 2).reshape(T, H, D)
        assert np.array_equal(got_k, want), scale
        assert np.array_equal(got_v, want), scale


def test_negative_slots_are_skipped():
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    desc = pkv.cache_desc(4, 2, 16, 64, "bf16")
    kp, vp = pkv.alloc_pools(desc)
    before_k, before_v = kp.clone(), vp.clone()
    x = torch.randn(3, 2, 64, device="cuda").to(torch.bfloat16)
    slots = torch.tensor([-1, 70, -5], dtype=torch.int64, device="cuda")   # 70: out of pool
    pkv.reshape_and_cache(x, x, slots, kp, vp, desc)
    torch.cuda.synchronize()
    assert torch.equal(kp.view(torch.int16), before_k.view(torch.int16))
    assert torch.equal(vp.view(torch.int16), before_v.view(torch.int16))


def _large_write_slots(pattern, T, B, N, rng):
    """Slots of T tokens in a pool of N blocks: ``prompts`` (sequences of random lengths laid
    end to end, each in its own randomly placed blocks, so chunks of B tokens straddle
    sequences), ``continued`` (the same, each sequence starting at a random row of its
    first block, as a prompt does after a cached prefix, with some tokens skipped),
    ``scattered`` (distinct random slots, some negative or past the pool), ``singles`` (a
    decode batch: each token alone at a random row of a block of its own), ``aligned``
    (one prompt starting at a block's first slot) or ``mixed`` (a batch that mixes prompt
    chunks, some starting within a block, with single decode tokens each at a random row of
    a block of its own)."""
    blocks = rng.permutation(N)
    if pattern == "aligned":
        t = np.arange(T)
        return blocks[t // B] * B + t % B
    if pattern == "singles":        # a decode batch: each token alone in a block of its own
        return (blocks[:T] * B + rng.integers(0, B, T)).astype(np.int64)
    if pattern == "scattered":
        s = rng.permutation(N * B)[:T].astype(np.int64)
        s[rng.random(T) < 0.05] = -1
        s[rng.random(T) < 0.02] = N * B + 7
        return s
    out, used = [], 0
    while sum(len(x) for x in out) < T:
        if pattern == "mixed" and rng.random() < 0.7:
            out.append(np.array([blocks[used] * B + int(rng.integers(0, B))]))
            used += 1
            continue
        n = int(min(rng.integers(1, 700), T - sum(len(x) for x in out)))
        first = int(rng.integers(0, B)) if pattern in ("continued", "mixed") else 0
        nb = -(-(first + n) // B)
        own = blocks[used:used + nb]
        used += nb
        p = np.arange(first, first + n)
        out.append(own[p // B] * B + p % B)
    s = np.concatenate(out).astype(np.int64)
    if pattern == "continued":
        s[rng.random(T) < 0.01] = -1
    return s


_IO = (("bf16", "bf16"), ("fp8", "bf16"), ("fp8", "f32"), ("f32", "f32"))
# 8 heads of 128: a chunk's rows split over several workgroups when the call has few chunks
LARGE = [(kv, inp, B, D, H) for kv, inp in _IO for B in (8, 16, 32) for D, H in ((64, 3), (128, 2))] \
    + [(kv, inp, 16, 128, 8) for kv, inp in _IO]


@pytest.mark.parametrize("case", LARGE, ids=lambda c: f"{c[0]}-{c[1]}-B{c[2]}-D{c[3]}-H{c[4]}")
def test_large_writes_bitexact(case):
    """Writes of thousands of tokens (the path for prefills: chunks of one block's worth of
    tokens, whole value rows for a run of tokens that fills a block in order, single
    elements otherwise) leave both pools bit-identical to the oracle's cache write, for
    prompts laid end to end (starting at a block's first row or within a block), prompts
    mixed with single decode tokens, one aligned prompt, scattered slots with skipped ones
    and a decode batch of single tokens."""
    kv, inp, B, D, H = case
    rng = np.random.default_rng(B * 1000 + D * 10 + H)
    T = (2600 if D == 128 else 700) + int(rng.integers(0, 40))   # both above the per-token path
    N = T + 64                     # room for a block per token (the decode-batch pattern)
    for pattern in _PATTERNS:
        _check_large_write(kv, inp, B, D, H, T, N, pattern, rng)


def _check_large_write(kv, inp, B, D, H, T, N, pattern, rng):
    """One reshape_and_cache call of T tokens in the given slot layout into a pool of N blocks,
    both pools compared bit for bit with the oracle's cache write."""
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    scale = 0.02 if kv == "fp8" else 1.0
    desc = pkv.cache_desc(N, H, B, D, kv, scale, scale)
    print(f"large write {kv}/{inp} B={B} D={D} H={H} {pattern} T={T} N={N}", flush=True)
    slots = _large_write_slots(pattern, T, B, N, rng)
    x = rng.standard_normal((2, T, H, D)).astype(np.float32)
    if inp == "bf16":
        xt = torch.from_numpy(x).to(torch.bfloat16)
        bits = xt.view(torch.int16).numpy().view(np.uint16)
        kin, vin = bits[0], bits[1]
        kd, vd = xt[0].contiguous().cuda(), xt[1].contiguous().cuda()
    else:
        kin, vin = x[0], x[1]
        kd, vd = torch.from_numpy(x[0]).cuda(), torch.from_numpy(x[1]).cuda()
    kp, vp = pkv.alloc_pools(desc)
    pkv.reshape_and_cache(kd, vd, torch.from_numpy(slots).cuda(), kp, vp, desc)
    ok, ov = ocache.new_pools(N, H, B, D, kv)
    ocache.reshape_and_cache(ok, ov, kin, vin, np.where(slots < N * B, slots, -1), inp, kv,
                             scale, scale)
    gk = kp.view(torch.int16).cpu().numpy().view(np.uint16) if kv == "bf16" else kp.cpu().numpy()
    gv = vp.view(torch.int16).cpu().numpy().view(np.uint16) if kv == "bf16" else vp.cpu().numpy()
    assert pools_equal_bits(gk, ok), pattern
    assert pools_equal_bits(gv, ov), pattern


_PATTERNS = ("prompts", "continued", "mixed", "aligned", "scattered", "singles")


def _draw_large(i):
    """A random large write: pool and input dtypes, block size, head size, heads (at most
    1024 elements per token), token count above the per-token path and slot layout."""
    r = np.random.default_rng(9100 + i)
    while True:
        kv, inp = _IO[int(r.integers(0, len(_IO)))]
        B, D = int(r.choice([8, 16, 32])), int(r.choice([64, 128]))
        H = int(r.choice([1, 2, 3, 4, 8, 16]))
        if H * D <= 1024:
            break
    T = int(r.integers(512, 2000))
    pattern = _PATTERNS[int(r.integers(0, len(_PATTERNS)))]
    N = T + 64 if pattern == "singles" else int(1.3 * T / B) + 64
    return kv, inp, B, D, H, T, N, pattern, 9200 + i


RANDOM_LARGE = [_draw_large(i) for i in range(16)]


@pytest.mark.parametrize("case", RANDOM_LARGE, ids=lambda c: f"s{c[8]}")
def test_large_writes_random(case):
    """A seeded random sweep of large writes (shapes where a chunk's rows split over one to
    four workgroups, every slot layout) bit-identical to the oracle's cache write."""
    kv, inp, B, D, H, T, N, pattern, seed = case
    _check_large_write(kv, inp, B, D, H, T, N, pattern, np.random.default_rng(seed))
