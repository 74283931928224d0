"""GPU parity of paged decode attention against the fp64 oracle.

Tolerances (max abs error of the output against the oracle): 1e-5 with an f32
cache, 1.5e-2 with a bf16 cache, 3e-2 with an fp8 cache (the oracle dequantises
the same fp8 codes).  Invariance checks compare the GPU with itself and must be
bit-identical: the kernels accumulate in logical token order only.
"""
import dataclasses

import numpy as np
import pytest

import workloads
from gpu_util import TOL, GpuState, out_host, torch_mod
from oracle_pipeline import decode as oracle_decode
from oracle_pipeline import run as oracle_run

pytestmark = pytest.mark.gpu

IMPLS = {"vector": 1, "mfma": 2}


def _cases():
    out = []
    for kv in ("bf16", "fp8"):
        for D in (64, 128):
            for B in (8, 16, 32):
                for g in (1, 4):
                    out.append(dict(seed=200 + len(out), S=4, Hq=2 * g, Hkv=2, D=D, B=B,
                                    max_ctx=300, kv_dtype=kv, in_dtype="bf16"))
    out.append(dict(seed=290, S=3, Hq=16, Hkv=1, D=128, B=16, max_ctx=200, kv_dtype="bf16",
                    in_dtype="bf16"))
    out.append(dict(seed=291, S=3, Hq=24, Hkv=3, D=128, B=16, max_ctx=120, kv_dtype="fp8",
                    in_dtype="bf16"))
    out.append(dict(seed=292, S=3, Hq=6, Hkv=2, D=128, B=16, max_ctx=100, kv_dtype="bf16",
                    in_dtype="bf16"))
    # the widest group at the narrow head size, and a two-KV-head 16-group
    out.append(dict(seed=293, S=3, Hq=16, Hkv=1, D=64, B=32, max_ctx=150, kv_dtype="fp8",
                    in_dtype="bf16"))
    out.append(dict(seed=294, S=3, Hq=32, Hkv=2, D=64, B=8, max_ctx=150, kv_dtype="bf16",
                    in_dtype="bf16"))
    return out


CASES = _cases()


def _id(c):
    return f"{c['kv_dtype']}-D{c['D']}-B{c['B']}-g{c['Hq'] // c['Hkv']}-s{c['seed']}"


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_decode_matches_oracle(case):
    wl = workloads.random_small(**case)
    print(f"case {_id(case)}", flush=True)
    st = oracle_run(wl)
    ref = oracle_decode(st)
    g = GpuState(wl)
    tol = TOL[wl.kv_dtype]
    for impl in ("mfma", "vector"):
        for ps in (0, 2 * wl.block_size, 64, 128):
            out = out_host(g.decode(ps, IMPLS[impl]))
            err = np.abs(out - ref).max()
            assert err <= tol, (impl, ps, err)


@pytest.mark.parametrize("impl", ["vector"])
def test_tiny_f32_config(impl):
    wl = workloads.get("tiny-f32")
    st = oracle_run(wl)
    ref = oracle_decode(st)
    g = GpuState(wl)
    for ps in (0, 16, 32):
        out = out_host(g.decode(ps, IMPLS[impl]))
        assert np.abs(out - ref).max() <= TOL["f32"], ps
    # the default family for an f32 pool is the vector kernel
    out = out_host(g.decode(0, 0))
    assert np.abs(out - ref).max() <= TOL["f32"]


def test_f32_pool_rejects_mfma():
    import paged_kv_cache_104_amd as pkv

    wl = workloads.get("tiny-f32")
    g = GpuState(wl)
    with pytest.raises(pkv.PagedKVError):
        g.decode(0, IMPLS["mfma"])


@pytest.mark.parametrize("impl", ["vector", "mfma"])
def test_fp8_every_code_decodes_exactly(impl):
    """ctx = 1: the output is the single cached value; with v_scale = 1 every finite E4M3
    code must come out exactly (bf16 holds every E4M3 value)."""
    import paged_kv_cache_104_amd as pkv
    from oracle import codec

    torch = torch_mod()
    D, B, S = 128, 16, 2
    desc = pkv.cache_desc(S, 1, B, D, "fp8", 1.0, 1.0)
    kp, vp = pkv.alloc_pools(desc)
    kp.zero_()
    codes = np.arange(256, dtype=np.uint8).reshape(S, D)
    v = vp.cpu().numpy()
    v[:, 0, :, 0] = codes                       # token 0 of block s holds codes[s]
    vp.copy_(torch.from_numpy(v))
    q = torch.zeros(S, 1, D, dtype=torch.bfloat16, device="cuda")
    tables = torch.arange(S, dtype=torch.int32, device="cuda").view(S, 1)
    lens = torch.ones(S, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    pkv.paged_attn_decode(q, kp, vp, tables, lens, 0.1, out, desc, 16, 0, impl=IMPLS[impl])
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()[:, 0, :].reshape(-1)
    want = codec.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    finite = ~np.isnan(want)
    assert np.array_equal(got[finite], want[finite])
    assert np.isnan(got[~finite]).all()


def _perm_copy(wl, seed):
    rng = np.random.default_rng(seed)
    return dataclasses.replace(wl, free_order=rng.permutation(wl.num_blocks).astype(np.int32),
                               _cache={})


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_output_independent_of_block_placement(kv):
    wl = workloads.random_small(301, S=5, Hq=8, Hkv=2, D=128, B=16, max_ctx=400, kv_dtype=kv,
                                in_dtype="bf16")
    a = GpuState(wl)
    b = GpuState(_perm_copy(wl, 9))
    assert not np.array_equal(a.tables.cpu().numpy(), b.tables.cpu().numpy())
    for impl in (1, 2):
        for ps in (0, 64):
            oa, ob = a.decode(ps, impl), b.decode(ps, impl)
            assert torch_mod().equal(oa.view(torch_mod().int16), ob.view(torch_mod().int16))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_unused_slots_never_leak(kv):
    """NaN-poisoned vs zero-filled unused slots and table padding: identical output."""
    torch = torch_mod()
    wl = workloads.random_small(302, S=6, Hq=4, Hkv=1, D=64, B=16, max_ctx=77, kv_dtype=kv,
                                in_dtype="bf16")
    a = GpuState(wl, poison=True)
    b = GpuState(wl, poison=False)
    # garbage in the table padding too
    tb = b.tables.clone()
    tb[tb < 0] = 10 ** 6
    b.tables = tb
    for impl in (1, 2):
        for ps in (0, 32):
            oa, ob = a.decode(ps, impl), b.decode(ps, impl)
            assert not torch.isnan(oa.float()).any()
            assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


def test_shared_prefix_equals_unshared():
    """Forked sequences sharing prefix blocks decode exactly like unshared copies."""
    from test_gpu_cache_ops import _shared_prefix_small

    torch = torch_mod()
    wl = _shared_prefix_small(11)
    shared = GpuState(wl)
    # unshared: every sample gets its own copy of the prefix
    ops = []
    n = 4
    prefix = 40
    for op in wl.setup_ops:
        if op[0] == "fork":
            ops.append(("add", op[2], prefix))
        else:
            ops.append(op)
    plain_wl = dataclasses.replace(wl, setup_ops=ops, num_blocks=wl.num_blocks * 3,
                                   free_order=np.random.default_rng(5).permutation(
                                       wl.num_blocks * 3).astype(np.int32), _cache={})
    plain = GpuState(plain_wl)
    st = oracle_run(wl)
    ref = oracle_decode(st)
    for impl in (1, 2):
        for ps in (0, 32):
            a, b = shared.decode(ps, impl), plain.decode(ps, impl)
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
            assert np.abs(out_host(a) - ref).max() <= TOL["bf16"]
    assert len(shared.pairs) == 0 and n == 4


def test_empty_and_single_token_contexts():
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    D, B, H = 128, 16, 2
    desc = pkv.cache_desc(8, H, B, D, "bf16")
    kp, vp = pkv.alloc_pools(desc)
    x = torch.randn(3, H, D, device="cuda").to(torch.bfloat16)
    pkv.reshape_and_cache(x, x, torch.tensor([16, 32, 48], device="cuda"), kp, vp, desc)
    q = torch.randn(3, 4 * H, D, device="cuda").to(torch.bfloat16)
    tables = torch.tensor([[1, -1], [2, -1], [3, -1]], dtype=torch.int32, device="cuda")
    lens = torch.tensor([0, 1, 1], dtype=torch.int32, device="cuda")
    for impl in (1, 2):
        for ps in (0, 16):
            out = torch.full_like(q, 7.0)
            pkv.paged_attn_decode(q, kp, vp, tables, lens, 0.1, out, desc, 32, ps, impl=impl)
            torch.cuda.synchronize()
            assert torch.equal(out[0].float(), torch.zeros_like(out[0].float()))
            for s in (1, 2):
                want = x[s].float().repeat_interleave(4, dim=0)
                assert torch.equal(out[s].float(), want)


def test_partition_sweep_long_context():
    """One long context split many ways: every partition size within tolerance."""
    wl = workloads.random_small(303, S=2, Hq=8, Hkv=2, D=128, B=16, max_ctx=3000, min_ctx=2000,
                                kv_dtype="bf16", in_dtype="bf16")
    st = oracle_run(wl)
    ref = oracle_decode(st)
    g = GpuState(wl)
    for ps in (0, 16, 48, 256, 512, 1024, 4096):
        for impl in (1, 2):
            err = np.abs(out_host(g.decode(ps, impl)) - ref).max()
            assert err <= TOL["bf16"], (ps, impl, err)


def test_shared_blocks_hint_changes_nothing():
    """Cached and streaming K/V loads give bit-identical outputs."""
    import paged_kv_cache_104_amd as pkv
    from test_gpu_cache_ops import _shared_prefix_small

    torch = torch_mod()
    g = GpuState(_shared_prefix_small(13))
    for ps in (0, 32):
        a = g.decode(ps, pkv.IMPL_MFMA)
        b = g.decode(ps, pkv.IMPL_MFMA | pkv.IMPL_SHARED_BLOCKS)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    with pytest.raises(pkv.PagedKVError):
        g.decode(0, 0x200)


def test_workspace_contents_never_matter():
    """Whatever the workspace held before (zeros, 0xFF, random bytes, the previous call's
    partial rows, another batch's), the output is bit-identical: every call writes what it
    later reads."""
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    wl = workloads.random_small(304, S=6, Hq=8, Hkv=2, D=128, B=16, max_ctx=3000, min_ctx=700,
                                kv_dtype="bf16", in_dtype="bf16")
    g = GpuState(wl)
    st = oracle_run(wl)
    ref = oracle_decode(st)
    S, Hq, D = g.q.shape
    n = pkv.decode_workspace_bytes(S, Hq, D, wl.max_context_len, 0)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    gen = torch.Generator(device="cpu").manual_seed(5)
    outs = []
    for fill in ("zeros", "ones", "random", "reuse", "reuse"):
        if fill == "zeros":
            ws.zero_()
        elif fill == "ones":
            ws.fill_(0xFF)
        elif fill == "random":
            ws.copy_(torch.randint(0, 256, (n,), generator=gen, dtype=torch.uint8))
        out = torch.empty_like(g.q)
        g.cache.decode(g.q, out, g.tables, g.lens, wl.scale, wl.max_context_len, 0, ws,
                       impl=pkv.IMPL_MFMA)
        torch.cuda.synchronize()
        outs.append(out)
    assert np.abs(out_host(outs[0]) - ref).max() <= TOL["bf16"]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    # a different batch (the first half of the sequences) on the same workspace, then the
    # full batch again
    half = S // 2
    out_h = torch.empty_like(g.q[:half])
    g.cache.decode(g.q[:half].contiguous(), out_h, g.tables[:half].contiguous(),
                   g.lens[:half].contiguous(), wl.scale, wl.max_context_len, 0, ws,
                   impl=pkv.IMPL_MFMA)
    out = torch.empty_like(g.q)
    g.cache.decode(g.q, out, g.tables, g.lens, wl.scale, wl.max_context_len, 0, ws,
                   impl=pkv.IMPL_MFMA)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), outs[0].view(torch.int16))
    assert np.abs(out_host(out_h) - ref[:half]).max() <= TOL["bf16"]


@pytest.mark.parametrize("case", [
    dict(seed=320, Hq=2, Hkv=2, D=128, kv_dtype="bf16"),
    dict(seed=321, Hq=8, Hkv=2, D=128, kv_dtype="bf16"),
    dict(seed=322, Hq=16, Hkv=1, D=128, kv_dtype="bf16"),
    dict(seed=323, Hq=8, Hkv=2, D=64, kv_dtype="bf16"),
    dict(seed=324, Hq=8, Hkv=2, D=128, kv_dtype="fp8"),
], ids=lambda c: f"{c['kv_dtype']}-D{c['D']}-g{c['Hq'] // c['Hkv']}")
def test_many_pairs_per_worker(case):
    """Hundreds of short contexts with a partition size that hands them all to one or two
    matrix-core workers: each worker ends far more pairs than its LDS stage holds (64 piece
    records, 8 KB of output rows), so the stage is written out inside the loop many times."""
    wl = workloads.random_small(case["seed"], S=150, Hq=case["Hq"], Hkv=case["Hkv"],
                                D=case["D"], B=16, max_ctx=40, kv_dtype=case["kv_dtype"],
                                in_dtype="bf16")
    print(f"many pairs {case}", flush=True)
    st = oracle_run(wl)
    ref = oracle_decode(st)
    g = GpuState(wl)
    tol = TOL[wl.kv_dtype]
    for ps in (8192, 1024, 0):
        out = out_host(g.decode(ps, IMPLS["mfma"]))
        err = np.abs(out - ref).max()
        assert err <= tol, (ps, err)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_batch_of_more_than_256_sequences(kv):
    """700 short contexts: the matrix-core workers find their start with the chunked scan
    (each lane's context lengths re-read chunk by chunk), which batches of at most 256
    sequences never take; ranges start anywhere among the three chunks."""
    wl = workloads.random_small(333, S=700, Hq=8, Hkv=2, D=128, B=16, max_ctx=90,
                                kv_dtype=kv, in_dtype="bf16")
    print(f"700 sequences {kv}", flush=True)
    ref = oracle_decode(oracle_run(wl))
    g = GpuState(wl)
    for ps in (0, 64, 2048):
        out = out_host(g.decode(ps, IMPLS["mfma"]))
        err = np.abs(out - ref).max()
        assert err <= TOL[kv], (ps, err)


@pytest.mark.parametrize("kv,impl", [("bf16", 2), ("fp8", 2), ("bf16", 1)])
def test_contexts_cut_at_max_context_len(kv, impl):
    """A max_context_len below some context lengths cuts those contexts at it: the result is
    the attention over their first max_context_len tokens (the oracle on the cut lengths)."""
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    wl = workloads.random_small(334, S=6, Hq=8, Hkv=2, D=128, B=16, max_ctx=900, min_ctx=300,
                                kv_dtype=kv, in_dtype="bf16")
    print(f"cut contexts {kv} impl {impl}", flush=True)
    st = oracle_run(wl)
    g = GpuState(wl)
    for cut in (500, 256, 17):
        st_cut = dataclasses.replace(st, ctx=np.minimum(st.ctx, cut))
        ref = oracle_decode(st_cut)
        for ps in (0, 128):
            out = torch.empty_like(g.q)
            pkv.paged_attn_decode(g.q, g.cache.k_pool, g.cache.v_pool, g.tables, g.lens,
                                  wl.scale, out, g.desc, cut, ps, impl=impl)
            torch.cuda.synchronize()
            err = np.abs(out_host(out) - ref).max()
            assert err <= TOL[kv], (cut, ps, err)


@pytest.mark.parametrize("impl", [1, 2])
def test_timing_events_hold_the_kernel(impl):
    """With the timing hook the decode launch records its own start and end: the pair's
    elapsed time is positive and bounded, the output is unchanged, and the hook applies to
    one launch only."""
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    wl = workloads.random_small(60, S=16, Hq=8, Hkv=2, D=128, B=16, max_ctx=2000,
                                kv_dtype="bf16", in_dtype="bf16")
    g = GpuState(wl)
    ref = g.decode(0, impl)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for x in e:
        x.record()
    torch.cuda.synchronize()
    pkv.time_next_decode(e[0], e[1])
    out = g.decode(0, impl)
    ms = e[0].elapsed_time(e[1])
    assert 0 < ms < 1000
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    out2 = g.decode(0, impl)                 # no events this time
    assert e[0].elapsed_time(e[1]) == ms
    assert torch.equal(out2.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_negative_and_zero_scale(kv):
    """The softmax scale is the caller's: a negative scale favours the smallest dot products
    and a zero scale gives the mean of the values.  Both kernel families against the oracle
    at the same scale."""
    from oracle import attention as oattn

    wl = workloads.random_small(330, S=5, Hq=8, Hkv=2, D=128, B=16, max_ctx=900,
                                kv_dtype=kv, in_dtype="bf16")
    st = oracle_run(wl)
    g = GpuState(wl)
    torch = torch_mod()
    for scale in (-wl.scale, -3.0 * wl.scale, 0.0):
        print(f"scale {scale}", flush=True)
        ref = oattn.paged_decode(st.q64(), st.k_pool, st.v_pool, st.tables, st.ctx, scale,
                                 wl.kv_dtype, st.k_scale, st.v_scale)
        for impl in (1, 2):
            for ps in (0, 64):
                out = torch.empty_like(g.q)
                g.cache.decode(g.q, out, g.tables, g.lens, scale, wl.max_context_len, ps,
                               impl=impl)
                torch.cuda.synchronize()
                err = np.abs(out_host(out) - ref).max()
                assert err <= TOL[kv], (scale, impl, ps, err)


def test_side_stream_matches_default_stream():
    """A decode (and a copy of blocks) launched on a side stream, with the wrapper allocating
    its workspace and uploading its pairs there, gives the default stream's output."""
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    wl = workloads.random_small(331, S=6, Hq=8, Hkv=2, D=128, B=16, max_ctx=2500, min_ctx=900,
                                kv_dtype="bf16", in_dtype="bf16")
    g = GpuState(wl)
    ref = g.decode(0, IMPLS["mfma"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        out = torch.empty_like(g.q)
        out.record_stream(side)
        pkv.paged_attn_decode(g.q, g.cache.k_pool, g.cache.v_pool, g.tables, g.lens, wl.scale,
                              out, g.desc, wl.max_context_len, 0, impl=IMPLS["mfma"],
                              stream=side)
        outs.append(out)
        # the freed workspace must not be handed to this allocation while the decode runs
        junk = torch.full((1 << 22,), 7, dtype=torch.int32, device="cuda")
        del junk
    side.synchronize()
    for out in outs:
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    # copy_blocks with host pairs uploaded on the side stream
    k0 = g.cache.k_pool.clone()
    used = set(g.tables.cpu().numpy().ravel().tolist()) - {-1}
    free = [b for b in range(wl.num_blocks) if b not in used]
    src = sorted(used)[:2]
    pairs = [(src[0], free[0]), (src[1], free[1])]
    pkv.copy_blocks(g.cache.k_pool, g.cache.v_pool, pairs, g.desc, stream=side)
    side.synchronize()
    for s_, d_ in pairs:
        assert torch.equal(g.cache.k_pool[d_].view(torch.int16), k0[s_].view(torch.int16))
