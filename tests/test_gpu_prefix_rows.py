"""GPU parity of the shared-prefix decode: forked samples form units that read their
shared prompt blocks once for all members' queries, then each member's own tokens; the
result must match the fp64 oracle within the dtype tolerance and the plain decode of the
same state, and with no shared run it must be the plain decode bit for bit."""
import numpy as np
import pytest

from gpu_util import TOL, GpuState, out_host, torch_mod
from oracle_pipeline import decode as oracle_decode
from oracle_pipeline import run as oracle_run
from test_gpu_cache_ops import _shared_prefix_small

pytestmark = pytest.mark.gpu


def _rows_decode(g, rows, seq_rows, ps, shared_blocks=False):
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    wl = g.wl
    out = torch.empty_like(g.q)
    pkv.paged_attn_decode_rows(g.q, g.cache.k_pool, g.cache.v_pool, g.tables, g.lens, wl.scale,
                               out, g.desc, wl.max_context_len, ps, rows, seq_rows,
                               shared_blocks=shared_blocks)
    torch.cuda.synchronize()
    return out


def _rows(g, group, min_blocks=1):
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    t = g.tables.cpu().numpy()
    ln = g.lens.cpu().numpy()
    rows, seq_rows = pkv.prefix_rows(t, ln, g.wl.block_size, group, min_blocks)
    return rows, seq_rows, torch.from_numpy(rows).cuda(), torch.from_numpy(seq_rows).cuda()


CASES = [
    dict(seed=401, prompts=3, n=4, prefix=40, D=64, Hkv=2, g=2),
    dict(seed=402, prompts=3, n=4, prefix=200, D=128, Hkv=2, g=4),
    dict(seed=403, prompts=2, n=4, prefix=520, D=128, Hkv=4, g=4, max_tail=300),
    dict(seed=404, prompts=2, n=3, prefix=97, D=128, Hkv=1, g=5),
    dict(seed=405, prompts=3, n=4, prefix=200, D=128, Hkv=2, g=4, kv_dtype="fp8"),
    dict(seed=406, prompts=2, n=4, prefix=130, D=64, Hkv=2, g=4, B=8),
    dict(seed=407, prompts=2, n=4, prefix=300, D=128, Hkv=2, g=2, B=32),
    # units wider than one 16-column tile: both query tiles of the kernel in use
    dict(seed=408, prompts=2, n=8, prefix=200, D=128, Hkv=2, g=4),
    dict(seed=409, prompts=2, n=8, prefix=300, D=128, Hkv=2, g=4, kv_dtype="fp8"),
    dict(seed=411, prompts=2, n=6, prefix=150, D=128, Hkv=1, g=5),
    dict(seed=412, prompts=1, n=32, prefix=100, D=64, Hkv=2, g=1, B=8),
    dict(seed=413, prompts=2, n=12, prefix=90, D=128, Hkv=2, g=2, B=32),
    dict(seed=414, prompts=2, n=5, prefix=140, D=64, Hkv=2, g=4, kv_dtype="fp8", B=16),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c['seed']}")
def test_rows_match_oracle_and_plain_decode(case):
    wl = _shared_prefix_small(**case)
    print(f"rows case {case}", flush=True)
    g = GpuState(wl)
    st = oracle_run(wl)
    ref = oracle_decode(st)
    group = wl.num_q_heads // wl.num_kv_heads
    rows, seq_rows, rows_d, sr_d = _rows(g, group)
    # every prompt's samples form one unit sharing the prompt's full blocks (the half-full
    # last prompt block was copied on the first divergent write)
    n, B = case["n"], wl.block_size
    assert n <= 32 // group
    assert len(rows) == case["prompts"], rows
    assert (rows[:, 1] == (case["prefix"] // B) * B).all() and (rows[:, 2] == n).all(), rows
    tol = TOL[wl.kv_dtype]
    plain = out_host(g.decode(0, 2))
    for ps in (0, 32, 256):
        out = out_host(_rows_decode(g, rows_d, sr_d, ps))
        err = np.abs(out - ref).max()
        assert err <= tol, (ps, err)
        assert np.abs(out - plain).max() <= tol


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_prompt_wider_than_a_unit_reread_with_cached_loads(kv):
    """12 samples of 4 heads per prompt: units of 8 and 4 members share the prompt, both
    flagged as read again; the decode with cached loads (the launch hint) gives the
    streaming decode's result bit for bit, within tolerance of the oracle."""
    torch = torch_mod()
    wl = _shared_prefix_small(415, prompts=2, n=12, prefix=200, D=128, Hkv=2, g=4,
                              kv_dtype=kv)
    print(f"rows reread case {kv}", flush=True)
    g = GpuState(wl)
    ref = oracle_decode(oracle_run(wl))
    rows, seq_rows, rows_d, sr_d = _rows(g, 4)
    assert rows[:, 2].tolist() == [8, 4, 8, 4] and (rows[:, 3] == 1).all(), rows
    for ps in (0, 128):
        a = _rows_decode(g, rows_d, sr_d, ps)
        b = _rows_decode(g, rows_d, sr_d, ps, shared_blocks=True)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), ps
        assert np.abs(out_host(b) - ref).max() <= TOL[kv], ps


def test_more_than_256_units():
    """300 prompts of two samples each: 300 units, so the workers find their start with the
    chunked scan over the unit descriptors (more than one group of 256)."""
    wl = _shared_prefix_small(416, prompts=300, n=2, prefix=40, D=64, Hkv=2, g=2, max_tail=20)
    print("300 units", flush=True)
    g = GpuState(wl)
    ref = oracle_decode(oracle_run(wl))
    rows, seq_rows, rows_d, sr_d = _rows(g, 2)
    assert len(rows) == 300 and (rows[:, 2] == 2).all(), rows[:4]
    plain = out_host(g.decode(0, 2))
    for ps in (0, 64):
        out = out_host(_rows_decode(g, rows_d, sr_d, ps))
        assert np.abs(out - ref).max() <= TOL[wl.kv_dtype], ps
        assert np.abs(out - plain).max() <= TOL[wl.kv_dtype], ps


def test_no_shared_run_is_the_plain_decode_bit_for_bit():
    torch = torch_mod()
    wl = _shared_prefix_small(410, prompts=2, n=4, prefix=100, D=128, Hkv=2, g=4)
    g = GpuState(wl)
    group = wl.num_q_heads // wl.num_kv_heads
    # a minimum longer than the prompt: every unit is a plain sequence
    rows, seq_rows, rows_d, sr_d = _rows(g, group, min_blocks=100)
    assert len(rows) == len(g.seqs) and (rows[:, 1] == 0).all() and (rows[:, 2] == 1).all()
    for ps in (0, 64):
        a = _rows_decode(g, rows_d, sr_d, ps)
        b = g.decode(ps, 2)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_interleaved_families_are_not_grouped():
    """Samples of different prompts alternating in the batch share nothing with their
    neighbours: no group is formed and the result is still right."""
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    wl = _shared_prefix_small(411, prompts=2, n=2, prefix=64, D=64, Hkv=2, g=2)
    g = GpuState(wl)
    order = [0, 2, 1, 3]                       # prompt 0, prompt 1, prompt 0, prompt 1
    t = g.tables.cpu().numpy()[order]
    ln = g.lens.cpu().numpy()[order]
    rows, seq_rows = pkv.prefix_rows(t, ln, wl.block_size, 2, 1)
    assert (rows[:, 2] == 1).all()
    st = oracle_run(wl)
    ref = oracle_decode(st)[order]
    q = g.q[order].contiguous()
    out = torch.empty_like(q)
    pkv.paged_attn_decode_rows(q, g.cache.k_pool, g.cache.v_pool,
                               g.tables[order].contiguous(), g.lens[order].contiguous(),
                               wl.scale, out, g.desc, wl.max_context_len, 0,
                               torch.from_numpy(rows).cuda(), torch.from_numpy(seq_rows).cuda())
    torch.cuda.synchronize()
    assert np.abs(out_host(out) - ref).max() <= TOL["bf16"]


def test_interleaved_families_regrouped_by_prefix_order():
    """The same interleaved batch, put in the library's prefix order: the families become
    consecutive, form units, and every sequence's output is the oracle's."""
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    wl = _shared_prefix_small(413, prompts=3, n=4, prefix=150, D=128, Hkv=2, g=4)
    g = GpuState(wl)
    inter = np.array([0, 4, 8, 1, 5, 9, 2, 6, 10, 3, 7, 11])
    t = g.tables.cpu().numpy()[inter]
    ln = g.lens.cpu().numpy()[inter]
    assert (pkv.prefix_rows(t, ln, wl.block_size, 4, 1)[0][:, 2] == 1).all()
    order = inter[pkv.prefix_order(t, ln, wl.block_size)]
    rows, seq_rows = pkv.prefix_rows(g.tables.cpu().numpy()[order], g.lens.cpu().numpy()[order],
                                     wl.block_size, 4, 1)
    assert len(rows) == 3 and (rows[:, 2] == 4).all()
    ref = oracle_decode(oracle_run(wl))[order]
    idx = torch.from_numpy(order).cuda()
    q = g.q[idx].contiguous()
    out = torch.empty_like(q)
    pkv.paged_attn_decode_rows(q, g.cache.k_pool, g.cache.v_pool, g.tables[idx].contiguous(),
                               g.lens[idx].contiguous(), wl.scale, out, g.desc,
                               wl.max_context_len, 0, torch.from_numpy(rows).cuda(),
                               torch.from_numpy(seq_rows).cuda())
    torch.cuda.synchronize()
    assert np.abs(out_host(out) - ref).max() <= TOL["bf16"]


def test_split_phases_equal_the_single_call():
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    wl = _shared_prefix_small(412, prompts=3, n=4, prefix=200, D=128, Hkv=2, g=4)
    g = GpuState(wl)
    rows, seq_rows, rows_d, sr_d = _rows(g, 4)
    ws = torch.empty(pkv.rows_workspace_bytes(g.desc, len(rows)), dtype=torch.uint8,
                     device="cuda")
    outs = []
    for phases in ((3,), (1, 2)):
        out = torch.empty_like(g.q)
        for ph in phases:
            pkv.paged_attn_decode_rows(g.q, g.cache.k_pool, g.cache.v_pool, g.tables, g.lens,
                                       wl.scale, out, g.desc, wl.max_context_len, 0, rows_d,
                                       sr_d, workspace=ws, phases=ph)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


@pytest.mark.parametrize("kv_dtype,D", [("bf16", 128), ("fp8", 64)])
def test_hand_built_units(kv_dtype, D):
    """Units the builder would not make but the kernel accepts: members that share no
    tokens (every member reads its own table), one-member units whose context is cut in
    two spans, and a last unit of a single sequence.  Each equals the oracle."""
    import workloads

    torch = torch_mod()
    wl = workloads.random_small(421, S=9, Hq=8, Hkv=2, D=D, B=16, max_ctx=700,
                                kv_dtype=kv_dtype, in_dtype="bf16", min_ctx=40)
    g = GpuState(wl)
    ref = oracle_decode(oracle_run(wl))
    lens = g.lens.cpu().numpy()
    units = np.array([[0, 0, 3, 0],                        # 0, 1, 2: no shared tokens
                      [3, 32, 1, 0],                       # 3: [0, 32) then [32, len)
                      [4, (int(lens[4]) // 16) * 16, 1, 0],  # 4: all full blocks, then the rest
                      [5, 0, 2, 0], [7, 0, 1, 0], [8, 16, 1, 0]], dtype=np.int32)
    seq_rows = np.zeros((9, 4), dtype=np.int32)
    for u, (s0, T, M, _) in enumerate(units):
        for m in range(M):
            seq_rows[s0 + m, :2] = [u, m]
    rows_d = torch.from_numpy(units).cuda()
    sr_d = torch.from_numpy(seq_rows).cuda()
    for ps in (0, 32, 128):
        out = out_host(_rows_decode(g, rows_d, sr_d, ps))
        assert np.abs(out - ref).max() <= TOL[kv_dtype], ps


def test_units_with_empty_and_single_token_members():
    """A unit of three members without shared tokens, one of them empty, and a unit whose
    members share one block and have one own token each: the empty member gets zeros, a
    one-token context returns its value row exactly."""
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    D, B, H = 128, 16, 2
    desc = pkv.cache_desc(8, H, B, D, "bf16")
    kp, vp = pkv.alloc_pools(desc)
    x = torch.randn(5, H, D, device="cuda").to(torch.bfloat16)
    # blocks 1..3 hold one token each; block 4 holds 16 shared tokens, blocks 5, 6 one each
    slots = [16, 32, 48] + list(range(64, 80))
    xs = torch.randn(len(slots), H, D, device="cuda").to(torch.bfloat16)
    xs[:3] = x[:3]
    pkv.reshape_and_cache(xs, xs, torch.tensor(slots, device="cuda"), kp, vp, desc)
    pkv.reshape_and_cache(x[3:], x[3:], torch.tensor([80, 96], device="cuda"), kp, vp, desc)
    q = torch.randn(5, 4 * H, D, device="cuda").to(torch.bfloat16)
    tables = torch.tensor([[1, -1], [-1, -1], [3, -1], [4, 5], [4, 6]], dtype=torch.int32,
                          device="cuda")
    lens = torch.tensor([1, 0, 1, 17, 17], dtype=torch.int32, device="cuda")
    units = torch.tensor([[0, 0, 3, 0], [3, 16, 2, 0]], dtype=torch.int32, device="cuda")
    seq_rows = torch.tensor([[0, 0, 0, 0], [0, 1, 0, 0], [0, 2, 0, 0], [1, 0, 0, 0],
                             [1, 1, 0, 0]], dtype=torch.int32, device="cuda")
    ref = torch.empty_like(q)
    pkv.paged_attn_decode(q, kp, vp, tables, lens, 0.1, ref, desc, 32, 0, impl=2)
    for ps in (0, 32):
        out = torch.full_like(q, 7.0)
        pkv.paged_attn_decode_rows(q, kp, vp, tables, lens, 0.1, out, desc, 32, ps, units,
                                   seq_rows)
        torch.cuda.synchronize()
        assert torch.equal(out[1].float(), torch.zeros_like(out[1].float()))
        for s in (0, 2):
            assert torch.equal(out[s].float(), x[s].float().repeat_interleave(4, dim=0))
        assert (out[3:].float() - ref[3:].float()).abs().max().item() <= TOL["bf16"]


def test_timing_hook_covers_the_unit_decode():
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    wl = _shared_prefix_small(414, prompts=2, n=4, prefix=200, D=128, Hkv=2, g=4)
    g = GpuState(wl)
    rows, seq_rows, rows_d, sr_d = _rows(g, 4)
    ref = _rows_decode(g, rows_d, sr_d, 0)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for x in e:
        x.record()
    torch.cuda.synchronize()
    pkv.time_next_decode(e[0], e[1])
    out = _rows_decode(g, rows_d, sr_d, 0)
    assert 0 < e[0].elapsed_time(e[1]) < 1000
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
