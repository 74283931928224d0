"""The decode step's append with device-resident block tables (append_tokens / DecodeBatch)
against the upload path (block manager tables + reshape_and_cache): same pools bit for bit,
the same device tables and lengths as the block manager after every step, and the same
decode output -- over steps that cross block boundaries, copy shared blocks on write, and
batches of more than one launch (256 tokens each)."""
import numpy as np
import pytest

from gpu_util import torch_mod

pytestmark = pytest.mark.gpu


def _engine(desc, N, seed):
    from paged_kv_cache_104_amd.engine import PagedKVCache

    order = np.random.default_rng(seed).permutation(N).astype(np.int32)
    return PagedKVCache(desc, order, device="cuda", poison=True)


def _setup(cache, rng, torch, S, H, D, forks):
    """S sequences with random contexts (written), and `forks` forked samples of seq 0."""
    for s in range(S):
        n = int(rng.integers(1, 60))
        cache.bm.add_seq(s, n)
        x = torch.from_numpy(rng.standard_normal((n, H, D), dtype=np.float32)).to(torch.bfloat16)
        cache.write(x.cuda(), (-x).cuda(), cache.bm.slots(s, 0, n))
    for f in range(forks):
        cache.bm.fork(0, S + f)
    return list(range(S + forks))


@pytest.mark.parametrize("S,forks", [(7, 3), (300, 2)])
def test_device_tables_follow_the_block_manager(S, forks):
    import paged_kv_cache_104_amd as pkv
    from paged_kv_cache_104_amd.engine import DecodeBatch

    torch = torch_mod()
    H, D, B = 2, 64, 16
    N = S * 8 + 64
    desc = pkv.cache_desc(N, H, B, D, "bf16")
    a, b = _engine(desc, N, 1), _engine(desc, N, 1)
    seqs = _setup(a, np.random.default_rng(2), torch, S, H, D, forks)
    _setup(b, np.random.default_rng(2), torch, S, H, D, forks)
    mb = 12
    batch = DecodeBatch(a, seqs, mb)
    rng = np.random.default_rng(3)
    q = torch.randn(len(seqs), 4 * H, D, device="cuda").to(torch.bfloat16)
    saw_copy = False
    for step in range(20):                           # crosses block boundaries
        kn = torch.from_numpy(rng.standard_normal((len(seqs), H, D), dtype=np.float32))
        kn = kn.to(torch.bfloat16).cuda()
        vn = (kn * 0.5).contiguous()
        s1, p1 = batch.append(kn, vn)
        s2, p2 = b.append_and_write(seqs, kn, vn)
        saw_copy |= len(p1) > 0
        assert np.array_equal(s1, s2) and np.array_equal(p1, p2)
        t, l = a.bm.block_tables(seqs, mb)
        torch.cuda.synchronize()
        assert np.array_equal(batch.tables.cpu().numpy(), t)
        assert np.array_equal(batch.lens.cpu().numpy(), l)
    assert saw_copy                                  # the forks copied their shared block
    assert torch.equal(a.k_pool.view(torch.int16), b.k_pool.view(torch.int16))
    assert torch.equal(a.v_pool.view(torch.int16), b.v_pool.view(torch.int16))
    tb, lb = b.tables(seqs, mb)
    oa, ob = torch.empty_like(q), torch.empty_like(q)
    a.decode(q, oa, batch.tables, batch.lens, 0.125, mb * B, 0)
    b.decode(q, ob, tb, lb, 0.125, mb * B, 0)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


def test_append_tokens_checks_positions():
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    desc = pkv.cache_desc(8, 1, 16, 64, "bf16")
    kp, vp = pkv.alloc_pools(desc)
    x = torch.zeros(2, 1, 64, dtype=torch.bfloat16, device="cuda")
    tables = torch.full((2, 4), -1, dtype=torch.int32, device="cuda")
    lens = torch.zeros(2, dtype=torch.int32, device="cuda")
    for slots, pos in (([17, 3], [1, 4]),          # pos % 16 != slot % 16
                       ([17, 200], [1, 0]),        # slot outside the pool
                       ([17, 3], [1, 64 + 3])):    # position beyond the table
        with pytest.raises(pkv.PagedKVError):
            pkv.append_tokens(x, x, slots, pos, kp, vp, desc, tables, lens)
    pkv.append_tokens(x, x, [17, -1], [1, 0], kp, vp, desc, tables, lens)
    torch.cuda.synchronize()
    assert tables.cpu().tolist() == [[1, -1, -1, -1], [-1, -1, -1, -1]]
    assert lens.cpu().tolist() == [2, 0]
