"""Prefix caching on the GPU: decoding a batch whose prompts found most of their blocks
cached gives bit for bit the output of the same contexts written out in full.

The chat workload's K/V draws follow its token structure (one stream per system
prompt, question and reply), so a block found cached holds exactly the K/V the
request would have written; the decode kernel accumulates in logical token
order only, so placement and sharing cannot change a bit of the output.
"""
import dataclasses
import math

import numpy as np
import pytest

import workloads
from gpu_util import TOL, GpuState, out_host, torch_mod
from oracle_pipeline import decode as oracle_decode
from oracle_pipeline import run as oracle_run

pytestmark = pytest.mark.gpu


def _written_out(wl):
    """The same decode batch with every context written in full, no caching."""
    ops = [("add", int(s), int(c) - 1) for s, c in zip(wl.decode_seqs, wl.ctx_lens)]
    N = int(math.ceil(1.25 * sum(workloads.blocks_for(int(c), wl.block_size)
                                 for c in wl.ctx_lens)))
    order = np.random.default_rng(17).permutation(N).astype(np.int32)
    return dataclasses.replace(wl, setup_ops=ops, extra_segments={}, prefix_caching=False,
                               num_blocks=N, free_order=order, _cache={}, name=wl.name + "-plain")


def test_chat_prefix_cache_equals_written_out():
    torch = torch_mod()
    wl = workloads.get("chat-prefix-cache-bf16")
    g = GpuState(wl, workers=16)
    st = g.cache.bm.cache_stats()
    print(f"cache stats {st}", flush=True)
    assert st["hit_tokens"] > 0.8 * st["query_tokens"]
    assert g.cache.shares_blocks()
    out = g.decode()
    plain = GpuState(_written_out(wl), workers=16)
    assert not plain.cache.shares_blocks()
    ref = plain.decode()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_small_chat_against_oracle():
    """A scaled-down chat script (evictions included) through the oracle's prefix cache."""
    torch = torch_mod()
    B, vocab = 16, 50
    rng = np.random.default_rng(3)
    sys_tok = [rng.integers(0, vocab, size=n) for n in (40, 70)]
    ops, extra, segs, ctx, turn2 = [], {}, [], [], []
    for u in range(6):                                   # first turns, released
        k = u % 2
        q1 = rng.integers(0, vocab, size=20 + u)
        r1 = rng.integers(0, vocab, size=9 + 2 * u)
        sid = 100 + u
        ops += [("add_tokens", sid, np.concatenate([sys_tok[k], q1])), ("extend_tokens", sid, r1),
                ("free", sid)]
        extra[sid] = [(20 + k, 0, len(sys_tok[k])), (30 + u, 0, len(q1)), (40 + u, 0, len(r1))]
        q2 = rng.integers(0, vocab, size=5 + u)
        if u % 3 != 2:                                    # four second turns form the batch
            turn2.append(("add_tokens", len(segs), np.concatenate([sys_tok[k], q1, r1, q2])))
            segs.append([(20 + k, 0, len(sys_tok[k])), (30 + u, 0, len(q1)), (40 + u, 0, len(r1)),
                         (50 + u, 0, len(q2) + 1)])
            ctx.append(len(sys_tok[k]) + len(q1) + len(r1) + len(q2) + 1)
    ops += turn2
    need = sum(workloads.blocks_for(c, B) for c in ctx)
    N = need - 6                                          # small pool: some released blocks evicted
    wl = workloads.Workload(
        name="small-chat", seed=21, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=B,
        num_blocks=N, kv_dtype="bf16", in_dtype="bf16", scale=1 / math.sqrt(128),
        partition_size=0, free_order=np.random.default_rng(4).permutation(N).astype(np.int32),
        setup_ops=ops, decode_seqs=np.arange(4, dtype=np.int64),
        ctx_lens=np.asarray(ctx, dtype=np.int64), _segments=lambda i: segs[i],
        extra_segments=extra, prefix_caching=True)
    ost = oracle_run(wl)
    assert ost.alloc.stats()["hit_tokens"] > 0
    g = GpuState(wl)
    assert np.array_equal(g.tables.cpu().numpy(), ost.tables)
    gk, gv = g.pools_host()
    used = sorted({int(b) for row, n in zip(ost.tables, ost.ctx)
                   for b in row[: -(-int(n) // B)]})
    assert np.array_equal(gk[used], ost.k_pool[used]) and np.array_equal(gv[used], ost.v_pool[used])
    for impl in (1, 2):
        out = out_host(g.decode(0, impl))
        assert np.abs(out - oracle_decode(ost)).max() <= TOL["bf16"]
    assert torch.cuda.is_available()
