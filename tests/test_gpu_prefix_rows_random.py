"""Seeded random sweep of the shared-prefix decode against the fp64 oracle: prompts, samples
per prompt (families wider than one unit included), prefix length, tails, head group, head
size, block size and pool dtype drawn per case, with and without the cached-load hint, at the
workload's softmax scale and at a 16 times larger one; errors held to the tolerance and to
the per-element rounding bound of the kernel's arithmetic."""
import numpy as np
import pytest

from gpu_util import PEAK, TOL, GpuState, out_host, peaked_tol, rounding_bound, torch_mod
from oracle_pipeline import decode as oracle_decode
from oracle_pipeline import run as oracle_run
from test_gpu_cache_ops import _shared_prefix_small

pytestmark = pytest.mark.gpu


def _draw(seed):
    rng = np.random.default_rng(7000 + seed)
    return dict(seed=6000 + seed, prompts=int(rng.integers(1, 7)), n=int(rng.integers(1, 13)),
                prefix=int(rng.integers(1, 600)), B=int(rng.choice([8, 16, 32])),
                Hkv=int(rng.choice([1, 2])), D=int(rng.choice([64, 128])),
                g=int(rng.choice([1, 2, 4, 8, 16])), max_tail=int(rng.integers(1, 300)),
                kv_dtype=str(rng.choice(["bf16", "fp8"]))), bool(rng.random() < 0.5), \
        int(rng.choice([0, 64, 512]))


CASES = [_draw(i) for i in range(16)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]['seed']}")
def test_random_families(case):
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    kw, cached, ps = case
    wl = _shared_prefix_small(**kw)
    print(f"random families {kw} cached {cached} ps {ps}", flush=True)
    g = GpuState(wl)
    st = oracle_run(wl)
    group = wl.num_q_heads // wl.num_kv_heads
    rows, seq_rows = pkv.prefix_rows(g.tables.cpu().numpy(), g.lens.cpu().numpy(),
                                     wl.block_size, group, 1)
    rows_d, seq_rows_d = torch.from_numpy(rows).cuda(), torch.from_numpy(seq_rows).cuda()
    for scale in (wl.scale, PEAK * wl.scale):
        ref = oracle_decode(st, scale=scale)
        tol = TOL[wl.kv_dtype] if scale == wl.scale else peaked_tol(wl.kv_dtype, ref)
        out = torch.empty_like(g.q)
        pkv.paged_attn_decode_rows(g.q, g.cache.k_pool, g.cache.v_pool, g.tables, g.lens, scale,
                                   out, g.desc, wl.max_context_len, ps, rows_d, seq_rows_d,
                                   shared_blocks=cached)
        torch.cuda.synchronize()
        err = np.abs(out_host(out) - ref)
        assert (err <= tol).all(), (scale, err.max())
        bound = rounding_bound(st, ref, scale)
        assert (err <= bound).all(), (scale, (err / bound).max())
