"""The no-allocation decode (pkv_paged_attn_decode_noalloc): the library's static scratch
instead of a caller's workspace.

It runs the kernels of pkv_paged_attn_decode, so its output must equal that entry point's
bit for bit, and both must be within the dtype tolerance of the fp64 oracle.  Two calls in
a row, the second on a smaller batch, check that whatever the first call left in the
scratch does not matter; the matrix-core and vector kernels, with and without partitions,
both run.  A batch whose pieces exceed the scratch is refused."""
import numpy as np
import pytest

import workloads
from gpu_util import TOL, GpuState, out_host, torch_mod
from oracle_pipeline import decode as oracle_decode
from oracle_pipeline import run as oracle_run

pytestmark = pytest.mark.gpu


def _both(g, wl, rows, ps, impl):
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    q = g.q[:rows].contiguous()
    t = g.tables[:rows].contiguous()
    ln = g.lens[:rows].contiguous()
    ref = torch.empty_like(q)
    pkv.paged_attn_decode(q, g.cache.k_pool, g.cache.v_pool, t, ln, wl.scale, ref, g.desc,
                          wl.max_context_len, ps, impl=impl)
    out = torch.full_like(q, 3.0)
    pkv.paged_attn_decode_noalloc(q, g.cache.k_pool, g.cache.v_pool, t, ln, wl.scale, out,
                                  g.desc, wl.max_context_len, ps, impl=impl)
    torch.cuda.synchronize()
    return out, ref


@pytest.mark.parametrize("kv,impl", [("bf16", 2), ("fp8", 2), ("bf16", 1), ("f32", 1)])
def test_noalloc_matches_workspace_decode(kv, impl):
    torch = torch_mod()
    wl = workloads.random_small(340 + impl, S=12, Hq=8, Hkv=2, D=128 if kv != "f32" else 64,
                                B=16, max_ctx=2500, min_ctx=300, kv_dtype=kv,
                                in_dtype="f32" if kv == "f32" else "bf16")
    print(f"noalloc {kv} impl {impl}", flush=True)
    ref_o = oracle_decode(oracle_run(wl))
    g = GpuState(wl)
    for rows, ps in ((12, 256), (5, 0), (12, 0), (3, 512)):   # larger, then smaller batches
        out, ref = _both(g, wl, rows, ps, impl)
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                           ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref), (rows, ps)
        err = np.abs(out_host(out) - ref_o[:rows]).max()
        assert err <= TOL[kv], (rows, ps, err)


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    # f32 pool, vector kernel, one-block partitions: S * Hq * P rows of (D + 2) floats
    S, Hq, D, B = 64, 16, 64, 16
    desc = pkv.cache_desc(8, Hq, B, D, "f32")
    kp, vp = pkv.alloc_pools(desc)
    q = torch.zeros(S, Hq, D, device="cuda")
    out = torch.empty_like(q)
    tables = torch.zeros(S, 1024, dtype=torch.int32, device="cuda")
    lens = torch.ones(S, dtype=torch.int32, device="cuda")
    need = S * Hq * (1024 * B // B) * (D + 2) * 4
    assert need > pkv.decode_scratch_bytes()
    with pytest.raises(pkv.PagedKVError, match="scratch"):
        pkv.paged_attn_decode_noalloc(q, kp, vp, tables, lens, 0.1, out, desc, 1024 * B, B)
