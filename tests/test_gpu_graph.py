"""The no-allocation decode under HIP graph capture: it allocates nothing and launches only
its kernels (no memset, no copy), so one call can be captured into a graph and replayed.
Every replay, with eager work and synchronisations between them, gives the eager call's
output bit for bit."""
import numpy as np
import pytest

import workloads
from gpu_util import GpuState, torch_mod

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_noalloc_decode_replays_from_a_graph(kv):
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    wl = workloads.random_small(341, S=10, Hq=8, Hkv=2, D=128, B=16, max_ctx=1500, min_ctx=200,
                                kv_dtype=kv, in_dtype="bf16")
    print(f"graph replay {kv}", flush=True)
    g = GpuState(wl)
    args = (g.q, g.cache.k_pool, g.cache.v_pool, g.tables, g.lens, wl.scale)

    def call(out):
        pkv.paged_attn_decode_noalloc(*args, out, g.desc, wl.max_context_len, 256)

    ref = torch.empty_like(g.q)
    call(ref)                                   # eager, also sets up the scratch address
    torch.cuda.synchronize()
    out = torch.empty_like(g.q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out)                               # a warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out)
    want = ref.view(torch.int16).cpu().numpy()
    for i in range(5):
        out.fill_(3.0)                          # eager work between replays
        other = torch.empty_like(g.q)
        call(other)                             # an eager call on the same scratch
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.view(torch.int16).cpu().numpy(), want), i
        assert np.array_equal(other.view(torch.int16).cpu().numpy(), want), i
