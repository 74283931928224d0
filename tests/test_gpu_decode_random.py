"""Seeded random sweep of the decode against the fp64 oracle: batch size, head group, head
size, block size, pool dtype, context lengths and partition size drawn per case, both kernel
families, at the workload's softmax scale and at a 16 times larger one.  Errors are held to
the dtype's tolerance and to the per-element bound of the kernel's rounding.  Each case is
small enough for the oracle to finish in well under a second."""
import numpy as np
import pytest

import workloads
from gpu_util import PEAK, TOL, GpuState, out_host, peaked_tol, rounding_bound
from oracle_pipeline import decode as oracle_decode
from oracle_pipeline import run as oracle_run

pytestmark = pytest.mark.gpu


def _draw(seed):
    rng = np.random.default_rng(9000 + seed)
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    B = int(rng.choice([8, 16, 32]))
    max_ctx = int(rng.choice([1, 17, 100, 700, 2500]))
    return dict(seed=5000 + seed, S=int(rng.integers(1, 41)), Hq=g * hkv, Hkv=hkv,
                D=int(rng.choice([64, 128])), B=B, max_ctx=max_ctx,
                min_ctx=int(rng.integers(1, max_ctx + 1)) if rng.random() < 0.3 else 1,
                kv_dtype=str(rng.choice(["bf16", "fp8"])), in_dtype="bf16",
                ps=int(rng.choice([0, B, 2 * B, 256, 1024])))


def _draw_wide(seed):
    """Batches of 100 to 400 sequences: more (sequence, KV head) pairs than a quarter of the
    workers, so the bf16 decode runs all of them (the small draws above run half)."""
    rng = np.random.default_rng(9500 + seed)
    hkv = int(rng.choice([2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8, 16]))
    B = int(rng.choice([8, 16, 32]))
    max_ctx = int(rng.choice([33, 200, 700]))
    return dict(seed=5500 + seed, S=int(rng.integers(100, 401)), Hq=g * hkv, Hkv=hkv,
                D=int(rng.choice([64, 128])), B=B, max_ctx=max_ctx, min_ctx=1,
                kv_dtype=str(rng.choice(["bf16", "fp8"])), in_dtype="bf16",
                ps=int(rng.choice([0, B, 256])))


CASES = [_draw(i) for i in range(24)] + [_draw_wide(i) for i in range(12)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c['seed']}")
def test_random_shape(case):
    case = dict(case)
    ps = case.pop("ps")
    wl = workloads.random_small(**case)
    print(f"random case {case} ps {ps}", flush=True)
    st = oracle_run(wl)
    g = GpuState(wl)
    # the workload's scale, then a peaked softmax whose outputs are single tokens' values
    for scale in (wl.scale, PEAK * wl.scale):
        ref = oracle_decode(st, scale=scale)
        bound = rounding_bound(st, ref, scale)
        tol = TOL[wl.kv_dtype] if scale == wl.scale else peaked_tol(wl.kv_dtype, ref)
        for impl in (2, 1):
            for p in (ps, 0):
                err = np.abs(out_host(g.decode(p, impl, scale=scale)) - ref)
                assert (err <= tol).all(), (scale, impl, p, err.max())
                assert (err <= bound).all(), (scale, impl, p, (err / bound).max())
