"""Seeded random sweep of the decode against the fp64 oracle: batch size, head group, head
size, block size, pool dtype, context lengths and partition size drawn per case, both kernel
families.  Each case is small enough for the oracle to finish in well under a second."""
import numpy as np
import pytest

import workloads
from gpu_util import TOL, GpuState, out_host
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


CASES = [_draw(i) for i in range(24)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c['seed']}")
def test_random_shape(case):
    case = dict(case)
    ps = case.pop("ps")
    wl = workloads.random_small(**case)
    print(f"random case {case} ps {ps}", flush=True)
    ref = oracle_decode(oracle_run(wl))
    g = GpuState(wl)
    for impl in (2, 1):
        for p in (ps, 0):
            out = out_host(g.decode(p, impl))
            err = np.abs(out - ref).max()
            assert err <= TOL[wl.kv_dtype], (impl, p, err)
