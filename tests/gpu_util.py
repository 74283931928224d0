"""GPU side of a workload, built through the HIP library only (tests' helper)."""
from __future__ import annotations

import numpy as np

import workloads


def torch_mod():
    import torch
    return torch


def gpu_available() -> bool:
    torch = torch_mod()
    return torch.cuda.is_available()


def desc_of(wl, pkv):
    k_scale, v_scale = wl.kv_scales()
    return pkv.cache_desc(wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim,
                          wl.kv_dtype, k_scale, v_scale)


class GpuState:
    """Pools filled through reshape_and_cache / copy_blocks from the workload's script,
    then the decode step's append + write; tables and lengths on the device."""

    def __init__(self, wl, keep=None, poison=True, workers=8, free_order=None):
        import paged_kv_cache_104_amd as pkv
        from paged_kv_cache_104_amd.engine import PagedKVCache, to_device

        torch = torch_mod()
        self.wl = wl
        self.pkv = pkv
        self.desc = desc_of(wl, pkv)
        fo = wl.free_order if free_order is None else free_order
        self.cache = PagedKVCache(self.desc, fo, device="cuda", poison=poison,
                                  prefix_caching=wl.prefix_caching)
        feeder = workloads.KVFeeder(wl, workloads.ops_seq_order(wl.setup_ops)
                                    + [int(s) for s in wl.decode_seqs], workers=workers)
        live = wl.data_seqs()
        kp = keep if keep is not None else (lambda s: True)
        last = {int(s): int(c) - 1 for s, c in zip(wl.decode_seqs, wl.ctx_lens)}
        new_rows = {}

        def source(seq):
            k, v = feeder(seq)
            if seq in last and seq not in new_rows:
                new_rows[seq] = (k[last[seq]].copy(), v[last[seq]].copy())
            return k, v

        try:
            self.cache.run_script(wl.setup_ops, source, wl.in_dtype,
                                  keep=lambda s: s in live and kp(s))
            seqs = [int(s) for s in wl.decode_seqs]
            for s in seqs:
                if s not in new_rows:
                    source(s)
        finally:
            feeder.close()
        kn = [new_rows[s][0] for s in seqs]
        vn = [new_rows[s][1] for s in seqs]
        self.k_new = to_device(np.stack(kn), wl.in_dtype, "cuda")
        self.v_new = to_device(np.stack(vn), wl.in_dtype, "cuda")
        self.slots, self.pairs = self.cache.append_and_write(seqs, self.k_new, self.v_new)
        self.seqs = seqs
        self.tables, self.lens = self.cache.tables(seqs, wl.max_blocks_per_seq)
        self.q = to_device(wl.q_input(), wl.in_dtype, "cuda")
        torch.cuda.synchronize()

    def decode(self, partition_size=None, impl=0, out=None):
        torch = torch_mod()
        wl = self.wl
        ps = wl.partition_size if partition_size is None else partition_size
        out = torch.empty_like(self.q) if out is None else out
        self.cache.decode(self.q, out, self.tables, self.lens, wl.scale, wl.max_context_len,
                          ps, impl=impl)
        torch.cuda.synchronize()
        return out

    def pools_host(self):
        """Pools as numpy arrays in the oracle's storage format."""
        torch = torch_mod()
        k, v = self.cache.k_pool, self.cache.v_pool
        if self.wl.kv_dtype == "bf16":
            return (k.view(torch.int16).cpu().numpy().view(np.uint16),
                    v.view(torch.int16).cpu().numpy().view(np.uint16))
        return k.cpu().numpy(), v.cpu().numpy()


def out_host(t) -> np.ndarray:
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


TOL = {"f32": 1e-5, "bf16": 1.5e-2, "fp8": 3e-2}


def pools_equal_bits(a: np.ndarray, b: np.ndarray) -> bool:
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))
