#!/usr/bin/env python3
"""Paged decode benchmark on one MI355X.

One step is one pass of the whole hot path over the batch:
  host   C++ block manager: append one token per sequence -> slots, copy pairs
  device copy_blocks (copy-on-write pairs, when there are any)
         append_tokens: the batch's new K/V into their slots, and the device-resident
         block tables and lengths brought up to date (slots and positions travel in
         the kernel arguments; the tables were uploaded once, before the steps)
         paged attention: decode kernel + merge of split contexts
Inputs are resident in HBM before the timed region.  Contexts grow by one
token per step, as in a real decode loop; the KV bytes of every step are
counted from the block manager's lengths.

Prints one JSON line.  `value` is the KV-read rate of the whole step
(algorithmic KV bytes / wall time of the timed steps); the `roofline` object is
the decode attention kernel alone, timed with HIP events on its stream.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: KV-read GB/s (fraction of HBM peak) + decode tokens/s"
HBM_PEAK_GBS = 8000.0
DEFAULT_CONFIG = "8b-gqa-bf16"
DOMINANT_KERNEL = "decode_mfma_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
DIAG_STEPS = 10        # untimed steps after the timed ones, with every kernel bracketed
FLUSH_STEPS = 10       # untimed steps after those, each after a write that evicts the KV
FLUSH_BYTES = 512 << 20
EVENT_EVERY = 2        # timed steps between two whose decode kernel records its own events
READ_REF_BYTES = 4 << 30


def _code_only(src: str) -> str:
    """C++ source without its comments and blank space, so that editing a comment does not
    count as a change of the kernel.  String and character literals are kept."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c == '"' or c == "'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the code of the sources the decode kernel is built from (decode.hip,
    device_common.h), comments and blank space left out."""
    h = hashlib.sha256()
    for f in ("decode.hip", "device_common.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_104_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(config: str):
    """HBM bytes per launch from committed counter runs, if taken on the current kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(config)
    if not entry or entry.get("kernel_source_sha") != kernel_source_hash():
        return None
    return entry.get("traffic_bytes_per_launch")


def build_gpu_state(wl, workers: int):
    import torch

    import workloads
    from paged_kv_cache_104_amd.engine import PagedKVCache, to_device

    import paged_kv_cache_104_amd as pkv

    k_scale, v_scale = wl.kv_scales()
    desc = pkv.cache_desc(wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim,
                          wl.kv_dtype, k_scale, v_scale)
    cache = PagedKVCache(desc, wl.free_order, device="cuda", poison=True,
                         prefix_caching=wl.prefix_caching)
    feeder = workloads.KVFeeder(wl, workloads.ops_seq_order(wl.setup_ops), workers=workers)
    last = {int(s): int(c) - 1 for s, c in zip(wl.decode_seqs, wl.ctx_lens)}
    rows = {}

    def source(seq):
        k, v = feeder(seq)
        if seq in last and seq not in rows:
            rows[seq] = (k[last[seq]].copy(), v[last[seq]].copy())
        return k, v

    live = wl.data_seqs()
    try:
        cache.run_script(wl.setup_ops, source, wl.in_dtype, keep=lambda s: s in live)
        for s in wl.decode_seqs:
            if int(s) not in rows:
                source(int(s))
    finally:
        feeder.close()
    seqs = [int(s) for s in wl.decode_seqs]
    k_new = to_device(np.stack([rows[s][0] for s in seqs]), wl.in_dtype, "cuda")
    v_new = to_device(np.stack([rows[s][1] for s in seqs]), wl.in_dtype, "cuda")
    q = to_device(wl.q_input(), wl.in_dtype, "cuda")
    torch.cuda.synchronize()
    return cache, desc, seqs, q, k_new, v_new


def run_gpu(wl, steps: int, warmup: int, partition_size: int, impl: int, workers: int,
            event_every: int = EVENT_EVERY, rows_mode: str = "auto",
            cached_loads: bool = False):
    import torch

    import paged_kv_cache_104_amd as pkv

    t_setup = time.perf_counter()
    cache, desc, seqs, q, k_new, v_new = build_gpu_state(wl, workers)
    log(f"setup {time.perf_counter() - t_setup:.1f}s: {wl.num_seqs} seqs, "
        f"{int(wl.ctx_lens.sum())} cached tokens, pool {wl.num_blocks} blocks")
    S, B = len(seqs), wl.block_size
    total = warmup + steps + DIAG_STEPS + FLUSH_STEPS
    max_ctx = wl.max_context_len + total
    max_blocks = -(-max_ctx // B)
    bytes_per_token = wl.kv_bytes_per_token()
    dev = "cuda"
    stream = torch.cuda.current_stream()
    # the batch's block tables and lengths stay on the device: uploaded once here, then each
    # step's append writes the new tokens and updates them in the same launch
    from paged_kv_cache_104_amd.engine import DecodeBatch
    st = cache.bm.stats()
    shared = st["logical_blocks"] > st["physical_blocks"]
    use_rows = shared and rows_mode != "off"
    if use_rows:
        # a serving batch's order is free: sequences that share leading blocks go next to
        # each other, so that the shared-prefix units can group them
        t_h, l_h = cache.bm.block_tables(seqs, max_blocks)
        order = pkv.prefix_order(t_h, l_h, B)
        seqs = [seqs[i] for i in order]
        idx = torch.from_numpy(order.astype(np.int64)).to(dev)
        q, k_new, v_new = q[idx].contiguous(), k_new[idx].contiguous(), v_new[idx].contiguous()
    batch = DecodeBatch(cache, seqs, max_blocks)
    out = torch.empty_like(q)
    ws_bytes = pkv.decode_workspace_bytes(S, wl.num_q_heads, wl.head_dim, max_ctx, partition_size)
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev) if ws_bytes else None
    # Every event_every-th timed step times its decode kernel: the launch itself records
    # the kernel's start and end in an event pair (pkv_time_next_decode), so the pair
    # holds the kernel alone; separate event records around it would add the idle time
    # they leave on the device (about 6 us each).  The diagnostic steps after the timed
    # ones also time the cache write and the merge; the flushed steps after those first
    # write a 512 MB scratch buffer (untimed), so that no KV line is left in the 256 MB
    # last-level cache or the L2s when the decode starts, and the cache holds dirty lines
    # of other data instead, as after the rest of a model's layer.  Every event is
    # recorded once here so none is created inside the timed loop.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(total)]
    for e in [x for row in ev for x in row]:
        e.record(stream)
    torch.cuda.synchronize()
    # forked samples share blocks: read them once for all sharers (shared-prefix units), or
    # per sequence; with cached_loads the K/V loads are ordinary ones that leave lines in the
    # caches for other readers (the shared-blocks hint) instead of streaming
    if use_rows:
        rows_d, seq_rows_d, reread = batch.shared_prefix_rows(wl.group, 1)
        n_rows = int(rows_d.shape[0])
        ws_bytes = pkv.rows_workspace_bytes(desc, n_rows)
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        log(f"shared-prefix units: {n_rows} units for {S} sequences, "
            f"{int((rows_d[:, 2] > 1).sum())} with shared blocks, "
            f"{int(rows_d[:, 3].sum())} read again by other units")
        reread = reread and cached_loads
    elif shared and cached_loads:
        impl |= pkv.IMPL_SHARED_BLOCKS
    kv_bytes = np.zeros(total)
    host_s = np.zeros(total)
    n_pairs = 0
    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    def flush(i):
        flush_buf.fill_(i % 251 + 1)

    def sampled(i):
        return i >= warmup + steps or (i - warmup) % event_every == 0

    def step(i, all_events=False):
        nonlocal n_pairs
        h0 = time.perf_counter()
        e = ev[i]
        if all_events:
            e[0].record(stream)
        _, pairs = batch.append(k_new, v_new)      # block manager, copies, write + tables
        if all_events:
            e[4].record(stream)
        n_pairs += len(pairs)
        kv_bytes[i] = float(batch.host_lens.sum()) * bytes_per_token
        if sampled(i):
            pkv.time_next_decode(e[1], e[2])       # the decode kernel's own start and end
        if use_rows:
            pkv.paged_attn_decode_rows(q, cache.k_pool, cache.v_pool, batch.tables, batch.lens,
                                       wl.scale, out, desc, max_ctx, partition_size, rows_d,
                                       seq_rows_d, workspace=workspace, phases=1,
                                       shared_blocks=reread)
        else:
            pkv.paged_attn_partials(q, cache.k_pool, cache.v_pool, batch.tables, batch.lens,
                                    wl.scale, out, desc, max_ctx, partition_size, workspace, impl)
        if use_rows:
            pkv.paged_attn_decode_rows(q, cache.k_pool, cache.v_pool, batch.tables, batch.lens,
                                       wl.scale, out, desc, max_ctx, partition_size, rows_d,
                                       seq_rows_d, workspace=workspace, phases=2,
                                       shared_blocks=reread)
        else:
            pkv.paged_attn_merge(out, batch.lens, wl.num_kv_heads, max_ctx, partition_size,
                                 workspace)
        if all_events:
            e[3].record(stream)
        host_s[i] = time.perf_counter() - h0

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()                      # no collector pauses inside the timed steps
    t0 = time.perf_counter()
    for i in range(warmup, warmup + steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(warmup + steps, warmup + steps + DIAG_STEPS):
        step(i, all_events=True)
    for i in range(warmup + steps + DIAG_STEPS, total):
        flush(i)
        step(i, all_events=True)
    torch.cuda.synchronize()
    gc.enable()
    timed = range(warmup, warmup + steps)
    diag = range(warmup + steps, warmup + steps + DIAG_STEPS)
    flushed = range(warmup + steps + DIAG_STEPS, total)
    timed_ev = [i for i in timed if sampled(i)]
    t_attn = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in timed_ev]) * 1e-3
    kv_attn = kv_bytes[timed_ev]
    t_write = np.array([ev[i][0].elapsed_time(ev[i][4]) for i in diag]) * 1e-3
    t_merge = np.array([ev[i][2].elapsed_time(ev[i][3]) for i in diag]) * 1e-3
    t_attn_diag = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in diag]) * 1e-3
    t_attn_flush = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in flushed]) * 1e-3
    t_merge_flush = np.array([ev[i][2].elapsed_time(ev[i][3]) for i in flushed]) * 1e-3
    kv_flush = kv_bytes[list(flushed)]
    kvb = kv_bytes[warmup:warmup + steps]
    assert torch.isfinite(out.float()).all(), "non-finite decode output"
    # the device tables the steps kept up to date equal the block manager's
    t_host, l_host = cache.bm.block_tables(seqs, max_blocks)
    assert np.array_equal(batch.tables.cpu().numpy(), t_host), "device block tables diverged"
    assert np.array_equal(batch.lens.cpu().numpy(), l_host), "device context lengths diverged"
    # bytes of distinct blocks (a block shared by several sequences counted once), last step
    tables, lens = cache.bm.block_tables(seqs, max_blocks)
    fill = {}
    for row, n in zip(tables, lens):
        nb = -(-int(n) // B)
        for j in range(nb):
            b = int(row[j])
            fill[b] = max(fill.get(b, 0), min(B, int(n) - j * B))
    unique_bytes = float(sum(fill.values())) * bytes_per_token
    cache_stats = cache.bm.cache_stats() if wl.prefix_caching else None
    return dict(wall=wall, kv_bytes=kvb, kv_attn=kv_attn, t_write=t_write, t_attn=t_attn,
                t_merge=t_merge,
                cache_stats=cache_stats,
                t_attn_diag=t_attn_diag, host_s=host_s[warmup:warmup + steps],
                t_attn_flush=t_attn_flush, t_merge_flush=t_merge_flush, kv_flush=kv_flush,
                max_ctx=max_ctx, ws_bytes=ws_bytes, n_pairs=n_pairs, shared=shared,
                rows=use_rows, rows_cached=use_rows and reread,
                cached_loads=bool(shared and cached_loads),
                unique_ratio=unique_bytes / float(kvb[-1]))


def cpu_baseline(wl, seconds: float, seconds_one: float = 5.0):
    """The oracle, as it stands, on a bounded sample of the workload's sequences: with all of
    its BLAS threads, and (a smaller sample) with one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import allocator as oalloc
    from oracle import attention as oattn
    from oracle import cache as ocache
    from oracle import codec

    k_scale, v_scale = wl.kv_scales()
    q = wl.q_input()
    q64 = codec.bf16_to_f64(q) if wl.in_dtype == "bf16" else q.astype(np.float64)
    # per setting: [wall seconds, KV bytes, sequences]
    acc = {"all": [0.0, 0.0, 0], "one": [0.0, 0.0, 0]}
    budget = {"all": seconds, "one": seconds_one}

    def timed(i, kp, vp, tables, lens, key):
        t = time.perf_counter()
        oattn.paged_decode(q64[i:i + 1], kp, vp, tables, lens, wl.scale, wl.kv_dtype,
                           k_scale, v_scale)
        a_ = acc[key]
        a_[0] += time.perf_counter() - t
        a_[1] += int(wl.ctx_lens[i]) * wl.kv_bytes_per_token()
        a_[2] += 1

    for i in range(wl.num_seqs):
        if all(acc[k][0] >= budget[k] for k in acc):
            break
        ctx = int(wl.ctx_lens[i])
        nb = -(-ctx // wl.block_size)
        a = oalloc.BlockAllocator(nb, wl.block_size)
        a.add_seq(0, ctx)
        kp, vp = ocache.new_pools(nb, wl.num_kv_heads, wl.block_size, wl.head_dim, wl.kv_dtype)
        k, v = wl.seq_kv_input(i)
        ocache.reshape_and_cache(kp, vp, k, v, a.slots(0, 0, ctx), wl.in_dtype, wl.kv_dtype,
                                 k_scale, v_scale)
        tables, lens = a.block_tables([0], nb)
        if acc["all"][0] < budget["all"]:
            timed(i, kp, vp, tables, lens, "all")
        if acc["one"][0] < budget["one"]:
            with threadpool_limits(limits=1):
                timed(i, kp, vp, tables, lens, "one")
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    try:
        nproc = int(subprocess.run(["nproc"], capture_output=True, text=True).stdout.strip())
    except (OSError, ValueError):
        nproc = None
    host = {"nproc": nproc, "sched_getaffinity": len(os.sched_getaffinity(0)),
            "os_cpu_count": os.cpu_count()}

    def desc(key, nthreads):
        wall, nbytes, n = acc[key]
        return (f"first {n} of {wl.num_seqs} sequences of {wl.name} "
                f"({int(sum(wl.ctx_lens[:n]))} cached tokens), decode attention only, "
                f"{wall:.1f} s wall, numpy float64 with {nthreads} BLAS thread(s)")

    wall, nbytes, n = acc["all"]
    wall1, nbytes1, n1 = acc["one"]
    return {
        "value": nbytes / wall / 1e9, "unit": "GB/s",
        "tokens_per_s": n / wall, "cores": int(threads), "kind": "oracle",
        "sample": desc("all", threads), "host_cores": host,
        "one_thread": {"value": nbytes1 / wall1 / 1e9, "unit": "GB/s",
                       "tokens_per_s": n1 / wall1, "cores": 1, "sample": desc("one", 1)},
    }


def read_reference(tile_bytes: int, same_bytes: int, total_bytes: int = READ_REF_BYTES,
                   reps: int = 5):
    """The library's plain read probe over a buffer far larger than the last-level cache:
    a sequential stream, and tiles of the workload's (block, KV head) tile size read in a
    random order (as the decode reads its blocks).  Best of a few launch widths, median of
    ``reps`` launches each (GB/s).  ``same_bytes``: random tiles adding up to the decode's
    own KV bytes per launch, each launch on tiles no earlier launch of that width read
    (while the buffer holds enough) and after the same 512 MB write as the flushed decode
    steps, so that a short launch is set against a read of its own size from HBM, ramp and
    tail included."""
    import torch

    import paged_kv_cache_104_amd as pkv

    buf = torch.empty(total_bytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    n = total_bytes // tile_bytes
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(0)).to("cuda")
    sink = torch.empty(8192 * 64, dtype=torch.int32, device="cuda")
    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    res = {}
    for name, ids in (("sequential", None), ("random_tiles", perm)):
        best = 0.0
        for wgs in (1024, 2048, 4096, 8192):
            ts = []
            for r in range(reps + 1):
                ev[0].record()
                pkv.read_probe(buf, tile_bytes, ids, n, sink, wgs)
                ev[1].record()
                torch.cuda.synchronize()
                if r:
                    ts.append(ev[0].elapsed_time(ev[1]) * 1e-3)
            best = max(best, n * tile_bytes / float(np.median(ts)) / 1e9)
        res[name] = round(best, 1)
    m = max(1, min(n, -(-same_bytes // tile_bytes)))
    best_t = None
    for wgs in (1024, 2048, 4096, 8192):
        ts = []
        for r in range(reps + 1):
            lo = (r * m) % max(1, n - m + 1)
            ids = perm[lo:lo + m]
            flush_buf.fill_(r + 1)
            ev[0].record()
            pkv.read_probe(buf, tile_bytes, ids, m, sink, wgs)
            ev[1].record()
            torch.cuda.synchronize()
            if r:
                ts.append(ev[0].elapsed_time(ev[1]) * 1e-3)
        t = float(np.median(ts))
        best_t = t if best_t is None else min(best_t, t)
    res["same_bytes"] = {"bytes": int(m * tile_bytes), "us": round(best_t * 1e6, 2),
                         "GBps": round(m * tile_bytes / best_t / 1e9, 1)}
    # the same bytes as one sequential stream, after the same write: no tile ids to wait
    # for, the upper bound for a read of this size
    best_t = None
    for wgs in (1024, 2048, 4096, 8192):
        ts = []
        for r in range(reps + 1):
            flush_buf.fill_(r + 1)
            ev[0].record()
            pkv.read_probe(buf, tile_bytes, None, m, sink, wgs)
            ev[1].record()
            torch.cuda.synchronize()
            if r:
                ts.append(ev[0].elapsed_time(ev[1]) * 1e-3)
        t = float(np.median(ts))
        best_t = t if best_t is None else min(best_t, t)
    res["same_bytes_sequential"] = {"bytes": int(m * tile_bytes), "us": round(best_t * 1e6, 2),
                                    "GBps": round(m * tile_bytes / best_t / 1e9, 1)}
    del buf, perm, sink, flush_buf
    return res


def copy_calibration(n_bytes: int, reps: int) -> None:
    """A plain device copy of known size, for scaling HBM counters (rocprofv3 --pmc)."""
    import torch

    src = torch.empty(n_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n_bytes, "reps": reps}))


def swap_sweep(total_bytes: int, reps: int, methods=("kernel", "dma")) -> None:
    """Host-link rate of swapping (K+V bytes moved / time) against block size, for the
    one-kernel copy and for one copy-engine transfer per block.  Device blocks are a
    random permutation and host blocks consecutive, as the block manager hands them out."""
    import torch

    import paged_kv_cache_104_amd as pkv

    rows = []
    for D in (64, 128):
        for B in (8, 16, 32):
            per_block = 2 * 8 * B * D * 2                  # K + V, 8 KV heads, bf16
            n = total_bytes // per_block
            desc = pkv.cache_desc(n, 8, B, D, "bf16")
            dk, dv = pkv.alloc_pools(desc, poison=False)
            hk, hv = pkv.alloc_host_pools(desc, n)
            perm = np.random.default_rng(B * D).permutation(n)
            out = np.stack([perm, np.arange(n)], 1)
            back = np.stack([np.arange(n), perm], 1)
            for method in methods:
                res = {}
                for name, args, pairs in (("out", (dk, dv, hk, hv), out), ("in", (hk, hv, dk, dv), back)):
                    pkv.swap_blocks(*args, pairs, desc, method)           # warm-up
                    torch.cuda.synchronize()
                    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                    ts = []
                    for _ in range(reps):
                        ev[0].record()
                        pkv.swap_blocks(*args, pairs, desc, method)
                        ev[1].record()
                        torch.cuda.synchronize()
                        ts.append(ev[0].elapsed_time(ev[1]) * 1e-3)
                    res[name] = round(n * per_block / float(np.median(ts)) / 1e9, 2)
                rows.append({"head_dim": D, "block_size": B, "block_bytes": per_block // 2,
                             "blocks": int(n), "method": method, "out_GBps": res["out"],
                             "in_GBps": res["in"]})
                log(f"swap D={D} B={B} {method}: out {res['out']} GB/s, in {res['in']} GB/s")
            del dk, dv, hk, hv
    print(json.dumps({"swap_sweep": rows, "bytes_per_direction": total_bytes, "reps": reps}))


def cache_ops_bench(tokens: int, reps: int) -> None:
    """The cache write and the copy-on-write block copy at scale, against the HBM roofline:
    ``tokens`` new tokens (a prefill's worth, 8 KV heads, D = 128, 16-token blocks) written
    through ``pkv_reshape_and_cache`` into whole blocks placed at random in the pool (bf16,
    and fp8 encoded from bf16), and ``pkv_copy_blocks`` over as many blocks' worth of random
    (src, dst) pairs.  Bytes are the algorithmic ones, read plus written; a plain device copy
    of the same bytes (torch ``copy_``) is timed beside them.  Then a decode step's write for
    batches of 1024 to 16384 sequences (each token alone in a block), in one call and in calls
    of 500 tokens.  Median of ``reps`` launches."""
    import torch

    import paged_kv_cache_104_amd as pkv

    H, D, B = 8, 128, 16
    n_blk = tokens // B
    rng = np.random.default_rng(11)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]) * 1e-3)
        return float(np.median(ts))

    rows = []
    for kv in ("bf16", "fp8"):
        scale = 0.05 if kv == "fp8" else 1.0
        desc = pkv.cache_desc(2 * n_blk + 1, H, B, D, kv, scale, scale)
        kp, vp = pkv.alloc_pools(desc, poison=False)
        elem = 2 if kv == "bf16" else 1
        # reshape_and_cache: one prompt in whole blocks at random places, a batch of prompts
        # of random lengths laid end to end (each in its own random blocks, so most chunks of
        # B tokens straddle two blocks), and distinct random slots (about half the rows of
        # the blocks they touch)
        k = torch.randn(tokens, H, D, device="cuda").to(torch.bfloat16)
        v = torch.randn(tokens, H, D, device="cuda").to(torch.bfloat16)
        blocks = rng.permutation(2 * n_blk + 1)
        t = np.arange(tokens)
        lens = []
        while sum(lens) < tokens:
            lens.append(int(min(rng.integers(1, 2001), tokens - sum(lens))))
        batch, used = [], 0
        for n in lens:
            p = np.arange(n)
            batch.append(blocks[used + p // B] * B + p % B)
            used += -(-n // B)
        scattered = rng.permutation(len(blocks) * B)[:tokens]
        for layout, sl in (("one prompt", blocks[t // B] * B + t % B),
                           (f"{len(lens)} prompts", np.concatenate(batch)),
                           ("scattered slots", scattered)):
            slots = torch.from_numpy(sl.astype(np.int64)).cuda()
            sec = timed(lambda: pkv.reshape_and_cache(k, v, slots, kp, vp, desc))
            nbytes = tokens * H * D * (2 + elem) * 2
            rows.append({"op": "reshape_and_cache", "kv_dtype": kv, "tokens": tokens,
                         "layout": layout, "bytes": nbytes, "us": round(sec * 1e6, 1),
                         "GBps": round(nbytes / sec / 1e9, 1),
                         "frac_of_hbm_peak": round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4)})
        # copy_blocks: n_blk pairs, sources and destinations disjoint, random
        perm = rng.permutation(2 * n_blk)
        pairs = torch.from_numpy(np.stack([perm[:n_blk], perm[n_blk:]], 1).astype(np.int64)).cuda()
        sec = timed(lambda: pkv.copy_blocks(kp, vp, pairs, desc))
        nbytes = n_blk * H * B * D * elem * 2 * 2
        rows.append({"op": "copy_blocks", "kv_dtype": kv, "pairs": n_blk,
                     "block_bytes": H * B * D * elem, "bytes": nbytes, "us": round(sec * 1e6, 1),
                     "GBps": round(nbytes / sec / 1e9, 1),
                     "frac_of_hbm_peak": round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4)})
        del kp, vp, k, v
    # a decode step's write for a large batch: every token alone at a random row of a block
    # of its own; one call (the large-write kernel, its rows split over several workgroups
    # per chunk) against calls of 500 tokens (the per-token kernel)
    for kv in ("bf16", "fp8"):
        scale = 0.05 if kv == "fp8" else 1.0
        elem = 2 if kv == "bf16" else 1
        for T in (1024, 4096, 16384):
            desc = pkv.cache_desc(T + 1, H, B, D, kv, scale, scale)
            kp, vp = pkv.alloc_pools(desc, poison=False)
            k = torch.randn(T, H, D, device="cuda").to(torch.bfloat16)
            v = torch.randn(T, H, D, device="cuda").to(torch.bfloat16)
            sl = rng.permutation(T + 1)[:T] * B + rng.integers(0, B, T)
            slots = torch.from_numpy(sl.astype(np.int64)).cuda()

            def calls():
                for a in range(0, T, 500):
                    pkv.reshape_and_cache(k[a:a + 500], v[a:a + 500], slots[a:a + 500], kp, vp,
                                          desc)
            one = timed(lambda: pkv.reshape_and_cache(k, v, slots, kp, vp, desc))
            split = timed(calls)
            nbytes = T * H * D * (2 + elem) * 2
            rows.append({"op": "reshape_and_cache", "kv_dtype": kv, "tokens": T,
                         "layout": "decode batch (one token per block)", "bytes": nbytes,
                         "us": round(one * 1e6, 1), "us_calls_of_500": round(split * 1e6, 1),
                         "GBps": round(nbytes / one / 1e9, 1)})
            del kp, vp, k, v
    # a plain device copy of the bf16 write's bytes (half read, half written)
    src = torch.empty(tokens * H * D * 2 * 2, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    sec = timed(lambda: dst.copy_(src))
    nbytes = 2 * src.numel()
    rows.append({"op": "torch_copy", "bytes": nbytes, "us": round(sec * 1e6, 1),
                 "GBps": round(nbytes / sec / 1e9, 1),
                 "frac_of_hbm_peak": round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4)})
    for r in rows:
        log(json.dumps(r))
    print(json.dumps({"cache_ops": rows, "reps": reps}), flush=True)


def quest_bench(wl, budget: int, steps: int, warmup: int, partition_size: int, impl: int,
                workers: int) -> None:
    """QUEST decode against the dense decode on the same decode steps.

    Each step appends one token per sequence (block manager, copies, the write and
    the table update, then the metadata of every row's last block); the QUEST
    decode (scoring, selection, decode kernel, merge) and the dense decode then run
    on the same state, each between a pair of HIP events.  Bytes QUEST reads: the
    metadata of every block of every context (2 rows of head_dim per block and KV
    head) plus the K and V of the chosen tokens."""
    import torch

    import paged_kv_cache_104_amd as pkv
    from paged_kv_cache_104_amd.engine import DecodeBatch

    cache, desc, seqs, q, k_new, v_new = build_gpu_state(wl, workers)
    S, B, H, D = len(seqs), wl.block_size, wl.num_kv_heads, wl.head_dim
    total = warmup + steps
    max_ctx = wl.max_context_len + total
    max_blocks = -(-max_ctx // B)
    batch = DecodeBatch(cache, seqs, max_blocks)
    cache.enable_quest(seqs)
    elt = {"bf16": 2, "fp8": 1, "f32": 4}[wl.kv_dtype]
    qws = torch.empty(pkv.quest_workspace_bytes(desc, S, wl.num_q_heads, max_blocks, max_ctx,
                                                partition_size, budget),
                      dtype=torch.uint8, device="cuda")
    dws = torch.empty(max(16, pkv.decode_workspace_bytes(S, wl.num_q_heads, D, max_ctx,
                                                         partition_size)),
                      dtype=torch.uint8, device="cuda")
    out_q, out_d = torch.empty_like(q), torch.empty_like(q)
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(total)]
    for e in [x for row in ev for x in row]:
        e.record(stream)
    torch.cuda.synchronize()
    meta_bytes, kv_bytes = np.zeros(total), np.zeros(total)
    for i in range(total):
        batch.append(k_new, v_new)
        lens = batch.host_lens
        meta_bytes[i] = float((-(-lens // B)).sum()) * H * 2 * D * elt
        kv_bytes[i] = float(lens.sum()) * wl.kv_bytes_per_token()
        e = ev[i]
        e[0].record(stream)
        pkv.quest_decode(q, cache.k_pool, cache.v_pool, cache.quest_meta, desc, batch.tables,
                         batch.lens, wl.scale, out_q, max_ctx, budget, partition_size, qws, impl)
        e[1].record(stream)
        pkv.paged_attn_decode(q, cache.k_pool, cache.v_pool, batch.tables, batch.lens, wl.scale,
                              out_d, desc, max_ctx, partition_size, dws, impl)
        e[2].record(stream)
    torch.cuda.synchronize()
    # tokens actually chosen in the last step (the selection is deterministic)
    _, sel_l = pkv.quest_select(q, cache.quest_meta, desc, batch.tables, batch.lens, max_ctx,
                                budget)
    chosen = float(sel_l.sum().item()) * 2 * D * elt
    timed = range(warmup, total)
    tq = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in timed]) * 1e-3
    td = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in timed]) * 1e-3
    assert torch.isfinite(out_q.float()).all(), "non-finite QUEST output"
    last_bytes = meta_bytes[-1] + chosen
    rate = last_bytes / float(tq[-5:].mean()) / 1e9
    print(json.dumps({"quest": {
        "workload": wl.name, "budget_blocks": budget, "budget_tokens": budget * B,
        "steps": steps, "warmup": warmup, "partition_size": partition_size,
        "quest_ms": round(float(tq.mean()) * 1e3, 4),
        "dense_ms": round(float(td.mean()) * 1e3, 4),
        "speedup_vs_dense": round(float(td.mean() / tq.mean()), 3),
        "last_step": {"metadata_bytes": int(meta_bytes[-1]), "chosen_kv_bytes": int(chosen),
                      "dense_kv_bytes": int(kv_bytes[-1]),
                      "kept_fraction": round(chosen / kv_bytes[-1], 4)},
        "achieved_GBps": round(rate, 1), "frac_of_hbm_peak": round(rate / HBM_PEAK_GBS, 4),
        "dense_GBps": round(float(kv_bytes[-1]) / float(td[-5:].mean()) / 1e9, 1),
    }}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--impl", type=int, default=0, help="0 auto, 1 vector, 2 mfma")
    ap.add_argument("--workers", type=int, default=16)
    ap.add_argument("--event-every", type=int, default=EVENT_EVERY,
                    help="time the decode kernel of every n-th timed step")
    ap.add_argument("--rows", choices=("auto", "off"), default="auto",
                    help="shared-prefix (unit) decode for batches whose sequences share blocks "
                         "(auto), or the per-sequence decode (off)")
    ap.add_argument("--cached-loads", action="store_true",
                    help="batches that share blocks: read K/V with ordinary loads (the "
                         "shared-blocks hint) instead of streaming them")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-reference", action="store_true",
                    help="skip the plain read probe (sequential and random tiles)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--swap-sweep", type=int, default=0, metavar="BYTES",
                    help="measure swapping rates moving BYTES of K+V each way, then exit")
    ap.add_argument("--swap-methods", default="kernel,dma")
    ap.add_argument("--cache-ops", type=int, default=0, metavar="TOKENS",
                    help="time the cache write and the block copy at scale (TOKENS new tokens "
                         "and as many blocks' worth of copies), then exit")
    ap.add_argument("--quest-budget", type=int, default=0, metavar="BLOCKS",
                    help="time the QUEST decode with this budget against the dense decode "
                         "on --config, then exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this paged-KV build has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 10)
        return 0
    if args.swap_sweep:
        swap_sweep(args.swap_sweep, 5, tuple(args.swap_methods.split(",")))
        return 0
    if args.cache_ops:
        cache_ops_bench(args.cache_ops, 10)
        return 0

    import torch

    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = workloads.get(args.config)
    if args.quest_budget:
        ps = wl.partition_size if args.partition_size is None else args.partition_size
        quest_bench(wl, args.quest_budget, args.steps, args.warmup, ps, args.impl, args.workers)
        return 0
    wl.cache_sequences = True          # keep the drawn inputs for the oracle's sample
    ps = wl.partition_size if args.partition_size is None else args.partition_size
    r = run_gpu(wl, args.steps, args.warmup, ps, args.impl, args.workers,
                event_every=max(1, args.event_every), rows_mode=args.rows,
                cached_loads=args.cached_loads)
    wall = r["wall"]
    total_bytes = float(r["kv_bytes"].sum())
    value = total_bytes / wall / 1e9
    attn_gbs = float((r["kv_attn"] / r["t_attn"]).mean()) / 1e9
    mean_ctx = float(r["kv_bytes"].mean()) / wl.kv_bytes_per_token() / wl.num_seqs
    traffic = measured_traffic(args.config)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.kv_dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name, "num_seqs": wl.num_seqs, "num_q_heads": wl.num_q_heads,
            "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
            "block_size": wl.block_size, "kv_dtype": wl.kv_dtype,
            "mean_context": round(mean_ctx, 1), "partition_size": ps,
            "kv_loads": ("shared-prefix units, cached loads" if r["rows_cached"] else
                         "shared-prefix units" if r["rows"] else
                         "cached (shared blocks)" if r["cached_loads"] else "streaming"),
            "prefix_cache": r["cache_stats"],
            "description": wl.description,
        },
        "decode_tokens_per_s": round(wl.num_seqs * args.steps / wall, 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "kernel_ms": {
            "decode_attention": round(float(r["t_attn"].mean()) * 1e3, 4),
            "reshape_and_cache+copy_blocks": round(float(r["t_write"].mean()) * 1e3, 4),
            "merge": round(float(r["t_merge"].mean()) * 1e3, 4),
            "decode_attention_diag": round(float(r["t_attn_diag"].mean()) * 1e3, 4),
            "decode_attention_p10_p50_p90": [round(float(np.percentile(r["t_attn"], p)) * 1e3, 4)
                                             for p in (10, 50, 90)],
            "decode_attention_flushed": round(float(r["t_attn_flush"].mean()) * 1e3, 4),
            "decode_attention_flushed_p10_p50_p90": [
                round(float(np.percentile(r["t_attn_flush"], p)) * 1e3, 4) for p in (10, 50, 90)],
            "merge_flushed": round(float(r["t_merge_flush"].mean()) * 1e3, 4),
        },
        "host_ms_per_step": round(float(r["host_s"].mean()) * 1e3, 4),
        "roofline": {
            "kernel": DOMINANT_KERNEL,
            "bound": "hbm",
            "achieved": round(attn_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(r["kv_attn"].mean()),
            "timed_launches": int(len(r["t_attn"])),
        },
    }
    flush_gbs = float((r["kv_flush"] / r["t_attn_flush"]).mean()) / 1e9
    result["roofline"]["achieved_flushed"] = round(flush_gbs, 1)
    # the attention kernels together: the decode and the merge of split contexts
    merged_gbs = float(r["kv_attn"].mean()) / (float(r["t_attn"].mean()) + float(r["t_merge"].mean())) / 1e9
    if r["shared"]:
        # blocks read by several sequences: the HBM roofline is judged on distinct bytes
        ub = attn_gbs * r["unique_ratio"]
        result["unique_kv_bytes_ratio"] = round(r["unique_ratio"], 4)
        result["roofline"]["achieved_logical"] = result["roofline"]["achieved"]
        result["roofline"]["achieved"] = round(ub, 1)
        result["roofline"]["frac"] = round(ub / HBM_PEAK_GBS, 4)
        result["roofline"]["algorithmic_bytes_per_launch"] = int(r["kv_attn"].mean()
                                                                 * r["unique_ratio"])
        result["roofline"]["achieved_flushed"] = round(flush_gbs * r["unique_ratio"], 1)
        merged_gbs *= r["unique_ratio"]
    result["roofline"]["frac_flushed"] = round(result["roofline"]["achieved_flushed"]
                                               / HBM_PEAK_GBS, 4)
    result["roofline"]["achieved_decode_and_merge"] = round(merged_gbs, 1)
    result["roofline"]["frac_decode_and_merge"] = round(merged_gbs / HBM_PEAK_GBS, 4)
    if not args.no_read_reference:
        log("timing the read probe")
        tile = wl.block_size * wl.head_dim * {"f32": 4, "bf16": 2, "fp8": 1}[wl.kv_dtype]
        ref = read_reference(tile, result["roofline"]["algorithmic_bytes_per_launch"])
        result["roofline"]["read_probe_GBps"] = {"tile_bytes": tile, **ref}
        result["roofline"]["stream_frac"] = round(result["roofline"]["achieved"]
                                                  / ref["sequential"], 4)
        # the flushed decode against a probe launch reading as many bytes from HBM
        result["roofline"]["same_bytes_frac"] = round(
            result["roofline"]["achieved_flushed"] / ref["same_bytes"]["GBps"], 4)
        result["roofline"]["same_bytes_sequential_frac"] = round(
            result["roofline"]["achieved_flushed"] / ref["same_bytes_sequential"]["GBps"], 4)
    if not args.no_cpu_baseline:
        log("timing the oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
