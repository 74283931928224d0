"""Seeded synthetic workloads for paged decode attention.

This module only *draws* inputs: random context lengths, random query/key/value
values, the initial order of the free-block list and the script of allocator
operations (add / fork / extend / append_batch / free) that a serving engine
would issue.  It holds none of the method's arithmetic: block tables, slots,
cache writes, copy-on-write pairs and attention are computed independently by
the CPU oracle (``oracle/``) and by the HIP library
(``paged_kv_cache_104_amd``) from the same draws.

The only block arithmetic here is the sizing rule "a sequence of n tokens holds
ceil(n / B) blocks", used to size pools (1.25x the blocks the live sequences
need) and to decide when the churn script of the fragmented-pool workload stops
allocating.  It never produces a block id.

Value conversions done here are input preparation by library routines: fp32
draws are rounded to bfloat16 with torch's CPU cast (round to nearest even),
and kept as raw 16-bit patterns so both sides read identical bits.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, Dict, List, Optional, Tuple

import numpy as np

# tags that separate the random streams of one seed
_TAG_Q = 0x51
_TAG_KV = 0x4B56
_TAG_META = 0x4D45


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def blocks_for(n_tokens: int, block_size: int) -> int:
    """Pool-sizing rule: blocks held by a sequence of ``n_tokens`` tokens."""
    return -(-int(n_tokens) // int(block_size))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (torch CPU cast, nearest-even); raw uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_as_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bits to float32 (exact; used only for the fp8 scale choice)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


Op = Tuple  # ('add', seq, n) | ('fork', parent, child) | ('extend', seq, n)
#             | ('append_batch', [seqs]) | ('free', seq)


@dataclasses.dataclass
class Workload:
    """One seeded paged-decode workload (one attention layer, one decode step)."""

    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    kv_dtype: str              # 'f32' | 'bf16' | 'fp8'  (pool storage)
    in_dtype: str              # 'f32' | 'bf16'  (k/v handed to reshape_and_cache; also q/out)
    scale: float
    partition_size: int
    free_order: np.ndarray     # int32: initial free list, head first
    setup_ops: List[Op]        # allocator script run before the decode step
    decode_seqs: np.ndarray    # int64 [S]: batch order of the decode step (ascending ids)
    ctx_lens: np.ndarray       # int64 [S]: context incl. the token decoded this step
    # logical context of a sequence -> list of (stream_id, first_row, n_rows) segments
    _segments: Callable[[int], List[Tuple[int, int, int]]]
    description: str = ""
    _scales: Optional[Tuple[float, float]] = None
    _cache: Dict[int, Tuple[np.ndarray, np.ndarray]] = dataclasses.field(default_factory=dict)
    cache_sequences: bool = False
    # sequences outside the decode batch whose tokens are written (and may be reused
    # through prefix caching after they end): seq id -> segments, as _segments
    extra_segments: Dict[int, List[Tuple[int, int, int]]] = dataclasses.field(default_factory=dict)
    prefix_caching: bool = False

    # ---- shapes --------------------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(len(self.decode_seqs))

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_context_len(self) -> int:
        return int(self.ctx_lens.max()) if len(self.ctx_lens) else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return blocks_for(self.max_context_len, self.block_size)

    def kv_bytes_per_token(self) -> int:
        """Bytes of K plus V that one cached token occupies in one layer."""
        elem = {"f32": 4, "bf16": 2, "fp8": 1}[self.kv_dtype]
        return 2 * self.num_kv_heads * self.head_dim * elem

    # ---- draws ---------------------------------------------------------------
    def q_f32(self) -> np.ndarray:
        """Query draws, fp32 N(0,1), [S, Hq, D]."""
        return _rng(self.seed, _TAG_Q, 0).standard_normal(
            (self.num_seqs, self.num_q_heads, self.head_dim), dtype=np.float32)

    def q_input(self) -> np.ndarray:
        """Query in its input format: float32, or raw bfloat16 bits (uint16)."""
        q = self.q_f32()
        return q if self.in_dtype == "f32" else to_bf16_bits(q)

    def _stream_rows(self, stream: int, n: int) -> Tuple[np.ndarray, np.ndarray]:
        x = _rng(self.seed, _TAG_KV, stream).standard_normal(
            (n, 2, self.num_kv_heads, self.head_dim), dtype=np.float32)
        return x[:, 0], x[:, 1]

    def seq_kv_f32(self, i: int) -> Tuple[np.ndarray, np.ndarray]:
        """fp32 draws of the whole logical context of batch entry ``i``: K, V [ctx, Hkv, D]."""
        ks, vs = [], []
        for stream, first, n in self._segments(i):
            k, v = self._stream_rows(stream, first + n)
            ks.append(k[first:first + n])
            vs.append(v[first:first + n])
        return np.concatenate(ks), np.concatenate(vs)

    def _segments_kv(self, segs) -> Tuple[np.ndarray, np.ndarray]:
        ks, vs = [], []
        for stream, first, n in segs:
            k, v = self._stream_rows(stream, first + n)
            ks.append(k[first:first + n])
            vs.append(v[first:first + n])
        return np.concatenate(ks), np.concatenate(vs)

    def seq_kv_input(self, i: int) -> Tuple[np.ndarray, np.ndarray]:
        """K, V of batch entry ``i`` in the input format of reshape_and_cache."""
        if i in self._cache:
            return self._cache[i]
        k, v = self.seq_kv_f32(i)
        if self.in_dtype == "bf16":
            k, v = to_bf16_bits(k), to_bf16_bits(v)
        if self.cache_sequences:
            self._cache[i] = (k, v)
        return k, v

    def extra_kv_input(self, seq: int) -> Tuple[np.ndarray, np.ndarray]:
        """K, V (input format) of a sequence outside the decode batch."""
        k, v = self._segments_kv(self.extra_segments[int(seq)])
        if self.in_dtype == "bf16":
            k, v = to_bf16_bits(k), to_bf16_bits(v)
        return k, v

    def data_seqs(self) -> set:
        """Sequences whose tokens are written: the decode batch and the extra sequences."""
        return {int(s) for s in self.decode_seqs} | set(self.extra_segments)

    def kv_scales(self) -> Tuple[float, float]:
        """fp8 per-tensor scales: amax(|K|)/448 and amax(|V|)/448 over all inputs, in fp32.

        For non-fp8 pools both are 1.0.
        """
        if self.kv_dtype != "fp8":
            return 1.0, 1.0
        if self._scales is None:
            ka = va = np.float32(0)
            for i in range(self.num_seqs):
                k, v = self.seq_kv_input(i)
                if self.in_dtype == "bf16":
                    k, v = bf16_bits_as_f32(k), bf16_bits_as_f32(v)
                ka = max(ka, np.abs(k).max())
                va = max(va, np.abs(v).max())
            self._scales = (float(np.float32(ka) / np.float32(448.0)),
                            float(np.float32(va) / np.float32(448.0)))
        return self._scales

    def seq_index(self) -> Dict[int, int]:
        return {int(s): i for i, s in enumerate(self.decode_seqs)}


# --------------------------------------------------------------------------- configs

def _simple_segments(ids: np.ndarray, ctx: np.ndarray):
    def seg(i: int):
        return [(int(ids[i]), 0, int(ctx[i]))]
    return seg


def _plain(name, seed, S, Hq, Hkv, D, B, ctx, kv_dtype, in_dtype, partition_size,
           pool_blocks=None, description="", free_order=None, churn_ops=None):
    ctx = np.asarray(ctx, dtype=np.int64)
    need = sum(blocks_for(c, B) for c in ctx)
    N = pool_blocks if pool_blocks is not None else int(math.ceil(1.25 * need))
    meta = _rng(seed, _TAG_META, 1)
    if free_order is None:
        free_order = meta.permutation(N).astype(np.int32)
    ids = np.arange(S, dtype=np.int64)
    ops: List[Op] = list(churn_ops or [])
    ops += [("add", int(s), int(c) - 1) for s, c in zip(ids, ctx)]
    return Workload(
        name=name, seed=seed, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
        block_size=B, num_blocks=N, kv_dtype=kv_dtype, in_dtype=in_dtype,
        scale=1.0 / math.sqrt(D), partition_size=partition_size,
        free_order=np.asarray(free_order, dtype=np.int32), setup_ops=ops,
        decode_seqs=ids, ctx_lens=ctx, _segments=_simple_segments(ids, ctx),
        description=description)


def tiny_f32() -> Workload:
    """4 sequences, ctx {7,16,40,41}, 2 q / 2 KV heads, D=64, B=16, pool of 64 blocks, fp32."""
    return _plain("tiny-f32", 1, 4, 2, 2, 64, 16, [7, 16, 40, 41], "f32", "f32", 0,
                  pool_blocks=64,
                  description="tiny fp32 paged decode, ctx {7,16,40,41}, 2q/2kv heads, D=64")


def mha7b_bf16() -> Workload:
    """7B-like MHA layer: 64 seqs, 32/32 heads, D=128, ctx U[128,2048], bf16."""
    ctx = _rng(2, _TAG_META, 0).integers(128, 2048, size=64, endpoint=True)
    return _plain("7b-mha-bf16", 2, 64, 32, 32, 128, 16, ctx, "bf16", "bf16", 512,
                  description="7B-like MHA layer, bf16 KV, 64 seqs, ctx U[128,2048]")


def mha13b_bf16_churn() -> Workload:
    """13B-like MHA layer: 256 seqs, 40 heads, D=128, lognormal ctx, churned pool, bf16."""
    seed, S, B = 3, 256, 16
    rng = _rng(seed, _TAG_META, 0)

    def draw(n):
        x = np.exp(rng.normal(math.log(600.0), 0.8, size=n))
        return np.clip(np.rint(x), 16, 4096).astype(np.int64)

    ctx = draw(S)
    need = sum(blocks_for(c, B) for c in ctx)
    N = int(math.ceil(1.25 * need))
    # churn: 8 rounds of (allocate dummies until < 20% free, free a random half),
    # then free every dummy in random order; the pool starts as FIFO 0..N-1
    ops: List[Op] = []
    free = N
    live: List[Tuple[int, int]] = []
    next_id = 10_000_000
    for _ in range(8):
        while free >= 0.2 * N:
            n = int(draw(1)[0])
            nb = blocks_for(n, B)
            if nb > free:
                break
            ops.append(("add", next_id, n))
            live.append((next_id, nb))
            free -= nb
            next_id += 1
        order = rng.permutation(len(live))
        drop = set(order[: len(live) // 2].tolist())
        for j in order[: len(live) // 2]:
            ops.append(("free", live[j][0]))
            free += live[j][1]
        live = [x for j, x in enumerate(live) if j not in drop]
    for j in rng.permutation(len(live)):
        ops.append(("free", live[j][0]))
    return _plain("13b-mha-bf16-churn", seed, S, 40, 40, 128, B, ctx, "bf16", "bf16", 512,
                  pool_blocks=N, free_order=np.arange(N, dtype=np.int32), churn_ops=ops,
                  description="13B-like MHA layer, bf16 KV, 256 seqs, lognormal ctx "
                              "(median 600, sigma 0.8, clip [16,4096]), churned pool")


def gqa8b(kv_dtype: str = "fp8", block_size: int = 16) -> Workload:
    """8B-like GQA layer: 128 seqs, 32 q / 8 KV heads, D=128, ctx U[1024,8192].

    ``block_size`` other than 16 gives the block-size sweep's variants: the same
    contexts and the same drawn K/V, in a pool of the other block size.
    """
    ctx = _rng(4, _TAG_META, 0).integers(1024, 8192, size=128, endpoint=True)
    name = "8b-gqa-" + kv_dtype + ("" if block_size == 16 else f"-b{block_size}")
    w = _plain(name, 4, 128, 32, 8, 128, block_size, ctx, kv_dtype, "bf16", 1024,
               description=f"8B-like GQA layer, {kv_dtype} KV, 128 seqs, 32q/8kv, "
                           f"ctx U[1024,8192], {block_size}-token blocks")
    return w


def mqa_bf16() -> Workload:
    """Multi-query layer: 128 seqs, 16 q heads sharing one KV head, D=128, ctx U[1024,8192]."""
    ctx = _rng(4, _TAG_META, 0).integers(1024, 8192, size=128, endpoint=True)
    return _plain("mqa-16q-bf16", 7, 128, 16, 1, 128, 16, ctx, "bf16", "bf16", 0,
                  description="multi-query layer, bf16 KV, 128 seqs, 16 q heads / 1 KV head, "
                              "ctx U[1024,8192]")


def chat_prefix_cache_bf16() -> Workload:
    """Chat serving with prefix caching: 8 system prompts, 128 users on their second turn
    (the first turn ran, finished and was released earlier), 64 users on their first turn.

    Token ids decide what the block manager finds cached; the K/V draws follow the
    same structure (one random stream per system prompt, question and reply), so equal
    token prefixes have equal K/V, as a model would give.
    """
    seed, B = 8, 16
    rng = _rng(seed, _TAG_META, 0)
    vocab = 32000
    n_sys, users, fresh = 8, 128, 64
    sys_len = rng.integers(1000, 2000, size=n_sys, endpoint=True)
    sys_tok = [rng.integers(0, vocab, size=int(n)) for n in sys_len]
    q1_len = rng.integers(32, 256, size=users, endpoint=True)
    r1_len = rng.integers(32, 256, size=users, endpoint=True)
    q2_len = rng.integers(16, 128, size=users, endpoint=True)
    qf_len = rng.integers(32, 256, size=fresh, endpoint=True)
    tok = lambda n: rng.integers(0, vocab, size=int(n))
    q1 = [tok(n) for n in q1_len]
    r1 = [tok(n) for n in r1_len]
    q2 = [tok(n) for n in q2_len]
    qf = [tok(n) for n in qf_len]
    ops: List[Op] = []
    extra: Dict[int, List[Tuple[int, int, int]]] = {}
    for u in range(users):                               # first turns: ran and ended
        k = u % n_sys
        sid = 1_000_000 + u
        ops.append(("add_tokens", sid, np.concatenate([sys_tok[k], q1[u]])))
        ops.append(("extend_tokens", sid, r1[u]))
        ops.append(("free", sid))
        extra[sid] = [(20_000 + k, 0, int(sys_len[k])), (30_000 + u, 0, int(q1_len[u])),
                      (40_000 + u, 0, int(r1_len[u]))]
    segs: List[List[Tuple[int, int, int]]] = []
    ctx = []
    for u in range(users):                               # second turns: the decode batch
        k = u % n_sys
        prompt = np.concatenate([sys_tok[k], q1[u], r1[u], q2[u]])
        ops.append(("add_tokens", u, prompt))
        segs.append([(20_000 + k, 0, int(sys_len[k])), (30_000 + u, 0, int(q1_len[u])),
                     (40_000 + u, 0, int(r1_len[u])), (50_000 + u, 0, int(q2_len[u]) + 1)])
        ctx.append(len(prompt) + 1)
    for v in range(fresh):                               # new users
        k = (3 * v) % n_sys
        prompt = np.concatenate([sys_tok[k], qf[v]])
        ops.append(("add_tokens", users + v, prompt))
        segs.append([(20_000 + k, 0, int(sys_len[k])), (60_000 + v, 0, int(qf_len[v]) + 1)])
        ctx.append(len(prompt) + 1)
    ctx = np.asarray(ctx, dtype=np.int64)
    ids = np.arange(users + fresh, dtype=np.int64)
    N = int(math.ceil(1.25 * sum(blocks_for(c, B) for c in ctx)))
    free_order = _rng(seed, _TAG_META, 1).permutation(N).astype(np.int32)
    return Workload(
        name="chat-prefix-cache-bf16", seed=seed, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=B, num_blocks=N, kv_dtype="bf16", in_dtype="bf16",
        scale=1.0 / math.sqrt(128), partition_size=0, free_order=free_order,
        setup_ops=ops, decode_seqs=ids, ctx_lens=ctx, _segments=lambda i: segs[i],
        extra_segments=extra, prefix_caching=True,
        description="chat with prefix caching: 8 system prompts U[1000,2000] tokens, 128 "
                    "second-turn users (first turn released and cached), 64 first-turn "
                    "users, 32q/8kv, bf16")


def shared_prefix_bf16() -> Workload:
    """64 prompts x 4 samples sharing a 1032-token prefix, tails U{0..512}, bf16, 32q/8kv.

    Each sample has, before the decode step, generated one divergent token (the
    write that copies the shared half-full block) plus ``tail`` more tokens; the
    decode step appends one token more: ctx = 1032 + 1 + tail + 1.
    """
    seed, P, n, B, prefix = 5, 64, 4, 16, 1032
    rng = _rng(seed, _TAG_META, 0)
    tails = rng.integers(0, 512, size=P * n, endpoint=True).astype(np.int64)
    ids = np.arange(P * n, dtype=np.int64)           # sample k of prompt p has id 4p+k
    ctx = prefix + 1 + tails + 1
    need = 0
    for p in range(P):
        need += prefix // B                            # shared full prefix blocks
        for k in range(n):                             # each sample ends with blocks of its own
            need += blocks_for(ctx[p * n + k] - (prefix // B) * B, B)
    N = int(math.ceil(1.25 * need))
    free_order = _rng(seed, _TAG_META, 1).permutation(N).astype(np.int32)
    ops: List[Op] = []
    for p in range(P):
        ops.append(("add", p * n, prefix))
        for k in range(1, n):
            ops.append(("fork", p * n, p * n + k))
    ops.append(("append_batch", [int(s) for s in ids]))   # first divergent token: copy-on-write
    for s in ids:
        if tails[s] > 0:
            ops.append(("extend", int(s), int(tails[s])))

    def seg(i: int):
        p = i // n
        return [(p * n, 0, prefix), (10_000 + i, 0, int(ctx[i]) - prefix)]

    return Workload(
        name="shared-prefix-bf16", seed=seed, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=B, num_blocks=N, kv_dtype="bf16", in_dtype="bf16",
        scale=1.0 / math.sqrt(128), partition_size=512, free_order=free_order,
        setup_ops=ops, decode_seqs=ids, ctx_lens=ctx, _segments=seg,
        description="64 prompts x 4 samples sharing a 1032-token prefix (64 full blocks + "
                    "one half-full shared block), one divergent token + tail U{0..512} "
                    "per sample, bf16, 32q/8kv")


def long_context_bf16() -> Workload:
    """One sequence with a 32768-token context, 32 q / 8 KV heads, 64 partitions of 512."""
    return _plain("long-32k-bf16", 6, 1, 32, 8, 128, 16, [32768], "bf16", "bf16", 512,
                  pool_blocks=2560,
                  description="single 32768-token sequence, bf16, 32q/8kv, 64 partitions of 512")


CONFIGS: Dict[str, Callable[[], Workload]] = {
    "tiny-f32": tiny_f32,
    "7b-mha-bf16": mha7b_bf16,
    "13b-mha-bf16-churn": mha13b_bf16_churn,
    "8b-gqa-fp8": lambda: gqa8b("fp8"),
    "8b-gqa-bf16": lambda: gqa8b("bf16"),
    "8b-gqa-bf16-b8": lambda: gqa8b("bf16", 8),
    "8b-gqa-bf16-b32": lambda: gqa8b("bf16", 32),
    "8b-gqa-fp8-b32": lambda: gqa8b("fp8", 32),
    "mqa-16q-bf16": mqa_bf16,
    "shared-prefix-bf16": shared_prefix_bf16,
    "chat-prefix-cache-bf16": chat_prefix_cache_bf16,
    "long-32k-bf16": long_context_bf16,
}


def get(name: str) -> Workload:
    return CONFIGS[name]()


def random_small(seed: int, *, S: int, Hq: int, Hkv: int, D: int, B: int,
                 max_ctx: int, kv_dtype: str, in_dtype: str, partition_size: int = 0,
                 min_ctx: int = 0, extra_blocks: int = 4, shuffle_free: bool = True) -> Workload:
    """Small seeded workload for parity sweeps (ragged contexts, scattered blocks)."""
    rng = _rng(seed, _TAG_META, 7)
    ctx = rng.integers(max(min_ctx, 1), max_ctx, size=S, endpoint=True).astype(np.int64)
    need = sum(blocks_for(c, B) for c in ctx)
    N = need + extra_blocks
    free_order = rng.permutation(N) if shuffle_free else np.arange(N)
    return _plain(f"random-{seed}", seed, S, Hq, Hkv, D, B, ctx, kv_dtype, in_dtype,
                  partition_size, pool_blocks=N, free_order=free_order,
                  description="random small parity case")


class KVFeeder:
    """Serves ``wl.seq_kv_input`` for sequences in a known order, drawing ahead on threads.

    numpy's generators release the GIL, so drawing several sequences at once
    scales with the cores.  ``seq_order`` lists sequence ids in the order they
    will be asked for; results stay available for a few further requests.
    """

    def __init__(self, wl: "Workload", seq_order, workers: int = 8, ahead: int = 16,
                 keep: int = 8):
        from collections import OrderedDict
        from concurrent.futures import ThreadPoolExecutor

        self.wl = wl
        self.index = wl.seq_index()
        seen, order = set(), []
        for s in seq_order:
            s = int(s)
            if s in self.index and s not in seen:
                seen.add(s)
                order.append(self.index[s])
        self.order = order
        self.pos = 0
        self.ahead = ahead
        self.keep = keep
        self.ex = ThreadPoolExecutor(max_workers=workers)
        self.futs: Dict[int, object] = {}
        self.done: "OrderedDict[int, Tuple[np.ndarray, np.ndarray]]" = OrderedDict()

    def _fill(self):
        while len(self.futs) < self.ahead and self.pos < len(self.order):
            i = self.order[self.pos]
            self.pos += 1
            if i not in self.futs and i not in self.done:
                self.futs[i] = self.ex.submit(self.wl.seq_kv_input, i)

    def by_index(self, i: int):
        if i in self.done:
            self.done.move_to_end(i)
            return self.done[i]
        self._fill()
        fut = self.futs.pop(i, None)
        r = fut.result() if fut is not None else self.wl.seq_kv_input(i)
        self.done[i] = r
        while len(self.done) > self.keep:
            self.done.popitem(last=False)
        self._fill()
        return r

    def __call__(self, seq: int):
        seq = int(seq)
        if seq not in self.index:
            return self.wl.extra_kv_input(seq)
        return self.by_index(self.index[seq])

    def close(self):
        self.ex.shutdown(wait=False, cancel_futures=True)


def ops_seq_order(ops) -> List[int]:
    """Sequence ids in the order an allocator script first writes tokens for them."""
    out = []
    for op in ops:
        if op[0] in ("add", "extend", "add_tokens", "extend_tokens"):
            out.append(int(op[1]))
        elif op[0] == "append_batch":
            out.extend(int(s) for s in op[1])
    return out
