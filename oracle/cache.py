"""Cache operations of the oracle (test infrastructure only).

Pool layout (a convention of this library; the ultralytics glossary's code
example shows only a key pool of shape (blocks, block size, head dim)):

* key pool   ``[num_blocks, num_kv_heads, block_size, head_dim]`` -- a token's
  key for one head is a contiguous row, as in the glossary example;
* value pool ``[num_blocks, num_kv_heads, head_dim, block_size]`` -- within a
  block, a value is stored dimension-major (the 16 tokens of one dimension are
  contiguous).

Storage is fp32 (float32), bf16 (raw uint16 bits) or fp8 (E4M3FN codes, uint8).

``reshape_and_cache`` writes token i's key and value to the slot
``slot_mapping[i]``: block ``slot // B``, position ``slot % B`` (glossary, "How
paging works": position pos of a sequence is row pos mod B of the block that
its table lists at entry pos div B).
A negative slot means "skip this token".  Every other byte of the pools is left
as it was.

``copy_blocks`` is the copy of copy-on-write (ithome article, section 4): for
each (src, dst) pair the whole destination block of both pools becomes a copy
of the source block.  Pairs must have src != dst, distinct destinations, and no
destination that is also a source, so that their order does not matter.
"""
from __future__ import annotations

import numpy as np

from . import codec

_STORAGE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}
_POISON = {"f32": np.float32(np.nan).view(np.uint32), "bf16": 0x7FC0, "fp8": 0x7F}


def storage_dtype(kv_dtype: str):
    return _STORAGE[kv_dtype]


def new_pools(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
              kv_dtype: str):
    """Empty K and V pools with every slot holding a NaN pattern."""
    kshape = (num_blocks, num_kv_heads, block_size, head_dim)
    vshape = (num_blocks, num_kv_heads, head_dim, block_size)
    dt = _STORAGE[kv_dtype]
    if kv_dtype == "f32":
        k = np.full(kshape, np.nan, dtype=np.float32)
        v = np.full(vshape, np.nan, dtype=np.float32)
    else:
        k = np.full(kshape, _POISON[kv_dtype], dtype=dt)
        v = np.full(vshape, _POISON[kv_dtype], dtype=dt)
    return k, v


def encode(x: np.ndarray, in_dtype: str, kv_dtype: str, scale: float) -> np.ndarray:
    """Input values (float32 or bf16 bits) -> pool storage values."""
    if kv_dtype == in_dtype:
        return np.asarray(x, dtype=_STORAGE[kv_dtype])
    if kv_dtype == "fp8":
        xf = codec.bf16_to_f32(x) if in_dtype == "bf16" else np.asarray(x, dtype=np.float32)
        return codec.e4m3_quantize(xf, scale)
    raise ValueError(f"unsupported input {in_dtype} for a {kv_dtype} pool")


def reshape_and_cache(k_pool, v_pool, k, v, slot_mapping, in_dtype: str, kv_dtype: str,
                      k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Write token i's K/V ([T, Hkv, D]) to slot ``slot_mapping[i]`` of the pools."""
    B = k_pool.shape[2]
    ke = encode(k, in_dtype, kv_dtype, k_scale)
    ve = encode(v, in_dtype, kv_dtype, v_scale)
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        block, pos = divmod(int(slot), B)
        k_pool[block, :, pos, :] = ke[i]
        v_pool[block, :, :, pos] = ve[i]


def check_pairs(pairs, num_blocks: int) -> np.ndarray:
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    src, dst = pairs[:, 0], pairs[:, 1]
    if ((pairs < 0) | (pairs >= num_blocks)).any():
        raise ValueError("block id out of range")
    if (src == dst).any():
        raise ValueError("src == dst")
    if len(set(dst.tolist())) != len(dst):
        raise ValueError("duplicate destination")
    if set(dst.tolist()) & set(src.tolist()):
        raise ValueError("a destination is also a source")
    return pairs


def copy_blocks(k_pool, v_pool, pairs) -> None:
    """Copy-on-write copies: block dst of both pools becomes block src."""
    for src, dst in check_pairs(pairs, k_pool.shape[0]):
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs) -> None:
    """Swapping (review of the vLLM paper, preemption paragraphs): whole blocks move
    between two pools of the same block shape, the device pool and a host pool.  For
    each (src, dst) pair block dst of the destination pools becomes block src of the
    source pools, K and V.  Destinations must be distinct; sources and destinations
    index different pools, so a destination may carry a source's number."""
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if ((pairs[:, 0] < 0) | (pairs[:, 0] >= src_k.shape[0])).any():
        raise ValueError("source block out of range")
    if ((pairs[:, 1] < 0) | (pairs[:, 1] >= dst_k.shape[0])).any():
        raise ValueError("destination block out of range")
    if len(set(pairs[:, 1].tolist())) != len(pairs):
        raise ValueError("duplicate destination")
    if src_k.shape[1:] != dst_k.shape[1:] or src_v.shape[1:] != dst_v.shape[1:]:
        raise ValueError("pools of different block shapes")
    for src, dst in pairs:
        dst_k[dst] = src_k[src]
        dst_v[dst] = src_v[src]


def apply_events(k_pool, v_pool, events, kv_input, in_dtype: str, kv_dtype: str,
                 k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Run the device work of an allocator script: copies and token writes, in order.

    ``kv_input(seq)`` returns that sequence's K, V in input format, indexed by
    logical position.
    """
    for ev in events:
        if ev[0] == "copy":
            copy_blocks(k_pool, v_pool, ev[1])
        else:
            _, seq, positions, slots = ev
            k, v = kv_input(seq)
            reshape_and_cache(k_pool, v_pool, k[positions], v[positions], slots,
                              in_dtype, kv_dtype, k_scale, v_scale)
