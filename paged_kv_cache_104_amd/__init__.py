"""Python binding of libpagedkv: paged-KV decode for AMD MI355X (gfx950).

Argument marshalling only: every step of the hot path runs in the HIP kernels
of ``libpagedkv.so`` (built in-tree by ``build_lib``); PyTorch provides device
memory and the current stream.  Importing this package without the built
library raises ImportError -- there is no CPU fallback.

Device calls (see include/pagedkv.h for layouts and error behaviour):
``reshape_and_cache``, ``copy_blocks``, ``paged_attn_decode``.
Host block manager: ``BlockManager`` (refcounted free-list allocator with fork
and copy-on-write).
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PKV_OK, PKV_E_INVAL, PKV_E_NOMEM, PKV_E_UNSUPPORTED, PKV_E_HIP = 0, -1, -2, -3, -4
PKV_F32, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2
IMPL_AUTO, IMPL_VECTOR, IMPL_MFMA = 0, 1, 2
IMPL_SHARED_BLOCKS = 0x100     # hint: some blocks are shared between sequences
DTYPES = {"f32": PKV_F32, "bf16": PKV_BF16, "fp8": PKV_FP8_E4M3}


class PagedKVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"pagedkv error {code}: {msg}")
        self.code = code


class NoMemory(PagedKVError):
    """The block manager has too few free blocks; its state is unchanged."""


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float)]


class BmStats(ctypes.Structure):
    _fields_ = [("free_blocks", ctypes.c_int32), ("used_blocks", ctypes.c_int32),
                ("tokens", ctypes.c_int64), ("slots_allocated", ctypes.c_int64),
                ("logical_blocks", ctypes.c_int64), ("physical_blocks", ctypes.c_int64)]


_i32, _i64, _f32, _vp, _sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                              ctypes.c_size_t)
_pi32, _pi64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)

_SIGNATURES = {
    "pkv_reshape_and_cache": (ctypes.c_int, [_vp, _vp, _i32, _vp, _i64, _vp, _vp,
                                             ctypes.POINTER(CacheDesc), _vp]),
    "pkv_copy_blocks": (ctypes.c_int, [_vp, _vp, _vp, _i64, ctypes.POINTER(CacheDesc), _vp]),
    "pkv_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pkv_paged_attn_decode": (ctypes.c_int, [_vp, _i32, _vp, _vp, ctypes.POINTER(CacheDesc), _vp,
                                             _i32, _vp, _i32, _i32, _f32, _vp, _i32, _i32, _vp,
                                             _sz, _vp]),
    "pkv_paged_attn_decode_ex": (ctypes.c_int, [_vp, _i32, _vp, _vp, ctypes.POINTER(CacheDesc),
                                                _vp, _i32, _vp, _i32, _i32, _f32, _vp, _i32,
                                                _i32, _vp, _sz, _vp, _i32]),
    "pkv_paged_attn_partials": (ctypes.c_int, [_vp, _i32, _vp, _vp, ctypes.POINTER(CacheDesc),
                                               _vp, _i32, _vp, _i32, _i32, _f32, _vp, _i32,
                                               _i32, _vp, _sz, _vp, _i32]),
    "pkv_paged_attn_merge": (ctypes.c_int, [_i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                            _vp, _sz, _vp, _vp]),
    "pkv_prefix_rows": (_i32, [_pi32, _pi32, _i32, _i32, _i32, _i32, _i32, _pi32, _pi32]),
    "pkv_prefix_order": (_i32, [_pi32, _pi32, _i32, _i32, _i32, _pi32]),
    "pkv_time_next_decode": (ctypes.c_int, [_vp, _vp]),
    "pkv_decode_scratch_bytes": (_sz, []),
    "pkv_paged_attn_decode_noalloc": (ctypes.c_int, [_vp, _i32, _vp, _vp,
                                                     ctypes.POINTER(CacheDesc), _vp, _i32, _vp,
                                                     _i32, _i32, _f32, _vp, _i32, _i32, _vp,
                                                     _i32]),
    "pkv_rows_workspace_bytes": (_sz, [ctypes.POINTER(CacheDesc), _i32]),
    "pkv_paged_attn_decode_rows": (ctypes.c_int, [_vp, _i32, _vp, _vp, ctypes.POINTER(CacheDesc),
                                                  _vp, _i32, _vp, _i32, _i32, _f32, _vp, _i32,
                                                  _i32, _vp, _i32, _vp, _vp, _sz, _vp, _i32]),
    "pkv_swap_blocks": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32,
                                       ctypes.POINTER(CacheDesc), _vp]),
    "pkv_swap_blocks_dma": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32,
                                           ctypes.POINTER(CacheDesc), _vp]),
    "pkv_memory_kind": (_i32, [_vp]),
    "pkv_append_tokens": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp,
                                         ctypes.POINTER(CacheDesc), _vp, _i32, _vp, _vp]),
    "pkv_quest_meta_bytes": (_sz, [ctypes.POINTER(CacheDesc)]),
    "pkv_quest_update_blocks": (ctypes.c_int, [_vp, ctypes.POINTER(CacheDesc), _vp, _vp, _vp,
                                               _i32, _vp]),
    "pkv_quest_update_tails": (ctypes.c_int, [_vp, ctypes.POINTER(CacheDesc), _vp, _vp, _i32,
                                              _vp, _i32, _vp]),
    "pkv_quest_workspace_bytes": (_sz, [ctypes.POINTER(CacheDesc), _i32, _i32, _i32, _i32, _i32,
                                        _i32]),
    "pkv_quest_select": (ctypes.c_int, [_vp, _i32, _vp, ctypes.POINTER(CacheDesc), _vp, _i32,
                                        _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "pkv_quest_decode": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, ctypes.POINTER(CacheDesc),
                                        _vp, _i32, _vp, _i32, _i32, _f32, _vp, _i32, _i32,
                                        _i32, _vp, _sz, _vp, _i32]),
    "pkv_read_probe": (ctypes.c_int, [_vp, _sz, _i64, _vp, _i64, _vp, _i32, _vp]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_char_p, []),
    "pkv_bm_create": (_vp, [_i32, _i32, _pi32, _i32]),
    "pkv_bm_destroy": (None, [_vp]),
    "pkv_bm_add_seq": (ctypes.c_int, [_vp, _i64, _i64]),
    "pkv_bm_fork": (ctypes.c_int, [_vp, _i64, _i64]),
    "pkv_bm_append": (ctypes.c_int, [_vp, _i64, _pi64, _pi64, _pi64]),
    "pkv_bm_append_batch": (ctypes.c_int, [_vp, _pi64, _i32, _pi64, _pi64, _pi32]),
    "pkv_bm_extend": (ctypes.c_int, [_vp, _i64, _i64, _pi64, _pi64, _pi64]),
    "pkv_bm_free_seq": (ctypes.c_int, [_vp, _i64]),
    "pkv_bm_slots": (ctypes.c_int, [_vp, _i64, _i64, _i64, _pi64]),
    "pkv_bm_block_tables": (ctypes.c_int, [_vp, _pi64, _i32, _pi32, _i32, _pi32]),
    "pkv_bm_stats": (ctypes.c_int, [_vp, ctypes.POINTER(BmStats)]),
    "pkv_bm_refcount": (_i32, [_vp, _i32]),
    "pkv_bm_seq_len": (_i64, [_vp, _i64]),
    "pkv_bm_free_list": (_i32, [_vp, _pi32, _i32]),
    "pkv_bm_set_prefix_caching": (ctypes.c_int, [_vp, _i32]),
    "pkv_bm_lookup": (ctypes.c_int, [_vp, _pi32, _i64, _pi64]),
    "pkv_bm_add_seq_tokens": (ctypes.c_int, [_vp, _i64, _pi32, _i64, _pi64]),
    "pkv_bm_append_batch_tokens": (ctypes.c_int, [_vp, _pi64, _pi32, _i32, _pi64, _pi64, _pi32]),
    "pkv_bm_extend_tokens": (ctypes.c_int, [_vp, _i64, _pi32, _i64, _pi64, _pi64, _pi64]),
    "pkv_bm_cache_stats": (ctypes.c_int, [_vp, _pi64]),
    "pkv_bm_evictable_list": (_i32, [_vp, _pi32, _i32]),
    "pkv_bm_set_host_pool": (ctypes.c_int, [_vp, _i32]),
    "pkv_bm_swap_out": (ctypes.c_int, [_vp, _pi64, _i32, _pi64, _i32, _pi32]),
    "pkv_bm_swap_in": (ctypes.c_int, [_vp, _pi64, _i32, _pi64, _i32, _pi32]),
    "pkv_bm_swap_stats": (ctypes.c_int, [_vp, _pi64]),
    "pkv_bm_host_refcount": (_i32, [_vp, _i32]),
    "pkv_bm_host_free_list": (_i32, [_vp, _pi32, _i32]),
    "pkv_bm_seq_blocks": (ctypes.c_int, [_vp, _i64, _pi32, _i32]),
    "pkv_bm_block_fills": (_i32, [_vp, _pi64, _i32, _pi32, _pi32, _i32]),
    "pkv_quest_blocks_of_slots": (_i32, [_pi64, _i64, _i32, _pi32, _pi32, _i32]),
}


# Host calls: what the host-only library (no device code) exports.
_HOST_ONLY = ("pkv_bm_", "pkv_prefix_rows", "pkv_prefix_order", "pkv_quest_blocks_of_slots",
              "pkv_last_error", "pkv_version")


def _load_host_only(path: str):
    """The host-only library (the block manager and the shared-prefix unit builder, e.g. the
    sanitizer build of build_lib.build_host_sanitized): host calls bound, device calls
    absent, so any device wrapper fails loudly."""
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        if not name.startswith(_HOST_ONLY):
            continue
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def _load():
    host_lib = os.environ.get("PKV_HOST_LIB")
    if host_lib:
        return _load_host_only(host_lib)
    # torch ships its own HIP runtime (soname libamdhip64.so.7).  Loading torch
    # first makes this library bind to that same runtime instead of bringing a
    # second copy into the process.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python paged_kv_cache_104_amd/build_lib.py` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        if not hasattr(lib, name):
            raise ImportError(f"{LIB_PATH} lacks {name}: it is stale, rebuild it with "
                              "`python paged_kv_cache_104_amd/build_lib.py`")
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(rc: int) -> None:
    if rc != PKV_OK:
        msg = lib.pkv_last_error().decode(errors="replace")
        if rc == PKV_E_NOMEM:
            raise NoMemory(rc, msg)
        raise PagedKVError(rc, msg)


def version() -> str:
    return lib.pkv_version().decode()


# ---------------------------------------------------------------------------- device side

def _torch():
    import torch
    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _on(stream=None):
    """Context in which a wrapper allocates its temporaries and uploads its arguments: with
    ``stream`` current, so that the caching allocator ties their memory to that stream (it is
    not handed out again before the library's work on ``stream`` is done) and the uploads are
    ordered before that work."""
    import contextlib

    if stream is None:
        return contextlib.nullcontext()
    return _torch().cuda.stream(stream)


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PKV_FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def cache_desc(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
               kv_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0) -> CacheDesc:
    return CacheDesc(num_blocks, num_kv_heads, block_size, head_dim, DTYPES[kv_dtype],
                     k_scale, v_scale)


def pool_shapes(desc: CacheDesc) -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
    """(key pool shape [N, H, B, D], value pool shape [N, H, D, B])."""
    N, H, B, D = desc.num_blocks, desc.num_kv_heads, desc.block_size, desc.head_dim
    return (N, H, B, D), (N, H, D, B)


def alloc_pools(desc: CacheDesc, device="cuda", poison: bool = True):
    """Allocate one layer's K and V pools (torch tensors); unused slots hold NaN patterns."""
    torch = _torch()
    tdt = {PKV_F32: torch.float32, PKV_BF16: torch.bfloat16, PKV_FP8_E4M3: torch.uint8}[desc.kv_dtype]
    ks, vs = pool_shapes(desc)
    k = torch.empty(ks, dtype=tdt, device=device)
    v = torch.empty(vs, dtype=tdt, device=device)
    if poison:
        if desc.kv_dtype == PKV_FP8_E4M3:
            k.fill_(0x7F)
            v.fill_(0x7F)
        else:
            k.fill_(float("nan"))
            v.fill_(float("nan"))
    return k, v


def _ptr(t) -> int:
    return int(t.data_ptr())


def append_tokens(k, v, slots, positions, k_pool, v_pool, desc: CacheDesc, block_tables,
                  context_lens, stream=None) -> None:
    """Decode-step append: write token i's K, V ([T, H, D]) to host slot ``slots[i]`` and set
    row i's device table entry for ``positions[i]`` and its context length."""
    ks, vs = pool_shapes(desc)
    _check_pool(k_pool, ks, desc, "k_pool")
    _check_pool(v_pool, vs, desc, "v_pool")
    sl = np.ascontiguousarray(slots, dtype=np.int64)
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    T = len(sl)
    if len(pos) != T or tuple(k.shape) != (T, desc.num_kv_heads, desc.head_dim) or k.shape != v.shape:
        raise ValueError(f"k/v must be [{T}, {desc.num_kv_heads}, {desc.head_dim}], one position per slot")
    if not (block_tables.is_cuda and context_lens.is_cuda and block_tables.is_contiguous()
            and context_lens.is_contiguous()):
        raise ValueError("block_tables and context_lens must be contiguous device tensors")
    if block_tables.shape[0] < T or context_lens.numel() < T:
        raise ValueError("fewer table rows than tokens")
    _check(lib.pkv_append_tokens(_ptr(k), _ptr(v), dtype_code(k), sl.ctypes.data, pos.ctypes.data,
                                 T, _ptr(k_pool), _ptr(v_pool), ctypes.byref(desc),
                                 _ptr(block_tables), int(block_tables.shape[1]),
                                 _ptr(context_lens), _stream(stream)))


def alloc_host_pools(desc: CacheDesc, num_host_blocks: int):
    """Pinned host K and V pools of ``num_host_blocks`` blocks with the device pools' block
    shape, for swapping (the GPU reads and writes them directly)."""
    torch = _torch()
    tdt = {PKV_F32: torch.float32, PKV_BF16: torch.bfloat16, PKV_FP8_E4M3: torch.uint8}[desc.kv_dtype]
    ks, vs = pool_shapes(desc)
    k = torch.empty((num_host_blocks,) + ks[1:], dtype=tdt, pin_memory=True)
    v = torch.empty((num_host_blocks,) + vs[1:], dtype=tdt, pin_memory=True)
    return k, v


def _check_swap_pool(t, shape, desc: CacheDesc, what: str) -> int:
    if not t.is_contiguous() or not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{what} must be a contiguous device tensor or pinned host tensor")
    if tuple(t.shape[1:]) != tuple(shape[1:]):
        raise ValueError(f"{what} block shape {tuple(t.shape[1:])} != {tuple(shape[1:])}")
    if dtype_code(t) != desc.kv_dtype:
        raise ValueError(f"{what} dtype {t.dtype} does not match the descriptor")
    return int(t.shape[0])


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs, desc: CacheDesc, method: str = "kernel",
                stream=None) -> None:
    """Move whole blocks between the device pools and pinned host pools (either way): block
    dst of ``dst_*`` becomes block src of ``src_*`` for each (src, dst) of ``pairs`` (host,
    checked).  ``method`` 'kernel' copies with one GPU kernel, 'dma' with one copy-engine
    transfer per run of consecutive blocks."""
    torch = _torch()
    ks, vs = pool_shapes(desc)
    ns = _check_swap_pool(src_k, ks, desc, "src_k")
    if _check_swap_pool(src_v, vs, desc, "src_v") != ns:
        raise ValueError("src_k and src_v hold different numbers of blocks")
    nd = _check_swap_pool(dst_k, ks, desc, "dst_k")
    if _check_swap_pool(dst_v, vs, desc, "dst_v") != nd:
        raise ValueError("dst_k and dst_v hold different numbers of blocks")
    p = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
    if len(p) == 0:
        return
    if ((p[:, 0] < 0) | (p[:, 0] >= ns) | (p[:, 1] < 0) | (p[:, 1] >= nd)).any():
        raise ValueError("block id out of range")
    if len(np.unique(p[:, 1])) != len(p):
        raise ValueError("duplicate destination")
    args = (_ptr(src_k), _ptr(src_v), _ptr(dst_k), _ptr(dst_v))
    if method == "kernel":
        with _on(stream):
            dev = torch.from_numpy(p).to("cuda")
            _check(lib.pkv_swap_blocks(*args, _ptr(dev), len(p), ns, nd, ctypes.byref(desc),
                                       _stream(stream)))
    elif method == "dma":
        _check(lib.pkv_swap_blocks_dma(*args, p.ctypes.data, len(p), ns, nd, ctypes.byref(desc),
                                       _stream(stream)))
    else:
        raise ValueError(f"unknown method {method}")


def _check_pool(t, shape, desc: CacheDesc, what: str) -> None:
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} shape {tuple(t.shape)} != {tuple(shape)}")
    if dtype_code(t) != desc.kv_dtype:
        raise ValueError(f"{what} dtype {t.dtype} does not match the descriptor")


def reshape_and_cache(k, v, slot_mapping, k_pool, v_pool, desc: CacheDesc, stream=None) -> None:
    """Write new tokens' K, V ([T, H, D]) to slots ``slot_mapping`` (int64 [T]; <0 skips)."""
    ks, vs = pool_shapes(desc)
    _check_pool(k_pool, ks, desc, "k_pool")
    _check_pool(v_pool, vs, desc, "v_pool")
    T = int(slot_mapping.numel())
    if tuple(k.shape) != (T, desc.num_kv_heads, desc.head_dim) or k.shape != v.shape:
        raise ValueError(f"k/v must be [{T}, {desc.num_kv_heads}, {desc.head_dim}]")
    if not (k.is_contiguous() and v.is_contiguous() and slot_mapping.is_contiguous()):
        raise ValueError("k, v and slot_mapping must be contiguous")
    if slot_mapping.dtype != _torch().int64 or not slot_mapping.is_cuda:
        raise ValueError("slot_mapping must be a device int64 tensor")
    _check(lib.pkv_reshape_and_cache(_ptr(k), _ptr(v), dtype_code(k), _ptr(slot_mapping), T,
                                     _ptr(k_pool), _ptr(v_pool), ctypes.byref(desc),
                                     _stream(stream)))


def check_pairs(pairs: np.ndarray, num_blocks: int) -> np.ndarray:
    """Host check of copy pairs: in range, src != dst, distinct dst, no dst that is a src."""
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if ((pairs < 0) | (pairs >= num_blocks)).any():
        raise ValueError("copy pair block id out of range")
    src, dst = pairs[:, 0], pairs[:, 1]
    if (src == dst).any():
        raise ValueError("copy pair with src == dst")
    if len(np.unique(dst)) != len(dst):
        raise ValueError("two copy pairs share a destination")
    if np.intersect1d(src, dst).size:
        raise ValueError("a copy destination is also a source")
    return pairs


def copy_blocks(k_pool, v_pool, pairs, desc: CacheDesc, stream=None) -> None:
    """Copy-on-write copies: block dst of both pools becomes block src.

    ``pairs`` on the host (list / numpy / CPU tensor, [n, 2]) is checked and
    uploaded; a device int64 tensor is passed as is (the caller vouches for it).
    """
    torch = _torch()
    ks, vs = pool_shapes(desc)
    _check_pool(k_pool, ks, desc, "k_pool")
    _check_pool(v_pool, vs, desc, "v_pool")
    if isinstance(pairs, torch.Tensor) and pairs.is_cuda:
        dev = pairs.contiguous()
        if dev.dtype != torch.int64:
            raise ValueError("device pairs must be int64")
    else:
        host = pairs.cpu().numpy() if isinstance(pairs, torch.Tensor) else pairs
        host = check_pairs(host, desc.num_blocks)
        if len(host) == 0:
            return
        with _on(stream):
            dev = torch.from_numpy(host).to(k_pool.device, non_blocking=False)
    n = int(dev.numel() // 2)
    if n == 0:
        return
    with _on(stream):
        _check(lib.pkv_copy_blocks(_ptr(k_pool), _ptr(v_pool), _ptr(dev), n, ctypes.byref(desc),
                                   _stream(stream)))


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int,
                           max_context_len: int, partition_size: int) -> int:
    return int(lib.pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len,
                                              partition_size))


def paged_attn_decode(q, k_pool, v_pool, block_tables, context_lens, scale: float, out,
                      desc: CacheDesc, max_context_len: int, partition_size: int = 0,
                      workspace=None, impl: int = IMPL_AUTO, stream=None):
    """Decode attention: q [S, Hq, D] over each sequence's paged context -> out [S, Hq, D]."""
    torch = _torch()
    ks, vs = pool_shapes(desc)
    _check_pool(k_pool, ks, desc, "k_pool")
    _check_pool(v_pool, vs, desc, "v_pool")
    S, Hq, D = q.shape
    if D != desc.head_dim or tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("q / out shapes or dtypes do not match")
    if not (q.is_contiguous() and out.is_contiguous() and block_tables.is_contiguous()
            and context_lens.is_contiguous()):
        raise ValueError("q, out, block_tables and context_lens must be contiguous")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    need = decode_workspace_bytes(S, Hq, D, max_context_len, partition_size)
    with _on(stream):
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_ptr = _ptr(workspace) if workspace is not None else 0
        ws_bytes = int(workspace.numel() * workspace.element_size()) if workspace is not None else 0
        _check(lib.pkv_paged_attn_decode_ex(
            _ptr(q), dtype_code(q), _ptr(k_pool), _ptr(v_pool), ctypes.byref(desc),
            _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), S, Hq,
            float(scale), _ptr(out), int(max_context_len), int(partition_size), ws_ptr, ws_bytes,
            _stream(stream), int(impl)))
    return out


def paged_attn_decode_noalloc(q, k_pool, v_pool, block_tables, context_lens, scale: float, out,
                              desc: CacheDesc, max_context_len: int, partition_size: int = 0,
                              impl: int = IMPL_AUTO, stream=None):
    """paged_attn_decode with the library's static scratch instead of a workspace: nothing
    is allocated (no tensor is created here either).  Calls that overlap on one device
    race on the scratch."""
    ks, vs = pool_shapes(desc)
    _check_pool(k_pool, ks, desc, "k_pool")
    _check_pool(v_pool, vs, desc, "v_pool")
    S, Hq, D = q.shape
    if D != desc.head_dim or tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("q / out shapes or dtypes do not match")
    if not (q.is_contiguous() and out.is_contiguous() and block_tables.is_contiguous()
            and context_lens.is_contiguous()):
        raise ValueError("q, out, block_tables and context_lens must be contiguous")
    _check_tables(block_tables, context_lens)
    if block_tables.shape[0] != S:
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    _check(lib.pkv_paged_attn_decode_noalloc(
        _ptr(q), dtype_code(q), _ptr(k_pool), _ptr(v_pool), ctypes.byref(desc),
        _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), S, Hq,
        float(scale), _ptr(out), int(max_context_len), int(partition_size), _stream(stream),
        int(impl)))
    return out


def decode_scratch_bytes() -> int:
    return int(lib.pkv_decode_scratch_bytes())


def paged_attn_partials(q, k_pool, v_pool, block_tables, context_lens, scale: float, out,
                        desc: CacheDesc, max_context_len: int, partition_size: int, workspace,
                        impl: int = IMPL_AUTO, stream=None):
    """First phase of paged_attn_decode (the per-partition kernel); see include/pagedkv.h."""
    S, Hq, D = q.shape
    ws_ptr = _ptr(workspace) if workspace is not None else 0
    ws_bytes = int(workspace.numel() * workspace.element_size()) if workspace is not None else 0
    _check(lib.pkv_paged_attn_partials(
        _ptr(q), dtype_code(q), _ptr(k_pool), _ptr(v_pool), ctypes.byref(desc),
        _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), S, Hq,
        float(scale), _ptr(out), int(max_context_len), int(partition_size), ws_ptr, ws_bytes,
        _stream(stream), int(impl)))


def paged_attn_merge(out, context_lens, num_kv_heads: int, max_context_len: int,
                     partition_size: int, workspace, stream=None):
    """Second phase of paged_attn_decode: merge split contexts into ``out``."""
    S, Hq, D = out.shape
    ws_ptr = _ptr(workspace) if workspace is not None else 0
    ws_bytes = int(workspace.numel() * workspace.element_size()) if workspace is not None else 0
    _check(lib.pkv_paged_attn_merge(dtype_code(out), _ptr(context_lens), S, Hq,
                                    int(num_kv_heads), D,
                                    int(max_context_len), int(partition_size), ws_ptr, ws_bytes,
                                    _ptr(out), _stream(stream)))


# ---------------------------------------------------------------------------- shared-prefix decode

def prefix_rows(tables: np.ndarray, lens: np.ndarray, block_size: int, group: int,
                min_shared_blocks: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """Units of the shared-prefix decode for a batch (host): ``(rows [U, 4], seq_rows [S, 4])``
    int32, built by the library from the batch's block tables and context lengths; a unit
    is {first sequence, shared tokens, members, 0}, seq_rows[s] = {unit, member, 0, 0}."""
    t = np.ascontiguousarray(tables, dtype=np.int32)
    ln = np.ascontiguousarray(lens, dtype=np.int32)
    S = int(t.shape[0])
    rows = np.zeros((max(1, S), 4), dtype=np.int32)
    seq_rows = np.zeros((max(1, S), 4), dtype=np.int32)
    n = int(lib.pkv_prefix_rows(t.ctypes.data_as(_pi32), ln.ctypes.data_as(_pi32), S,
                                int(t.shape[1]) if t.ndim == 2 else 0, int(block_size),
                                int(group), int(min_shared_blocks),
                                rows.ctypes.data_as(_pi32), seq_rows.ctypes.data_as(_pi32)))
    _check(min(n, 0))
    return rows[:n].copy(), seq_rows[:S].copy()


def time_next_decode(start=None, stop=None):
    """The calling thread's next decode kernel records its own start and end in these
    torch.cuda.Event objects (created beforehand, timing enabled); no arguments cancels."""
    _check(lib.pkv_time_next_decode(ctypes.c_void_p(start.cuda_event if start else 0),
                                    ctypes.c_void_p(stop.cuda_event if stop else 0)))


def prefix_order(tables: np.ndarray, lens: np.ndarray, block_size: int) -> np.ndarray:
    """Batch order (host int32 [S]) that puts sequences sharing leading blocks next to
    each other; order[k] is the batch index of the k-th sequence."""
    t = np.ascontiguousarray(tables, dtype=np.int32)
    ln = np.ascontiguousarray(lens, dtype=np.int32)
    S = int(t.shape[0])
    order = np.zeros(max(1, S), dtype=np.int32)
    _check(lib.pkv_prefix_order(t.ctypes.data_as(_pi32), ln.ctypes.data_as(_pi32), S,
                                int(t.shape[1]) if t.ndim == 2 else 0, int(block_size),
                                order.ctypes.data_as(_pi32)))
    return order[:S].copy()


def rows_workspace_bytes(desc: CacheDesc, num_rows: int) -> int:
    return int(lib.pkv_rows_workspace_bytes(ctypes.byref(desc), int(num_rows)))


def paged_attn_decode_rows(q, k_pool, v_pool, block_tables, context_lens, scale: float, out,
                           desc: CacheDesc, max_context_len: int, partition_size: int,
                           rows, seq_rows, workspace=None, phases: int = 3, stream=None,
                           shared_blocks: bool = False):
    """Shared-prefix decode (see include/pagedkv.h): ``rows`` / ``seq_rows`` are device int32
    tensors [R, 4] / [S, 4] (``prefix_rows`` builds them on the host).  ``shared_blocks``
    adds PKV_IMPL_SHARED_BLOCKS to ``phases`` (cached K/V loads; for batches in which some
    unit's reread field is set)."""
    torch = _torch()
    S, Hq, D = q.shape
    if rows.dtype != torch.int32 or seq_rows.dtype != torch.int32:
        raise ValueError("rows and seq_rows must be int32")
    if rows.dim() != 2 or rows.shape[1] != 4 or tuple(seq_rows.shape) != (S, 4):
        raise ValueError("rows must be [R, 4] and seq_rows [S, 4]")
    if not (rows.is_contiguous() and seq_rows.is_contiguous()):
        raise ValueError("rows and seq_rows must be contiguous")
    R = int(rows.shape[0])
    with _on(stream):
        if workspace is None:
            workspace = torch.empty(rows_workspace_bytes(desc, R), dtype=torch.uint8,
                                    device=q.device)
        ws_bytes = int(workspace.numel() * workspace.element_size())
        _check(lib.pkv_paged_attn_decode_rows(
            _ptr(q), dtype_code(q), _ptr(k_pool), _ptr(v_pool), ctypes.byref(desc),
            _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), S, Hq,
            float(scale), _ptr(out), int(max_context_len), int(partition_size), _ptr(rows), R,
            _ptr(seq_rows), _ptr(workspace), ws_bytes, _stream(stream),
            int(phases) | (IMPL_SHARED_BLOCKS if shared_blocks else 0)))
    return out


# ---------------------------------------------------------------------------- QUEST

def quest_meta_shape(desc: CacheDesc) -> Tuple[int, ...]:
    """[N, H, 2, D]: per block and KV head, the channel-wise minimum (row 0) and maximum
    (row 1) of its valid keys, in the pool's element type."""
    return (desc.num_blocks, desc.num_kv_heads, 2, desc.head_dim)


def alloc_quest_meta(desc: CacheDesc, device="cuda"):
    torch = _torch()
    tdt = {PKV_F32: torch.float32, PKV_BF16: torch.bfloat16, PKV_FP8_E4M3: torch.uint8}[desc.kv_dtype]
    meta = torch.zeros(quest_meta_shape(desc), dtype=tdt, device=device)
    assert meta.numel() * meta.element_size() == lib.pkv_quest_meta_bytes(ctypes.byref(desc))
    return meta


def _check_meta(meta, desc: CacheDesc) -> None:
    _check_pool(meta, quest_meta_shape(desc), desc, "meta")


def _dev_i32(x, device):
    torch = _torch()
    if isinstance(x, torch.Tensor) and x.is_cuda:
        if x.dtype != torch.int32 or not x.is_contiguous():
            raise ValueError("device index arrays must be contiguous int32")
        return x
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x), dtype=np.int32)).to(device)


def quest_update_blocks(k_pool, meta, blocks, counts, desc: CacheDesc, stream=None) -> None:
    """Recompute the metadata of ``blocks[i]`` over its first ``counts[i]`` slots (distinct
    blocks; host arrays are uploaded)."""
    ks, _ = pool_shapes(desc)
    _check_pool(k_pool, ks, desc, "k_pool")
    _check_meta(meta, desc)
    with _on(stream):
        b, c = _dev_i32(blocks, k_pool.device), _dev_i32(counts, k_pool.device)
        if b.numel() != c.numel():
            raise ValueError("one count per block")
        if b.numel() == 0:
            return
        _check(lib.pkv_quest_update_blocks(_ptr(k_pool), ctypes.byref(desc), _ptr(meta),
                                           _ptr(b), _ptr(c), int(b.numel()), _stream(stream)))


def quest_blocks_of_slots(slots, block_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """(distinct blocks, fill counts) touched by a write to host ``slots``, computed by the
    library (pkv_quest_blocks_of_slots)."""
    sl = np.ascontiguousarray(np.asarray(slots, dtype=np.int64).ravel())
    cap = len(sl)
    blocks = np.empty(max(1, cap), np.int32)
    fills = np.empty(max(1, cap), np.int32)
    n = int(lib.pkv_quest_blocks_of_slots(sl.ctypes.data_as(_pi64), len(sl), int(block_size),
                                          blocks.ctypes.data_as(_pi32),
                                          fills.ctypes.data_as(_pi32), cap))
    _check(min(n, 0))
    return blocks[:n].copy(), fills[:n].copy()


def quest_update_tails(k_pool, meta, block_tables, context_lens, desc: CacheDesc,
                       stream=None) -> None:
    """After a decode-step append: recompute each row's last block from device tables."""
    ks, _ = pool_shapes(desc)
    _check_pool(k_pool, ks, desc, "k_pool")
    _check_meta(meta, desc)
    _check_tables(block_tables, context_lens)
    _check(lib.pkv_quest_update_tails(_ptr(k_pool), ctypes.byref(desc), _ptr(meta),
                                      _ptr(block_tables), int(block_tables.shape[1]),
                                      _ptr(context_lens), int(context_lens.numel()),
                                      _stream(stream)))


def _check_tables(block_tables, context_lens) -> None:
    torch = _torch()
    if not (block_tables.is_cuda and context_lens.is_cuda and block_tables.is_contiguous()
            and context_lens.is_contiguous()):
        raise ValueError("block_tables and context_lens must be contiguous device tensors")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != context_lens.numel():
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")


def quest_workspace_bytes(desc: CacheDesc, num_seqs: int, num_q_heads: int, max_blocks: int,
                          max_context_len: int, partition_size: int, budget_blocks: int) -> int:
    n = int(lib.pkv_quest_workspace_bytes(ctypes.byref(desc), num_seqs, num_q_heads, max_blocks,
                                          max_context_len, partition_size, budget_blocks))
    if n == 0:
        raise PagedKVError(PKV_E_INVAL, (lib.pkv_last_error() or b"").decode())
    return n


def _quest_ws(workspace, desc, q, block_tables, max_context_len, partition_size, budget):
    torch = _torch()
    S, Hq, _ = q.shape
    need = quest_workspace_bytes(desc, S, Hq, int(block_tables.shape[1]), max_context_len,
                                 partition_size, budget)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    return workspace, int(workspace.numel() * workspace.element_size())


def quest_select(q, meta, desc: CacheDesc, block_tables, context_lens, max_context_len: int,
                 budget_blocks: int, workspace=None, stream=None):
    """(sel_tables [S*H, min(max_blocks, budget)], sel_lens [S*H]): per (sequence, KV head)
    the chosen blocks in logical order as block * H + head, and their tokens."""
    torch = _torch()
    _check_meta(meta, desc)
    _check_tables(block_tables, context_lens)
    S, Hq, D = q.shape
    if D != desc.head_dim or not q.is_contiguous() or block_tables.shape[0] != S:
        raise ValueError("q must be a contiguous [S, Hq, D] with one table row per sequence")
    H = desc.num_kv_heads
    width = max(1, min(int(block_tables.shape[1]), int(budget_blocks)))
    with _on(stream):
        sel_t = torch.full((S * H, width), -1, dtype=torch.int32, device=q.device)
        sel_l = torch.zeros(S * H, dtype=torch.int32, device=q.device)
        ws, wsb = _quest_ws(workspace, desc, q, block_tables, max_context_len, 0, budget_blocks)
        _check(lib.pkv_quest_select(_ptr(q), dtype_code(q), _ptr(meta), ctypes.byref(desc),
                                    _ptr(block_tables), int(block_tables.shape[1]),
                                    _ptr(context_lens), S, Hq, int(max_context_len),
                                    int(budget_blocks), _ptr(sel_t), _ptr(sel_l), _ptr(ws), wsb,
                                    _stream(stream)))
    return sel_t, sel_l


def quest_decode(q, k_pool, v_pool, meta, desc: CacheDesc, block_tables, context_lens,
                 scale: float, out, max_context_len: int, budget_blocks: int,
                 partition_size: int = 0, workspace=None, impl: int = IMPL_AUTO, stream=None):
    """Decode attention over the QUEST-chosen ``budget_blocks`` blocks of every
    (sequence, KV head); arguments as paged_attn_decode plus the metadata and budget."""
    ks, vs = pool_shapes(desc)
    _check_pool(k_pool, ks, desc, "k_pool")
    _check_pool(v_pool, vs, desc, "v_pool")
    _check_meta(meta, desc)
    _check_tables(block_tables, context_lens)
    S, Hq, D = q.shape
    if D != desc.head_dim or tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("q / out shapes or dtypes do not match")
    if not (q.is_contiguous() and out.is_contiguous()) or block_tables.shape[0] != S:
        raise ValueError("q and out must be contiguous, one table row per sequence")
    with _on(stream):
        ws, wsb = _quest_ws(workspace, desc, q, block_tables, max_context_len, partition_size,
                            budget_blocks)
        _check(lib.pkv_quest_decode(_ptr(q), dtype_code(q), _ptr(k_pool), _ptr(v_pool),
                                    _ptr(meta), ctypes.byref(desc), _ptr(block_tables),
                                    int(block_tables.shape[1]), _ptr(context_lens), S, Hq,
                                    float(scale), _ptr(out), int(max_context_len),
                                    int(partition_size), int(budget_blocks), _ptr(ws), wsb,
                                    _stream(stream), int(impl)))
    return out


# ---------------------------------------------------------------------------- measurement aid

def read_probe(buf, tile_bytes: int, tile_ids, num_tiles: int, sink, workgroups: int = 2048,
               stream=None) -> None:
    """Plain HBM read of ``num_tiles`` tiles of ``buf`` (a device tensor): tile i at
    ``tile_ids[i] * tile_bytes`` (device int64), or tiles 0.. in order when ``tile_ids`` is
    None.  ``sink`` is a device tensor of ``workgroups * 64`` 32-bit words (one per lane of
    the one-wave workgroups)."""
    torch = _torch()
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink.numel() * sink.element_size() < workgroups * 64 * 4 or not sink.is_cuda:
        raise ValueError(f"sink must be a device tensor of at least {workgroups * 64} words")
    if tile_ids is not None:
        if not tile_ids.is_cuda or tile_ids.dtype != torch.int64 or tile_ids.numel() < num_tiles:
            raise ValueError("tile_ids must be a device int64 tensor of num_tiles ids")
    _check(lib.pkv_read_probe(_ptr(buf), int(buf.numel() * buf.element_size()), int(tile_bytes),
                              _ptr(tile_ids) if tile_ids is not None else 0, int(num_tiles),
                              _ptr(sink), int(workgroups), _stream(stream)))


# ---------------------------------------------------------------------------- host side

def _np_ptr(a: np.ndarray, typ):
    return a.ctypes.data_as(ctypes.POINTER(typ))


class BlockManager:
    """Refcounted block allocator (C++): free list, block tables, fork, copy-on-write."""

    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None):
        if free_order is None:
            h = lib.pkv_bm_create(num_blocks, block_size, None, 0)
        else:
            fo = np.ascontiguousarray(free_order, dtype=np.int32)
            h = lib.pkv_bm_create(num_blocks, block_size, _np_ptr(fo, ctypes.c_int32), len(fo))
        if not h:
            raise PagedKVError(PKV_E_INVAL, lib.pkv_last_error().decode())
        self._h = ctypes.c_void_p(h)
        # kept on the instance: at interpreter shutdown the module's globals (lib among
        # them) may already be gone when __del__ runs
        self._destroy = lib.pkv_bm_destroy
        self.num_blocks = num_blocks
        self.block_size = block_size

    def __del__(self):
        h = getattr(self, "_h", None)
        destroy = getattr(self, "_destroy", None)
        if h is not None and h.value and destroy is not None:
            destroy(h)
            self._h = None

    def add_seq(self, seq: int, num_tokens: int) -> None:
        _check(lib.pkv_bm_add_seq(self._h, seq, num_tokens))

    def fork(self, parent: int, child: int) -> None:
        _check(lib.pkv_bm_fork(self._h, parent, child))

    def append(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        slot, src, dst = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib.pkv_bm_append(self._h, seq, ctypes.byref(slot), ctypes.byref(src),
                                 ctypes.byref(dst)))
        return slot.value, ((src.value, dst.value) if src.value >= 0 else None)

    def append_batch(self, seqs: Iterable[int]) -> Tuple[np.ndarray, np.ndarray]:
        s = np.ascontiguousarray(list(seqs), dtype=np.int64)
        slots = np.empty(len(s), dtype=np.int64)
        pairs = np.empty((max(1, len(s)), 2), dtype=np.int64)
        n = ctypes.c_int32()
        _check(lib.pkv_bm_append_batch(self._h, _np_ptr(s, ctypes.c_int64), len(s),
                                       _np_ptr(slots, ctypes.c_int64),
                                       _np_ptr(pairs, ctypes.c_int64), ctypes.byref(n)))
        return slots, pairs[: n.value].copy()

    def extend(self, seq: int, n: int) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
        slots = np.empty(max(1, n), dtype=np.int64)
        src, dst = ctypes.c_int64(), ctypes.c_int64()
        _check(lib.pkv_bm_extend(self._h, seq, n, _np_ptr(slots, ctypes.c_int64),
                                 ctypes.byref(src), ctypes.byref(dst)))
        return slots[:n].copy(), ([(src.value, dst.value)] if src.value >= 0 else [])

    def free_seq(self, seq: int) -> None:
        _check(lib.pkv_bm_free_seq(self._h, seq))

    def slots(self, seq: int, start: int, n: int) -> np.ndarray:
        out = np.empty(max(1, n), dtype=np.int64)
        _check(lib.pkv_bm_slots(self._h, seq, start, n, _np_ptr(out, ctypes.c_int64)))
        return out[:n].copy()

    def block_tables(self, seqs: Sequence[int], max_blocks: int,
                     out_tables: Optional[np.ndarray] = None,
                     out_lens: Optional[np.ndarray] = None):
        s = np.ascontiguousarray(list(seqs), dtype=np.int64)
        tables = out_tables if out_tables is not None else np.empty((len(s), max_blocks), np.int32)
        lens = out_lens if out_lens is not None else np.empty(len(s), np.int32)
        _check(lib.pkv_bm_block_tables(self._h, _np_ptr(s, ctypes.c_int64), len(s),
                                       _np_ptr(tables, ctypes.c_int32), max_blocks,
                                       _np_ptr(lens, ctypes.c_int32)))
        return tables, lens

    def stats(self) -> dict:
        st = BmStats()
        _check(lib.pkv_bm_stats(self._h, ctypes.byref(st)))
        return {f: getattr(st, f) for f, _ in BmStats._fields_}

    def refcount(self, block: int) -> int:
        return int(lib.pkv_bm_refcount(self._h, block))

    def seq_len(self, seq: int) -> int:
        return int(lib.pkv_bm_seq_len(self._h, seq))

    def free_list(self) -> List[int]:
        n = lib.pkv_bm_free_list(self._h, None, 0)
        out = np.empty(max(1, n), dtype=np.int32)
        lib.pkv_bm_free_list(self._h, _np_ptr(out, ctypes.c_int32), n)
        return out[:n].tolist()

    # -- prefix caching ------------------------------------------------------
    def set_prefix_caching(self, enable: bool = True) -> None:
        _check(lib.pkv_bm_set_prefix_caching(self._h, 1 if enable else 0))

    @staticmethod
    def _tokens(tokens) -> np.ndarray:
        return np.ascontiguousarray(np.asarray(tokens, dtype=np.int64).astype(np.int32))

    def lookup(self, tokens) -> int:
        t = self._tokens(tokens)
        out = ctypes.c_int64()
        _check(lib.pkv_bm_lookup(self._h, _np_ptr(t, ctypes.c_int32), len(t), ctypes.byref(out)))
        return out.value

    def add_seq_tokens(self, seq: int, tokens) -> int:
        """Admit a sequence with its tokens; returns how many leading tokens were cached."""
        t = self._tokens(tokens)
        out = ctypes.c_int64()
        _check(lib.pkv_bm_add_seq_tokens(self._h, seq, _np_ptr(t, ctypes.c_int32), len(t),
                                         ctypes.byref(out)))
        return out.value

    def append_batch_tokens(self, seqs: Iterable[int], tokens) -> Tuple[np.ndarray, np.ndarray]:
        s = np.ascontiguousarray(list(seqs), dtype=np.int64)
        t = self._tokens(tokens)
        if len(t) != len(s):
            raise ValueError("one token per sequence")
        slots = np.empty(len(s), dtype=np.int64)
        pairs = np.empty((max(1, len(s)), 2), dtype=np.int64)
        n = ctypes.c_int32()
        _check(lib.pkv_bm_append_batch_tokens(self._h, _np_ptr(s, ctypes.c_int64),
                                              _np_ptr(t, ctypes.c_int32), len(s),
                                              _np_ptr(slots, ctypes.c_int64),
                                              _np_ptr(pairs, ctypes.c_int64), ctypes.byref(n)))
        return slots, pairs[: n.value].copy()

    def extend_tokens(self, seq: int, tokens) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
        t = self._tokens(tokens)
        n = len(t)
        slots = np.empty(max(1, n), dtype=np.int64)
        src, dst = ctypes.c_int64(), ctypes.c_int64()
        _check(lib.pkv_bm_extend_tokens(self._h, seq, _np_ptr(t, ctypes.c_int32), n,
                                        _np_ptr(slots, ctypes.c_int64), ctypes.byref(src),
                                        ctypes.byref(dst)))
        return slots[:n].copy(), ([(src.value, dst.value)] if src.value >= 0 else [])

    def cache_stats(self) -> dict:
        out = np.zeros(4, dtype=np.int64)
        _check(lib.pkv_bm_cache_stats(self._h, _np_ptr(out, ctypes.c_int64)))
        return {"cached_blocks": int(out[0]), "evictable_blocks": int(out[1]),
                "hit_tokens": int(out[2]), "query_tokens": int(out[3])}

    # -- swapping ------------------------------------------------------------
    def set_host_pool(self, num_host_blocks: int) -> None:
        _check(lib.pkv_bm_set_host_pool(self._h, num_host_blocks))

    def seq_blocks(self, seq: int) -> List[int]:
        n = lib.pkv_bm_seq_blocks(self._h, seq, None, 0)
        if n < 0:
            raise PagedKVError(PKV_E_INVAL, f"unknown sequence {seq}")
        out = np.empty(max(1, n), dtype=np.int32)
        lib.pkv_bm_seq_blocks(self._h, seq, _np_ptr(out, ctypes.c_int32), n)
        return out[:n].tolist()

    def _swap(self, fn, seqs) -> np.ndarray:
        s = np.ascontiguousarray(list(seqs), dtype=np.int64)
        cap = sum(max(0, lib.pkv_bm_seq_blocks(self._h, int(x), None, 0)) for x in s)
        pairs = np.empty((max(1, cap), 2), dtype=np.int64)
        n = ctypes.c_int32()
        _check(fn(self._h, _np_ptr(s, ctypes.c_int64), len(s), _np_ptr(pairs, ctypes.c_int64),
                  cap, ctypes.byref(n)))
        return pairs[: n.value].copy()

    def swap_out(self, seqs) -> np.ndarray:
        """Move a set of sequences to the host pool; returns (device, host) pairs to copy."""
        return self._swap(lib.pkv_bm_swap_out, seqs)

    def swap_in(self, seqs) -> np.ndarray:
        """Move swapped-out sequences back; returns (host, device) pairs to copy."""
        return self._swap(lib.pkv_bm_swap_in, seqs)

    def swap_stats(self) -> dict:
        out = np.zeros(3, dtype=np.int64)
        _check(lib.pkv_bm_swap_stats(self._h, _np_ptr(out, ctypes.c_int64)))
        return {"host_free_blocks": int(out[0]), "host_blocks": int(out[1]),
                "swapped_seqs": int(out[2])}

    def block_fills(self, seqs) -> Tuple[np.ndarray, np.ndarray]:
        """(distinct blocks, filled slots) of the sequences' blocks (pkv_bm_block_fills)."""
        s = np.ascontiguousarray(list(seqs), dtype=np.int64)
        n = int(lib.pkv_bm_block_fills(self._h, _np_ptr(s, ctypes.c_int64), len(s), None, None, 0))
        _check(min(n, 0))
        blocks = np.empty(max(1, n), np.int32)
        fills = np.empty(max(1, n), np.int32)
        m = int(lib.pkv_bm_block_fills(self._h, _np_ptr(s, ctypes.c_int64), len(s),
                                       _np_ptr(blocks, ctypes.c_int32),
                                       _np_ptr(fills, ctypes.c_int32), n))
        _check(min(m, 0))
        return blocks[:n].copy(), fills[:n].copy()

    def host_refcount(self, block: int) -> int:
        return int(lib.pkv_bm_host_refcount(self._h, block))

    def host_free_list(self) -> List[int]:
        n = lib.pkv_bm_host_free_list(self._h, None, 0)
        out = np.empty(max(1, n), dtype=np.int32)
        lib.pkv_bm_host_free_list(self._h, _np_ptr(out, ctypes.c_int32), n)
        return out[:n].tolist()

    def evictable_list(self) -> List[int]:
        n = lib.pkv_bm_evictable_list(self._h, None, 0)
        out = np.empty(max(1, n), dtype=np.int32)
        lib.pkv_bm_evictable_list(self._h, _np_ptr(out, ctypes.c_int32), n)
        return out[:n].tolist()
