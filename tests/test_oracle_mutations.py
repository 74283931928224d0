"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

A pin set that lets a dropped term, a wrong index, a wrong sign or a
transposed operand through would not pin anything; every mutation below must
make at least one of the listed checks fail.
"""
import numpy as np
import pytest

import pins
from oracle import allocator as oalloc
from oracle import attention as oattn
from oracle import cache as ocache
from oracle import codec


def _fails(checks):
    for c in checks:
        try:
            c()
        except Exception:
            return True
    return False


def _attend_no_scale(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    z = K @ q
    p = np.exp(z - z.max())
    return (p / p.sum()) @ V


def _attend_drop_last(q, K, V, scale):
    K, V = K[:-1], V[:-1]
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    z = scale * (K @ q)
    p = np.exp(z - z.max())
    return (p / p.sum()) @ V


def _attend_no_normalise(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    z = scale * (K @ q)
    return np.exp(z - z.max()) @ V


def _attend_sign(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    z = -scale * (K @ q)
    p = np.exp(z - z.max())
    return (p / p.sum()) @ V


def _gather_keys_offset(k_pool, table, ctx, kv_head):
    B = k_pool.shape[2]
    t = np.arange(ctx)
    return k_pool[np.asarray(table)[t // B], kv_head, (t + 1) % B, :]


def _gather_keys_wrong_block(k_pool, table, ctx, kv_head):
    B = k_pool.shape[2]
    t = np.arange(ctx)
    return k_pool[np.asarray(table)[t % len(table)] if len(table) else [], kv_head, t % B, :]


def _gather_values_transposed(v_pool, table, ctx, kv_head):
    B = v_pool.shape[3]
    t = np.arange(ctx)
    n, hkv, d, b = v_pool.shape
    vp = v_pool.reshape(n, hkv, b, d)          # the value block's memory read as [B, D]
    return vp[np.asarray(table)[t // B], kv_head, t % B, :]


def _e4m3_table_fnuz():
    vals = []
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 0xF, code & 7
        vals.append(s * m * 2.0 ** -10 if e == 0 else s * (1 + m / 8) * 2.0 ** (e - 8))
    return np.array(vals)


def _encode_ties_away(y):
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    mags = codec.E4M3_TABLE[:0x7F]
    hi = np.clip(np.searchsorted(mags, a), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    code = np.where(mags[hi] - a <= a - mags[lo], hi, lo)
    code = np.where(a > 448, 0x7E, code).astype(np.uint8)
    return code | (np.signbit(y).astype(np.uint8) << np.uint8(7))


def _encode_truncate(y):
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    mags = codec.E4M3_TABLE[:0x7F]
    code = np.clip(np.searchsorted(mags, a, side="right") - 1, 0, 0x7E).astype(np.uint8)
    return code | (np.signbit(y).astype(np.uint8) << np.uint8(7))


def _bf16_to_f32_shift15(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(15)).view(np.float32)


def _bf16_to_f32_by_value(bits):
    return np.asarray(bits, dtype=np.uint16).astype(np.float32)


def _bf16_to_f32_low_half(bits):
    # the 16 bits placed in the low half of the word (a byte-order / view mistake)
    return np.asarray(bits, dtype=np.uint16).astype(np.uint32).view(np.float32)


class _PopTail(oalloc.BlockAllocator):
    def _pop(self):
        b = self.free.pop()
        self.ref[b] = 1
        return b


def _append_no_cow(self, seq):
    pos = self.lens[seq]
    table = self.tables[seq]
    if pos % self.block_size == 0:
        table.append(self._pop())
    slot = table[pos // self.block_size] * self.block_size + pos % self.block_size
    self.lens[seq] = pos + 1
    return slot, None


def _append_cow_no_decrement(self, seq):
    pos = self.lens[seq]
    table = self.tables[seq]
    pair = None
    if pos % self.block_size == 0:
        table.append(self._pop())
    elif self.ref[table[-1]] > 1:
        old, new = table[-1], self._pop()
        table[-1] = new
        pair = (old, new)
    slot = table[pos // self.block_size] * self.block_size + pos % self.block_size
    self.lens[seq] = pos + 1
    return slot, pair


def _free_to_head(self, seq):
    for b in self.tables.pop(seq):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.appendleft(b)
    del self.lens[seq]


def _copy_blocks_k_only(k_pool, v_pool, pairs):
    for src, dst in ocache.check_pairs(pairs, k_pool.shape[0]):
        k_pool[dst] = k_pool[src]


def _reshape_v_untransposed(k_pool, v_pool, k, v, slot_mapping, in_dtype, kv_dtype,
                            k_scale=1.0, v_scale=1.0):
    B = k_pool.shape[2]
    ke = ocache.encode(k, in_dtype, kv_dtype, k_scale)
    ve = ocache.encode(v, in_dtype, kv_dtype, v_scale)
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        b, p = divmod(int(slot), B)
        k_pool[b, :, p, :] = ke[i]
        flat = v_pool[b].reshape(v_pool.shape[1], -1)
        flat[:, p * v_pool.shape[2]:(p + 1) * v_pool.shape[2]] = ve[i]


MUTATIONS = {
    "attention without scale": (oattn, "attend", _attend_no_scale,
                                [pins.check_attention_vs_sdpa]),
    "attention drops last token": (oattn, "attend", _attend_drop_last,
                                   [pins.check_attention_vs_sdpa, pins.check_single_token_context]),
    "softmax not normalised": (oattn, "attend", _attend_no_normalise,
                               [pins.check_attention_vs_sdpa, pins.check_identical_keys]),
    "logit sign flipped": (oattn, "attend", _attend_sign, [pins.check_attention_vs_sdpa]),
    "GQA heads interleaved instead of grouped": (
        oattn, "kv_head_of", lambda h, hq, hkv: h % hkv,
        [pins.check_attention_vs_sdpa, pins.check_gqa_is_repeated_mha]),
    "gather reads the next slot": (oattn, "gather_keys", _gather_keys_offset,
                                   [pins.check_glossary_example, pins.check_attention_vs_sdpa]),
    "gather indexes the table by t % len": (oattn, "gather_keys", _gather_keys_wrong_block,
                                            [pins.check_glossary_example,
                                             pins.check_attention_vs_sdpa]),
    "values read with the key layout": (oattn, "gather_values", _gather_values_transposed,
                                        [pins.check_attention_vs_sdpa,
                                         pins.check_single_token_context]),
    "value cache written untransposed": (ocache, "reshape_and_cache", _reshape_v_untransposed,
                                         [pins.check_copy_on_write,
                                          pins.check_attention_vs_sdpa,
                                          pins.check_cache_write_only_touches_slots]),
    "fp8 decoded with the FNUZ bias": (codec, "E4M3_TABLE", _e4m3_table_fnuz(),
                                       [pins.check_e4m3_decode]),
    "bf16 widened with a 15-bit shift": (codec, "bf16_to_f32", _bf16_to_f32_shift15,
                                         [pins.check_bf16_widening, pins.check_fp8_cache_encode,
                                          pins.check_attention_vs_sdpa]),
    "bf16 patterns converted as integers": (codec, "bf16_to_f32", _bf16_to_f32_by_value,
                                            [pins.check_bf16_widening,
                                             pins.check_fp8_cache_encode,
                                             pins.check_attention_vs_sdpa]),
    "bf16 patterns in the low half of the word": (codec, "bf16_to_f32", _bf16_to_f32_low_half,
                                                  [pins.check_bf16_widening,
                                                   pins.check_fp8_cache_encode,
                                                   pins.check_attention_vs_sdpa]),
    "fp8 ties rounded away from zero": (codec, "e4m3_encode_f32", _encode_ties_away,
                                        [pins.check_e4m3_encode]),
    "fp8 truncated": (codec, "e4m3_encode_f32", _encode_truncate, [pins.check_e4m3_encode]),
    "allocator pops the tail of the free list": (oalloc, "BlockAllocator", _PopTail,
                                                 [pins.check_glossary_example,
                                                  pins.check_optiverse_block_table]),
    "no copy on write": (oalloc.BlockAllocator, "append", _append_no_cow,
                         [pins.check_copy_on_write, pins.check_sharing_invariance]),
    "copy on write keeps the old count": (oalloc.BlockAllocator, "append",
                                          _append_cow_no_decrement, [pins.check_copy_on_write]),
    "freed blocks pushed to the head": (oalloc.BlockAllocator, "free_seq", _free_to_head,
                                        [pins.check_optiverse_block_table]),
    "copy_blocks forgets the values": (ocache, "copy_blocks", _copy_blocks_k_only,
                                       [pins.check_copy_blocks_invariant,
                                        pins.check_copy_on_write]),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    target, attr, value, checks = MUTATIONS[name]
    if target is codec and attr == "E4M3_TABLE":
        monkeypatch.setattr(codec, "_MAGNITUDES", value[:0x7F])
    monkeypatch.setattr(target, attr, value)
    assert _fails(checks), f"no pin caught: {name}"


def test_unmutated_checks_pass():
    for c in pins.ALL:
        c()
