"""Paged KV cache: sizes, byte layout, insertion through a slot mapping, gather.

Test infrastructure only (see the package docstring).

Sources on the pages: page sizes 32 and 64 ("Laguna FP8 KV -- replicated
embedding win, page-32 build, and host boundary", section "Page-32 attention
experiment"); the per-token payload 2 * 8 * 128 = 2,048 values, 4,096 B in BF16
and 2,048 B in FP8, and the 48-layer / draft / TP4 aggregates ("Laguna S 2.1
KV-cache precision decision", section "BF16 versus FP8 in concrete terms").
The pages name no slot mapping, block table or byte layout: those are the
library's documented interface (include/fkv.h), which this module restates
independently:

  element size   E = 1 byte (FP8 E4M3FN) or 2 bytes (BF16 bit pattern)
  K pool         index(blk, h, o, d) = ((blk*Hkv + h)*bs + o)*128 + d
  V pool         index(blk, h, o, d) = (blk*Hkv + h)*bs*128 + (o//8)*1024 + d*8 + o%8
  token slot     s -> blk = s // bs, o = s % bs; negative slots are skipped

(index counts elements of size E). Each (block, head) owns one contiguous
bs*128-element slab in each pool; within a V slab every group of 8 keys is
stored dimension-major.
"""

import numpy as np

from . import e4m3

HEAD_DIM = 128
FP8 = "fp8_e4m3fn"
BF16 = "bf16"


def elem_bytes(cache_dtype):
    return {FP8: 1, BF16: 2}[cache_dtype]


def payload_bytes_per_token(num_kv_heads, cache_dtype, head_dim=HEAD_DIM):
    """K + V payload of one token in one layer: 2 * Hkv * head_dim elements."""
    return 2 * num_kv_heads * head_dim * elem_bytes(cache_dtype)


def pool_bytes(num_blocks, block_size, num_kv_heads, cache_dtype, head_dim=HEAD_DIM):
    """Size of ONE pool (K or V)."""
    return num_blocks * num_kv_heads * block_size * head_dim * elem_bytes(cache_dtype)


def k_index(blk, h, o, d, block_size, num_kv_heads):
    return ((blk * num_kv_heads + h) * block_size + o) * HEAD_DIM + d


def v_index(blk, h, o, d, block_size, num_kv_heads):
    return (blk * num_kv_heads + h) * block_size * HEAD_DIM + (o // 8) * (8 * HEAD_DIM) + d * 8 + (o % 8)


def new_pools(num_blocks, block_size, num_kv_heads, cache_dtype, fill=0):
    n = num_blocks * num_kv_heads * block_size * HEAD_DIM
    dt = np.uint8 if cache_dtype == FP8 else np.uint16
    return np.full(n, fill, dtype=dt), np.full(n, fill, dtype=dt)


def insert(k_pool, v_pool, k_bits, v_bits, slot_mapping, k_scale, v_scale, block_size, num_kv_heads, cache_dtype):
    """Write tokens [T, Hkv, 128] (BF16 bit patterns) into the pools.

    FP8 cache: the stored bytes are e4m3.quantize(x, scale) per element.
    BF16 cache: the BF16 bit patterns are stored unchanged (scales unused).
    """
    k_bits = np.asarray(k_bits, dtype=np.uint16)
    v_bits = np.asarray(v_bits, dtype=np.uint16)
    T = k_bits.shape[0]
    assert k_bits.shape == (T, num_kv_heads, HEAD_DIM) and v_bits.shape == k_bits.shape
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    if not np.any(keep):
        return
    slots = slots[keep]
    if cache_dtype == FP8:
        kc = e4m3.quantize(k_bits[keep], k_scale)
        vc = e4m3.quantize(v_bits[keep], v_scale)
    else:
        kc, vc = k_bits[keep], v_bits[keep]
    blk = (slots // block_size)[:, None, None]
    o = (slots % block_size)[:, None, None]
    h = np.arange(num_kv_heads)[None, :, None]
    d = np.arange(HEAD_DIM)[None, None, :]
    k_pool[k_index(blk, h, o, d, block_size, num_kv_heads)] = kc
    v_pool[v_index(blk, h, o, d, block_size, num_kv_heads)] = vc


def gather(pool, which, block_table_row, seq_len, block_size, num_kv_heads):
    """Logical [seq_len, Hkv, 128] view of one sequence's cache elements.

    Key j lives in physical block block_table_row[j // bs] at offset j % bs.
    """
    j = np.arange(seq_len)
    blk = np.asarray(block_table_row, dtype=np.int64)[j // block_size][:, None, None]
    o = (j % block_size)[:, None, None]
    h = np.arange(num_kv_heads)[None, :, None]
    d = np.arange(HEAD_DIM)[None, None, :]
    idx = (k_index if which == "k" else v_index)(blk, h, o, d, block_size, num_kv_heads)
    return pool[idx]


def dequantize_elements(elems, scale, cache_dtype):
    """float64 K/V values of stored elements: decode * scale (FP8) or the BF16 value."""
    if cache_dtype == FP8:
        return e4m3.dequantize(elems, scale)
    return e4m3.bf16_bits_to_f32(elems).astype(np.float64)
