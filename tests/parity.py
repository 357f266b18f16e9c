"""Oracle references for synthetic layers and the parity metric.

The attention gate is the row-normalised error: for every (sequence, query row,
query head) row, max_d |o_gpu - o_ref| / max_d |o_ref|, and the largest value
over all rows must stay <= 2e-3 (fp32 accumulation on the GPU, float64 in the
oracle). Inserted cache bytes must match bit for bit.
"""

import numpy as np

from oracle import attention, e4m3, paged

ATTN_TOL = 2e-3
POISON = {"fp8_e4m3fn": 0x7F, "bf16": 0xFFFF}


def logical_kv(lay, b, t1=None, heads=None):
    """float64 K, V [L, Hkv', 128] of sequence b as the oracle dequantises them."""
    L = int(lay.seq_lens[b]) if t1 is None else t1
    k, v = lay.kv_bits(b, 0, L)
    if heads is not None:
        k, v = k[:, heads], v[:, heads]
    if lay.cache_dtype == paged.FP8:
        return (e4m3.dequantize(e4m3.quantize(k, lay.k_scale), lay.k_scale),
                e4m3.dequantize(e4m3.quantize(v, lay.v_scale), lay.v_scale))
    return (e4m3.bf16_bits_to_f32(k).astype(np.float64), e4m3.bf16_bits_to_f32(v).astype(np.float64))


def q_f64(lay, b):
    return e4m3.bf16_bits_to_f32(lay.q_bits()[b]).astype(np.float64)


def reference(lay, b, kv_heads=None):
    """Oracle output of sequence b: [M, Hq, 128] float64 (NaN rows for heads not computed)."""
    G = lay.num_q_heads // lay.num_kv_heads
    kvh = list(range(lay.num_kv_heads)) if kv_heads is None else list(kv_heads)
    k, v = logical_kv(lay, b, heads=kvh)
    q = q_f64(lay, b)
    out = np.full(q.shape, np.nan)
    for j, g in enumerate(kvh):
        sl = slice(g * G, (g + 1) * G)
        out[:, sl] = attention.decode_attention(q[:, sl], k[:, j:j + 1], v[:, j:j + 1], lay.q_len,
                                                lay.window_left, lay.softmax_scale)
    return out


def row_errors(gpu, ref):
    """Row-normalised errors over the last axis, ignoring rows where ref is NaN."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ok = ~np.isnan(ref).any(axis=-1)
    num = np.abs(gpu - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    err = np.where(ok, num / den, 0.0)
    bad_nonfinite = ok & ~np.isfinite(gpu).all(axis=-1)
    return np.where(bad_nonfinite, np.inf, err)


def oracle_pools(lay, seqs=None):
    """Oracle pools after inserting every token of the listed sequences (poisoned elsewhere)."""
    kp, vp = paged.new_pools(lay.num_blocks, lay.block_size, lay.num_kv_heads, lay.cache_dtype,
                             fill=POISON[lay.cache_dtype])
    for b in (range(lay.num_seqs) if seqs is None else seqs):
        L = int(lay.seq_lens[b])
        k, v = lay.kv_bits(b, 0, L)
        paged.insert(kp, vp, k, v, lay.slots(b, 0, L), lay.k_scale, lay.v_scale, lay.block_size,
                     lay.num_kv_heads, lay.cache_dtype)
    return kp, vp
