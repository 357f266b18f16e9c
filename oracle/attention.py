"""Decode attention over the dequantised cache, dense, float64.

Test infrastructure only (see the package docstring).

What the pages fix: exact q1 and M12 paged attention ("Laguna S 2.1 INT4 --
calibrated FP8 KV on Intel B70", section "Initial optimization order"); a
width-12 verify window (section Contract); q=18, kv=2, head size 128 with global
(-1,-1) and sliding (64,0) windows ("Laguna FP8 KV -- replicated embedding win,
page-32 build, and host boundary", section "Page-32 attention experiment"); 36
sliding-window layers with a 512-token window and 12 global layers ("Laguna S
2.1 KV-cache precision decision", section "BF16 versus FP8 in concrete terms");
exactness is judged against an FP8 teacher, so the reference is attention over
the dequantised FP8 values, never over the BF16 originals (Contract, and
"Recommendation" on the precision-decision page).

Readings taken where the pages are silent:
  * seq_len L counts the cached tokens after the M new ones are inserted; query
    row i (0 <= i < M) sits at absolute position p_i = L - M + i;
  * key j is visible to row i iff lo_i <= j <= p_i with lo_i = 0 for global
    attention (window_left < 0) and lo_i = max(0, p_i - window_left) otherwise
    (flash-attention (left, right=0) convention: a 512-token window is
    window_left = 511);
  * GQA groups are contiguous: query head h reads KV head h // (Hq // Hkv);
  * scores s_j = softmax_scale * <q, k_j>, softmax over the visible keys, and
    out = sum_j softmax_j * v_j. softmax_scale is an explicit argument
    (1/sqrt(128) in every workload here).
"""

import numpy as np


def visible_range(seq_len, q_len, i, window_left):
    """[lo, hi] inclusive key range for query row i."""
    p = seq_len - q_len + i
    lo = 0 if window_left < 0 else max(0, p - window_left)
    return lo, p


def decode_attention(q, k, v, q_len, window_left, softmax_scale):
    """One sequence. q [M, Hq, D], k and v [L, Hkv, D] (float64) -> out [M, Hq, D].

    Row-by-row: for each query row and head, softmax over its visible keys of
    its KV group, then the weighted sum of V.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    M, Hq, D = q.shape
    L, Hkv, _ = k.shape
    assert M == q_len and L >= M and Hq % Hkv == 0
    G = Hq // Hkv
    out = np.empty((M, Hq, D), dtype=np.float64)
    for i in range(M):
        lo, hi = visible_range(L, M, i, window_left)
        for h in range(Hq):
            g = h // G
            s = softmax_scale * (k[lo:hi + 1, g, :] @ q[i, h, :])
            w = np.exp(s - s.max())
            out[i, h, :] = (w @ v[lo:hi + 1, g, :]) / w.sum()
    return out


def paged_decode(k_pool, v_pool, q_bits, block_table, seq_lens, q_len, window_left, softmax_scale,
                 k_scale, v_scale, block_size, num_kv_heads, cache_dtype):
    """Decode attention for a batch straight from the paged pools.

    q_bits [B, M, Hq, 128] BF16 bit patterns; block_table [B, max_blocks];
    seq_lens [B]. Returns float64 [B, M, Hq, 128].
    """
    from . import e4m3, paged
    B = q_bits.shape[0]
    outs = []
    for b in range(B):
        L = int(seq_lens[b])
        kq = paged.gather(k_pool, "k", block_table[b], L, block_size, num_kv_heads)
        vq = paged.gather(v_pool, "v", block_table[b], L, block_size, num_kv_heads)
        k = paged.dequantize_elements(kq, k_scale, cache_dtype)
        v = paged.dequantize_elements(vq, v_scale, cache_dtype)
        q = e4m3.bf16_bits_to_f32(q_bits[b]).astype(np.float64)
        outs.append(decode_attention(q, k, v, q_len, window_left, softmax_scale))
    return np.stack(outs) if outs else np.zeros((0,) + tuple(q_bits.shape[1:]), dtype=np.float64)
