"""Oracle references for synthetic layers and the parity metric.

The attention gate is the row-normalised error: for every (sequence, query row,
query head) row, max_d |o_gpu - o_ref| / max_d |o_ref|, and the largest value
over all rows must stay <= 2e-3 (fp32 accumulation on the GPU, float64 in the
oracle). Inserted cache bytes must match bit for bit; after the Q/K norm + RoPE step,
bit for bit wherever the float64 value is not within the float32 error band of a BF16
rounding boundary, and otherwise one of the two roundings (norm_rope_bounds below).
"""

import numpy as np

from oracle import attention, e4m3, normrope, paged

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


# ---- Q/K RMSNorm + RoPE: what a float32 evaluation may return ------------------------------
# The kernel evaluates the norm and the rotation in float32 (fixed order, every operation
# rounded once); the oracle evaluates them in float64 and rounds to BF16 once. The two agree
# bit for bit except where an exact value lies so close to a BF16 rounding boundary that the
# float32 error can cross it. These bands bound the float32 error of one element:
#   y = x w / sqrt(mean(x^2) + eps): 128 squares summed (at most 12 roundings deep), one add,
#     one square root, one division, two products: below 16 units of 2^-24 relative;
#   z = y_d c - y_e s: two products and one difference: below 3 units of 2^-24 times
#     (|y_d c| + |y_e s|).
Y_BAND = 16 * 2.0 ** -24
Z_BAND = 3 * 2.0 ** -24


def _bf16_neighbours(r):
    """(next BF16 value below, next above) of BF16 values r (float64 arrays)."""
    bits = normrope.bf16_bits(r).astype(np.int32)
    up = np.where(r >= 0, bits + 1, bits - 1)     # magnitude order reverses for negative values
    dn = np.where(r > 0, bits - 1, bits + 1)
    up = np.where(r == 0, 0x0001, up)
    dn = np.where(r == 0, 0x8001, dn)
    f = lambda b: normrope.bf16_f32(b.astype(np.uint16)).astype(np.float64)
    return f(dn), f(up)


def norm_rope_bounds(x_bits, w_bits, eps, cos_sin, positions):
    """Per output element of fkv_qk_norm_rope_insert: the interval [lo, hi] (float64, BF16
    values) a float32 evaluation can round to, and exact = (lo == hi).

    Each normalised component y may round to either BF16 neighbour of a rounding boundary
    when the float64 value lies within Y_BAND of it; the rotation takes every combination of
    the admissible y of its pair, widened by Z_BAND, and rounds the ends once. Padding rows
    (position outside the table) are exactly zero."""
    nr = normrope
    valid, cos, sin = nr.table_rows(cos_sin, positions)
    y64 = nr.rmsnorm_f64(x_bits, w_bits, eps)
    yb = nr.bf16_round(y64)
    dn, up = _bf16_neighbours(yb)
    other = np.where(y64 > yb, up, dn)
    near = (y64 != yb) & (np.abs(y64 - (yb + other) / 2.0) <= Y_BAND * np.abs(y64))
    alt = np.where(near, other, yb)
    c = cos[:, None, :].astype(np.float64)
    s = sin[:, None, :].astype(np.float64)
    lo_y, hi_y = (yb[..., :nr.HALF], alt[..., :nr.HALF]), (yb[..., nr.HALF:], alt[..., nr.HALF:])
    zl = [a * c - b * s for a in lo_y for b in hi_y]
    zh = [b * c + a * s for a in lo_y for b in hi_y]
    mag_l = np.maximum.reduce([np.abs(a * c) + np.abs(b * s) for a in lo_y for b in hi_y])
    mag_h = np.maximum.reduce([np.abs(b * c) + np.abs(a * s) for a in lo_y for b in hi_y])
    zmin = np.concatenate([np.minimum.reduce(zl) - Z_BAND * mag_l, np.minimum.reduce(zh) - Z_BAND * mag_h], -1)
    zmax = np.concatenate([np.maximum.reduce(zl) + Z_BAND * mag_l, np.maximum.reduce(zh) + Z_BAND * mag_h], -1)
    lo, hi = nr.bf16_round(zmin), nr.bf16_round(zmax)
    lo[~valid] = 0.0
    hi[~valid] = 0.0
    return lo, hi, lo == hi


def check_bf16_within(got_bits, lo, hi, label):
    """Every BF16 element lies in its admissible interval; returns the number of elements
    whose interval holds more than one value and the number that differ from lo."""
    g = normrope.bf16_f32(got_bits).astype(np.float64)
    bad = ~((g >= lo) & (g <= hi))
    assert not bad.any(), (f"{label}: {int(bad.sum())} elements outside their admissible BF16 interval, first at "
                           f"{np.argwhere(bad)[0]}: got {g[bad][0]!r}, interval [{lo[bad][0]!r}, {hi[bad][0]!r}]")
    return int((lo != hi).sum()), int((g != lo).sum())


def check_norm_rope_k_pool(gk, kp_ref, lay, st, lo, hi, label):
    """GPU K pool against the oracle's: bytes outside the new tokens' K' rows equal the oracle;
    inside them each element is a code (FP8) or BF16 value admissible for its interval: the
    plain insert of any BF16 K' in [lo, hi] (the E4M3 encoding of x / k_scale is monotone)."""
    pg = paged
    valid = (st.positions >= 0) & (st.positions < st.cos_sin.shape[0]) & (st.slot_mapping >= 0) \
        & (st.slot_mapping < lay.num_blocks * lay.block_size)
    T, H = st.k_bits.shape[0], lay.num_kv_heads
    blk, off = np.divmod(st.slot_mapping.astype(np.int64), lay.block_size)
    idx = pg.k_index(blk[:, None, None], np.arange(H)[None, :, None], off[:, None, None],
                     np.arange(128)[None, None, :], lay.block_size, H)
    sel = np.broadcast_to(valid[:, None, None], idx.shape)
    mask = np.zeros(gk.shape, dtype=bool)
    mask[idx[sel]] = True
    assert np.array_equal(gk[~mask], kp_ref[~mask]), f"{label}: K pool bytes outside the new rows differ"
    got = gk[idx[sel]]
    if lay.cache_dtype == "fp8_e4m3fn":
        lo_c = e4m3.quantize(normrope.bf16_bits(lo[sel]), lay.k_scale)
        hi_c = e4m3.quantize(normrope.bf16_bits(hi[sel]), lay.k_scale)
        gv, lv, hv = e4m3.decode(got), e4m3.decode(lo_c), e4m3.decode(hi_c)
        bad = ~((gv >= lv) & (gv <= hv))
        assert not bad.any(), f"{label}: {int(bad.sum())} K' codes outside their admissible range"
        return int((lo_c != hi_c).sum()), int((got != lo_c).sum())
    return check_bf16_within(got, lo[sel], hi[sel], label + " K'")
