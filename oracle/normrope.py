"""Per-head Q/K RMSNorm and rotary position embedding (RoPE) ahead of the scaled E4M3 insert.

Test infrastructure only (see the package docstring).

The pages place the scaled E4M3 insertion right after the per-head Q/K normalisation and
RoPE ("Laguna S 2.1 INT4 -- calibrated FP8 KV on Intel B70", section "Initial optimization
order", third item) and count an exact fused Q/K RMSNorm + RoPE stack among the gains
("Laguna S 2.1 B70 campaign transfer ledger", section "Result progression and what actually
worked"). They give no formula, epsilon, rotary base or pairing. Readings taken:
  * RMSNorm over the 128 dims of one head vector with one learned weight vector of 128 per
    tensor (one for Q, one for K): y = x * w / sqrt(mean(x^2) + eps);
  * RoPE in the rotate-half form over all 128 dims: dims d and d + 64 (d < 64) form a pair
    rotated by the angle of frequency d at the token's position,
        z_d = y_d cos - y_(d+64) sin,   z_(d+64) = y_(d+64) cos + y_d sin.
    The caller passes the table (one row per position: 64 cosines, then 64 sines, float32),
    so the rotary base is the caller's;
  * activations are BF16: the normalised vector is rounded to BF16, the rotated one again;
    K is then quantised like any inserted key, V is inserted unchanged, Q is returned;
  * a token whose position lies outside the table is padding: its Q row is returned as
    zeros and its K/V are not inserted; a negative slot only skips the insert (as in the
    plain insert).

Every step is the formula above evaluated in float64, and each BF16 value is the float64
result rounded once to the nearest BF16 value, ties to even. No other rounding takes
place; in particular the float64 values are never rounded through float32 first.
"""

import numpy as np

from . import paged

HEAD_DIM = 128
HALF = HEAD_DIM // 2

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127   # largest finite BF16 value
_BF16_MIN_EXP = -133                          # spacing of the BF16 subnormals: 2^-126 * 2^-7


def bf16_round(x):
    """float64 -> the nearest BF16 value (ties to even), returned as float64.

    BF16 keeps 8 significant bits: a value in [2^(e-1), 2^e) is rounded to a multiple of
    2^(e-8), and below 2^-126 to a multiple of 2^-133 (the subnormals). Dividing by that
    power of two is exact, np.rint rounds half to even, and multiplying back is exact.
    Results beyond the largest finite BF16 value become infinities; NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)  # x = m 2^e with 0.5 <= |m| < 1 (e = 0 for zero)
    q = np.maximum(e.astype(np.int64) - 8, _BF16_MIN_EXP)
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
        r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, x), r)
    r = np.where(np.isfinite(x), r, x)
    return np.where(x == 0.0, x, r)  # keeps the sign of zero


def bf16_bits(x):
    """BF16 bit patterns of bf16_round(x) (the rounded value is exact in float32)."""
    r = bf16_round(x).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def bf16_f32(bits):
    """BF16 bits -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rmsnorm_f64(x_bits, w_bits, eps):
    """y = x * w / sqrt(mean(x^2) + eps) in float64, before rounding: [..., 128]."""
    x = bf16_f32(x_bits).astype(np.float64)
    w = bf16_f32(w_bits).astype(np.float64)
    return x * w / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + float(eps))


def rmsnorm(x_bits, w_bits, eps):
    """RMSNorm of BF16 head vectors [..., 128] with a BF16 weight [128] -> BF16 bits."""
    return bf16_bits(rmsnorm_f64(x_bits, w_bits, eps))


def rope_f64(y_bits, cos, sin):
    """Rotate-half RoPE of BF16 vectors [..., 128] by cos / sin [..., 64], float64, before rounding."""
    y = bf16_f32(y_bits).astype(np.float64)
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    lo, hi = y[..., :HALF], y[..., HALF:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def rope(y_bits, cos, sin):
    """Rotate-half RoPE of BF16 vectors [..., 128] -> BF16 bits."""
    return bf16_bits(rope_f64(y_bits, cos, sin))


def table_rows(cos_sin, positions):
    """(valid [T], cos [T, 64], sin [T, 64]) for token positions; invalid rows read row 0."""
    pos = np.asarray(positions, dtype=np.int64)
    table = np.asarray(cos_sin, dtype=np.float32)
    valid = (pos >= 0) & (pos < table.shape[0])
    rows = table[np.where(valid, pos, 0)]
    return valid, rows[:, :HALF], rows[:, HALF:]


def norm_rope(x_bits, w_bits, eps, cos_sin, positions):
    """RMSNorm then RoPE of x [T, H, 128] at positions [T] from the table cos_sin [P, 128].

    Rows of tokens whose position is outside [0, P) come back as zeros (padding).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    valid, cos, sin = table_rows(cos_sin, positions)
    out = rope(rmsnorm(x_bits, w_bits, eps), cos[:, None, :], sin[:, None, :])
    out[~valid] = 0
    return out


def norm_rope_insert(k_pool, v_pool, q_bits, k_bits, v_bits, q_w, k_w, eps, cos_sin, positions, slot_mapping,
                     k_scale, v_scale, block_size, num_kv_heads, cache_dtype="fp8_e4m3fn"):
    """The whole step for T tokens: returns Q' (BF16 bits [T, Hq, 128]) and inserts K' and V
    into the pools (in place) at slot_mapping through the plain insert; tokens with a negative
    slot or a position outside the table insert nothing."""
    pos = np.asarray(positions, dtype=np.int64)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    q_out = norm_rope(q_bits, q_w, eps, cos_sin, pos)
    k_rot = norm_rope(k_bits, k_w, eps, cos_sin, pos)
    valid = (pos >= 0) & (pos < np.asarray(cos_sin).shape[0])
    slots = np.where(valid, slots, -1)
    paged.insert(k_pool, v_pool, k_rot, np.asarray(v_bits, dtype=np.uint16), slots, k_scale, v_scale, block_size,
                 num_kv_heads, cache_dtype)
    return q_out
