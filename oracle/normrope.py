"""Per-head Q/K RMSNorm and rotary position embedding (RoPE) ahead of the scaled E4M3 insert.

Test infrastructure only (see the package docstring).

The pages place the scaled E4M3 insertion right after the per-head Q/K normalisation and
RoPE ("Laguna S 2.1 INT4 -- calibrated FP8 KV on Intel B70", section "Initial optimization
order", third item) and count an exact fused Q/K RMSNorm + RoPE stack among the gains
("Laguna S 2.1 B70 campaign transfer ledger", section "Result progression and what actually
worked"). They give no formula, epsilon, rotary base or pairing. Readings taken:
  * RMSNorm over the 128 dims of one head vector with one learned weight vector of 128 per
    tensor (one for Q, one for K): y = x * r * w, r = 1 / sqrt(mean(x^2) + eps);
  * RoPE in the rotate-half form over all 128 dims: dims d and d + 64 (d < 64) form a pair
    rotated by the angle of frequency d at the token's position. The caller passes the
    table (one row per position: 64 cosines, then 64 sines), so the base is the caller's;
  * activations are BF16: the normalised vector is rounded to BF16, the rotated one again;
    K is then quantised like any inserted key, V is inserted unchanged, Q is returned;
  * a token whose position lies outside the table is padding: its Q row is returned as
    zeros and its K/V are not inserted; a negative slot only skips the insert (as in the
    plain insert).

A BF16 rounding and a quantised code are decisions taken by floating point, so the oracle
takes them in float32 in one fixed order, which the GPU path follows step for step:
  1. per group of 8 consecutive dims (16 groups): s = s + x*x, each product and sum
     rounded to float32, starting from s = x_0*x_0;
  2. the 16 group sums by a butterfly: for k in 1, 2, 4, 8: s_g = s_g + s_(g xor k);
  3. ms = s / 128 (exact), t = ms + eps, r = 1 / sqrt(t) (IEEE square root, IEEE division);
  4. y_d = bf16(float32(x_d * r) * w_d);
  5. z_d = bf16(float32(y_d * c) - float32(y_(d+64) * s)) and
     z_(d+64) = bf16(float32(y_(d+64) * c) + float32(y_d * s)).
"""

import numpy as np

from . import paged

HEAD_DIM = 128
HALF = HEAD_DIM // 2


def bf16_bits(x):
    """float32 -> BF16 bits, rounded to nearest, ties to even (NaN stays a quiet NaN).

    The BF16 value is the upper half of the float32 bits; rounding adds half of the
    dropped half-word, minus one unless the kept part is odd (ties go to the even one).
    """
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = np.where(nan, (b >> 16) | 0x40, r)
    return r.astype(np.uint16)


def bf16_f32(bits):
    """BF16 bits -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rms_scale(x):
    """Step 1-2: the float32 sum of squares of each 128-vector in the fixed order.

    x: float32 [..., 128]. Returns float32 [...].
    """
    x = np.asarray(x, dtype=np.float32)
    g = x.reshape(x.shape[:-1] + (16, 8))
    s = g[..., 0] * g[..., 0]
    for j in range(1, 8):
        s = (s + g[..., j] * g[..., j]).astype(np.float32)
    idx = np.arange(16)
    for k in (1, 2, 4, 8):
        s = (s + s[..., idx ^ k]).astype(np.float32)
    assert np.all(s == s[..., :1])
    return s[..., 0]


def rmsnorm(x_bits, w_bits, eps):
    """Steps 1-4: RMSNorm of BF16 head vectors [..., 128] with BF16 weight [128] -> BF16 bits."""
    x = bf16_f32(x_bits)
    w = bf16_f32(w_bits)
    s = rms_scale(x)
    ms = (s / np.float32(HEAD_DIM)).astype(np.float32)
    t = (ms + np.float32(eps)).astype(np.float32)
    r = (np.float32(1.0) / np.sqrt(t, dtype=np.float32)).astype(np.float32)
    xr = (x * r[..., None]).astype(np.float32)
    return bf16_bits((xr * w).astype(np.float32))


def rope(y_bits, cos, sin):
    """Step 5: rotate-half RoPE of BF16 vectors [..., 128] by float32 cos/sin [..., 64] -> BF16 bits."""
    y = bf16_f32(y_bits)
    c = np.asarray(cos, dtype=np.float32)
    s = np.asarray(sin, dtype=np.float32)
    lo, hi = y[..., :HALF], y[..., HALF:]
    z_lo = ((lo * c).astype(np.float32) - (hi * s).astype(np.float32)).astype(np.float32)
    z_hi = ((hi * c).astype(np.float32) + (lo * s).astype(np.float32)).astype(np.float32)
    return bf16_bits(np.concatenate([z_lo, z_hi], axis=-1))


def norm_rope(x_bits, w_bits, eps, cos_sin, positions):
    """RMSNorm then RoPE of x [T, H, 128] at positions [T] from the table cos_sin [P, 128].

    Rows of tokens whose position is outside [0, P) come back as zeros (padding).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T = x_bits.shape[0]
    pos = np.asarray(positions, dtype=np.int64)
    table = np.asarray(cos_sin, dtype=np.float32)
    valid = (pos >= 0) & (pos < table.shape[0])
    rows = table[np.where(valid, pos, 0)]  # [T, 128]
    cos = rows[:, None, :HALF]
    sin = rows[:, None, HALF:]
    out = rope(rmsnorm(x_bits, w_bits, eps), cos, sin)
    out[~valid] = 0
    assert out.shape == (T,) + x_bits.shape[1:]
    return out


def norm_rope_insert(k_pool, v_pool, q_bits, k_bits, v_bits, q_w, k_w, eps, cos_sin, positions, slot_mapping,
                     k_scale, v_scale, block_size, num_kv_heads):
    """The whole step for T tokens: returns Q' (BF16 bits [T, Hq, 128]) and inserts K' and V
    into the FP8 pools (in place) at slot_mapping; tokens with a negative slot or a position
    outside the table insert nothing."""
    pos = np.asarray(positions, dtype=np.int64)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    q_out = norm_rope(q_bits, q_w, eps, cos_sin, pos)
    k_rot = norm_rope(k_bits, k_w, eps, cos_sin, pos)
    valid = (pos >= 0) & (pos < np.asarray(cos_sin).shape[0])
    slots = np.where(valid, slots, -1)
    paged.insert(k_pool, v_pool, k_rot, np.asarray(v_bits, dtype=np.uint16), slots, k_scale, v_scale, block_size,
                 num_kv_heads, "fp8_e4m3fn")
    return q_out

