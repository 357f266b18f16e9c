"""Pins of the oracle's Q/K RMSNorm + RoPE + insert step against things other than itself:

- the BF16 rounding: torch's float32 -> bfloat16 cast (round to nearest even) on float32
  inputs, and an exact brute force with Python fractions on float64 inputs (the nearest BF16
  value, ties to even, with no intermediate float32 rounding);
- RMSNorm: the library routine torch.nn.functional.rms_norm in float64;
- RoPE: multiplication of the complex pair (y_d + i y_(d+64)) by cos + i sin in numpy, and the
  relative-position property of rotary embeddings;
- closed forms: a constant vector normalises to its sign times the weight; scaling the input
  by a power of two leaves the result unchanged when eps = 0; position 0 is the identity; a
  unit vector in dim d moves into dim d + 64 by the sine of column d;
- the insert: K' codes decode to the float64 pipeline value within half an E4M3 step plus
  the BF16 roundings, V is inserted exactly as the plain insert does, and padding tokens
  write nothing.
"""

import numpy as np
import pytest
import torch

from fp8_kv_paged_amd import synth
from oracle import e4m3, normrope, paged

EPS24 = 2.0 ** -24


def _bf16_half_ulp(x):
    """Half the BF16 spacing at |x| (float64), for finite normal x."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 8)


def _rand_bf16(rng, shape, scale=1.0):
    return synth.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(1e3),
        rng.standard_normal(1000).astype(np.float32) * np.float32(1e-39),   # subnormals
        np.array([0.0, -0.0, 3.3895314e38, -3.3895314e38, np.inf, -np.inf], dtype=np.float32),
        # exact ties: the dropped half-word is 0x8000, kept parts odd and even
        (np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40000000 | 0x18000], dtype=np.uint32)).view(np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(normrope.bf16_bits(x), want)
    assert np.isnan(normrope.bf16_f32(normrope.bf16_bits(np.array([np.nan], np.float32))))[0]


def _nearest_bf16_fraction(x):
    """Exact nearest BF16 value of a finite float64 x, ties to even, by brute force over the
    two BF16 values that bracket it (Python fractions: no rounding anywhere)."""
    from fractions import Fraction
    xf = Fraction(float(x))
    if xf == 0:
        return 0.0
    b32 = np.array([x], dtype=np.float32).view(np.uint32)[0]
    cands = set()
    for base in (int(b32) >> 16, (int(b32) >> 16) - 1, (int(b32) >> 16) + 1):
        for sgn in (0, 0x8000):
            bits = (base & 0x7FFF) | sgn
            if (bits & 0x7F80) != 0x7F80:
                cands.add(bits)
    best = None
    for bits in cands:
        v = Fraction(float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]))
        d = abs(v - xf)
        if best is None or d < best[0] or (d == best[0] and (bits & 1) == 0):
            best = (d, bits, v)
    return float(best[2])


def test_bf16_rounding_of_float64_values_is_one_rounding():
    rng = np.random.default_rng(7)
    xs = list(rng.standard_normal(1500) * 10.0 ** rng.integers(-6, 6, 1500))
    one = 1.0
    # just above / below BF16 ties: a float32 intermediate would round these to the tie and
    # then to even, a single rounding does not
    xs += [one + 2.0 ** -8 + 2.0 ** -40, one + 2.0 ** -8 - 2.0 ** -40, -(3.0 + 2.0 ** -7 + 2.0 ** -45),
           one + 3 * 2.0 ** -8 - 2.0 ** -38, 2.0 ** -130 + 2.0 ** -140, 1.5 * 2.0 ** -133]
    # exact ties: to even
    xs += [one + 2.0 ** -8, one + 3 * 2.0 ** -8, -(one + 2.0 ** -8)]
    got = normrope.bf16_round(np.array(xs))
    want = np.array([_nearest_bf16_fraction(x) for x in xs])
    assert np.array_equal(got, want)
    assert normrope.bf16_round(np.array([one + 2.0 ** -8 + 2.0 ** -40]))[0] == one + 2.0 ** -7
    assert normrope.bf16_round(np.array([one + 2.0 ** -8]))[0] == one
    # overflow, infinities, signed zero
    assert np.isinf(normrope.bf16_round(np.array([3.4e38]))).all()
    assert normrope.bf16_bits(np.array([-0.0]))[0] == 0x8000


def test_rmsnorm_matches_torch_rms_norm():
    rng = np.random.default_rng(8)
    x = _rand_bf16(rng, (300, 4, 128), scale=3.0)
    w = synth.f32_to_bf16_bits(rng.uniform(0.5, 1.5, 128).astype(np.float32))
    for eps in (1e-6, 1e-2):
        xt = torch.from_numpy(normrope.bf16_f32(x).astype(np.float64))
        wt = torch.from_numpy(normrope.bf16_f32(w).astype(np.float64))
        ref = torch.nn.functional.rms_norm(xt, (128,), wt, eps).numpy()
        assert np.allclose(normrope.rmsnorm_f64(x, w, eps), ref, rtol=1e-13, atol=0.0)
        assert np.array_equal(normrope.rmsnorm(x, w, eps), normrope.bf16_bits(ref))


@pytest.mark.parametrize("eps,scale", [(1e-6, 5.0), (1e-2, 5.0), (1e-2, 0.05)])  # the last: eps dominates
def test_rmsnorm_matches_the_float64_formula(eps, scale):
    rng = np.random.default_rng(3)
    x = _rand_bf16(rng, (400, 3, 128), scale=scale)
    w = synth.f32_to_bf16_bits(rng.uniform(0.5, 1.5, 128).astype(np.float32))
    y = normrope.bf16_f32(normrope.rmsnorm(x, w, eps)).astype(np.float64)
    xf = normrope.bf16_f32(x).astype(np.float64)
    wf = normrope.bf16_f32(w).astype(np.float64)
    y64 = xf * wf / np.sqrt((xf ** 2).mean(axis=-1, keepdims=True) + eps)
    bound = _bf16_half_ulp(y64) + 20 * EPS24 * np.abs(y64)
    assert np.all(np.abs(y - y64) <= bound)
    # the weight is applied per dimension, not per head: reversing it changes the result
    y_rev = normrope.bf16_f32(normrope.rmsnorm(x, w[::-1].copy(), eps)).astype(np.float64)
    assert not np.allclose(y_rev, y64, rtol=1e-2)


def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(4)
    w = synth.f32_to_bf16_bits(rng.uniform(0.5, 1.5, 128).astype(np.float32))
    for c in (0.75, -3.0, 1.0e-3, 96.0):
        x = synth.f32_to_bf16_bits(np.full((1, 128), c, np.float32))
        y = normrope.rmsnorm(x, w, 0.0)
        want = w if c > 0 else (w ^ np.uint16(0x8000))
        assert np.array_equal(y[0], want), c
    # eps = 0: scaling the input by 2^k changes nothing
    x = _rand_bf16(rng, (64, 128), scale=2.0)
    base = normrope.rmsnorm(x, w, 0.0)
    for k in (-5, 3, 9):
        xs = synth.f32_to_bf16_bits(normrope.bf16_f32(x) * np.float32(2.0 ** k))
        assert np.array_equal(normrope.rmsnorm(xs, w, 0.0), base), k


def test_rope_identity_at_position_zero_and_pairing():
    table = synth.rope_table(300)
    assert np.all(table[0, :64] == 1.0) and np.all(table[0, 64:] == 0.0)
    rng = np.random.default_rng(5)
    y = _rand_bf16(rng, (7, 128))
    z0 = normrope.rope(y, table[0, :64], table[0, 64:])
    assert np.array_equal(z0, y)
    # a unit vector in dim d (d < 64) turns toward dim d + 64 by the angle of column d,
    # and one in dim d + 64 turns toward -d
    p = 257
    c, s = table[p, :64], table[p, 64:]
    for d in (0, 1, 17, 63):
        e = np.zeros(128, np.float32)
        e[d] = 1.0
        z = normrope.bf16_f32(normrope.rope(synth.f32_to_bf16_bits(e), c, s))
        want = np.zeros(128, np.float32)
        want[d], want[d + 64] = c[d], s[d]
        assert np.array_equal(z, normrope.bf16_f32(normrope.bf16_bits(want))), d
        e2 = np.zeros(128, np.float32)
        e2[d + 64] = 1.0
        z2 = normrope.bf16_f32(normrope.rope(synth.f32_to_bf16_bits(e2), c, s))
        want2 = np.zeros(128, np.float32)
        want2[d], want2[d + 64] = -s[d], c[d]
        assert np.array_equal(z2, normrope.bf16_f32(normrope.bf16_bits(want2))), d


def test_rope_matches_complex_rotation_and_keeps_relative_positions():
    table = synth.rope_table(4096)
    rng = np.random.default_rng(6)
    y = _rand_bf16(rng, (50, 128))
    pos = rng.integers(0, 4096, 50)
    z = normrope.bf16_f32(normrope.rope(y, table[pos, :64], table[pos, 64:])).astype(np.float64)
    yf = normrope.bf16_f32(y).astype(np.float64)
    f = synth.ROPE_BASE ** (-np.arange(64) / 64.0)
    rot = (yf[:, :64] + 1j * yf[:, 64:]) * np.exp(1j * pos[:, None] * f[None, :])
    z64 = np.concatenate([rot.real, rot.imag], axis=1)
    # float32 table and products, one BF16 rounding
    assert np.all(np.abs(z - z64) <= _bf16_half_ulp(z64) + 1e-6 * np.abs(yf).max(axis=1, keepdims=True))
    # <rope(q, p), rope(k, p')> depends on p - p' only (up to the BF16 roundings)
    q, k = _rand_bf16(rng, (1, 128)), _rand_bf16(rng, (1, 128))

    def dot(pq, pk):
        a = normrope.bf16_f32(normrope.rope(q, table[pq, :64], table[pq, 64:])).astype(np.float64)
        b = normrope.bf16_f32(normrope.rope(k, table[pk, :64], table[pk, 64:])).astype(np.float64)
        return float((a * b).sum())
    nq = np.linalg.norm(normrope.bf16_f32(q)) * np.linalg.norm(normrope.bf16_f32(k))
    for (pq, pk, d) in ((100, 40, 1000), (7, 3, 2500), (3000, 2990, 1)):
        assert abs(dot(pq, pk) - dot(pq + d, pk + d)) <= 0.03 * nq


def test_insert_step_against_the_float64_pipeline_and_padding():
    lay = synth.tiny_layer(501, [70, 5, 33], num_q_heads=18, num_kv_heads=2, block_size=32, q_len=12)
    st = synth.norm_rope_step(lay)
    # one token whose position falls outside the table, one with a negative slot
    st.positions = st.positions.copy()
    st.slot_mapping = st.slot_mapping.copy()
    untouched = [int(st.slot_mapping[3]), int(st.slot_mapping[5])]
    assert min(untouched) >= 0
    st.positions[3] = st.cos_sin.shape[0]
    st.slot_mapping[5] = -1
    kp, vp = paged.new_pools(lay.num_blocks, lay.block_size, lay.num_kv_heads, "fp8_e4m3fn", fill=0xA5)
    k0, v0 = kp.copy(), vp.copy()
    q_out = normrope.norm_rope_insert(kp, vp, st.q_bits, st.k_bits, st.v_bits, st.q_w, st.k_w, st.eps, st.cos_sin,
                                      st.positions, st.slot_mapping, lay.k_scale, lay.v_scale, lay.block_size,
                                      lay.num_kv_heads)
    T = st.positions.shape[0]
    valid = (st.positions >= 0) & (st.positions < st.cos_sin.shape[0])
    assert np.all(q_out[~valid] == 0)
    # the same inserts through the plain insert: V unchanged, K after norm + RoPE
    kq, vq = k0.copy(), v0.copy()
    k_rot = normrope.norm_rope(st.k_bits, st.k_w, st.eps, st.cos_sin, st.positions)
    slots = np.where(valid, st.slot_mapping, -1)
    paged.insert(kq, vq, k_rot, st.v_bits, slots, lay.k_scale, lay.v_scale, lay.block_size, lay.num_kv_heads,
                 "fp8_e4m3fn")
    assert np.array_equal(kp, kq) and np.array_equal(vp, vq)
    # the padding tokens' slots still hold the fill bytes
    for sl in untouched:
        blk, off = divmod(sl, lay.block_size)
        for h in range(lay.num_kv_heads):
            assert np.all(kp[paged.k_index(blk, h, off, np.arange(128), lay.block_size, lay.num_kv_heads)] == 0xA5)
            assert np.all(vp[paged.v_index(blk, h, off, np.arange(128), lay.block_size, lay.num_kv_heads)] == 0xA5)
    # K' codes against the float64 pipeline: within half an E4M3 step of the BF16 K' / k_scale
    xf = normrope.bf16_f32(st.k_bits).astype(np.float64)
    wf = normrope.bf16_f32(st.k_w).astype(np.float64)
    y64 = xf * wf / np.sqrt((xf ** 2).mean(axis=-1, keepdims=True) + st.eps)
    pos = np.where(valid, st.positions, 0)
    f = synth.ROPE_BASE ** (-np.arange(64) / 64.0)
    ang = pos[:, None, None] * f[None, None, :]
    z64 = np.concatenate([y64[..., :64] * np.cos(ang) - y64[..., 64:] * np.sin(ang),
                          y64[..., 64:] * np.cos(ang) + y64[..., :64] * np.sin(ang)], axis=-1)
    for t in range(T):
        if not valid[t] or st.slot_mapping[t] < 0:
            continue
        blk, off = divmod(int(st.slot_mapping[t]), lay.block_size)
        for h in range(lay.num_kv_heads):
            code = kp[paged.k_index(blk, h, off, np.arange(128), lay.block_size, lay.num_kv_heads)]
            got = e4m3.decode(code)
            y = z64[t, h] / float(lay.k_scale)
            # E4M3 half-step (relative 2^-4, absolute 2^-10 in the subnormals), plus the BF16
            # rounding of the normalised pair before the rotation (it cancels in small outputs)
            # and of the rotated value
            pair = np.abs(y64[t, h]) + np.abs(np.roll(y64[t, h], 64))
            bound = (np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10)
                     + (pair + np.abs(z64[t, h])) * 2.0 ** -8 / float(lay.k_scale))
            assert np.all(np.abs(got - np.clip(y, -448, 448)) <= bound), (t, h)

