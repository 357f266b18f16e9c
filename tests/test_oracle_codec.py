"""Pins of the oracle's E4M3FN codec and quantiser against things other than itself.

- printed code values of the OCP E4M3FN format (tests/golden/e4m3_codes.txt);
- the library routine torch.float8_e4m3fn (decode of all 256 codes; encode after
  clamping to +-448, because torch's cast is not saturating);
- closed-form round trips (every finite code, unit and power-of-two scales: the
  draft cache layers use scale 1.0 per "Laguna S 2.1 INT4 -- calibrated FP8 KV on
  Intel B70", section Contract).
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_codes.txt")


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(y_f32):
    t = torch.from_numpy(np.ascontiguousarray(y_f32, dtype=np.float32))
    return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_golden_code_values():
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 15
    for code_s, val_s in rows:
        code = int(code_s, 16)
        got = e4m3.decode(np.array([code], np.uint8))[0]
        want = float(val_s)
        if math.isnan(want):
            assert math.isnan(got), code_s
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (code_s, got, want)


def test_decode_matches_torch_all_codes():
    ours = e4m3.decode(np.arange(256, dtype=np.uint8))
    ref = _torch_decode_all()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF only
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert len(codes) == 254
    back = e4m3.encode(e4m3.decode(codes).astype(np.float32))
    assert np.array_equal(back, codes)


def test_midpoints_tie_to_even_and_match_torch():
    mags = e4m3.decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (mags[:-1] + mags[1:]) / 2)  # exact in fp32
    got = e4m3.encode(mids)
    # the lower neighbour has code k, the upper k+1: the tie goes to the even one
    k = np.arange(len(mids))
    assert np.array_equal(got, np.where(k % 2 == 0, k, k + 1).astype(np.uint8))
    assert np.array_equal(got, _torch_encode(mids))
    assert np.array_equal(e4m3.encode(-mids), _torch_encode(-mids))
    # worked values: 0.06640625 sits between 0.0625 (0x18) and 0.0703125 (0x19)
    assert e4m3.encode(np.float32(0.06640625)) == 0x18
    assert e4m3.encode(np.float32(2.0 ** -10)) == 0x00
    assert e4m3.encode(np.float32(-(2.0 ** -10))) == 0x80
    assert e4m3.encode(np.float32(1.5 * 2.0 ** -10)) == 0x01


def test_saturation_and_specials():
    ys = np.array([448, 449, 463.9, 464, 465, 480, 1e4, np.inf], dtype=np.float32)
    assert np.all(e4m3.encode(ys) == 0x7E)
    assert np.all(e4m3.encode(-ys) == 0xFE)
    assert e4m3.encode(np.float32(np.nan)) == 0x7F
    assert e4m3.encode(np.float32(-np.nan)) == 0xFF
    assert e4m3.encode(np.float32(0.0)) == 0x00
    assert e4m3.encode(np.float32(-0.0)) == 0x80
    # just below the largest normal: 432 is the midpoint of 416 and 448 -> even code 0x7E? 416=0x7D (odd), 448=0x7E
    assert e4m3.encode(np.float32(432.0)) == 0x7E
    assert e4m3.encode(np.float32(431.99)) == 0x7D


def _scales(n, seed=7):
    r = np.random.default_rng(seed)
    s = list(r.uniform(0.01, 0.1, size=n).astype(np.float32))
    s += [np.float32(1.0), np.float32(0.5), np.float32(2.0 ** -6), np.float32(0.0625), np.float32(3.0)]
    return s


def test_quantize_exhaustive_bf16_against_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = e4m3.bf16_bits_to_f32(bits)
    finite_or_inf = ~np.isnan(x)
    bits = bits[finite_or_inf]
    x = x[finite_or_inf]
    assert len(bits) == 65536 - 254  # 2 * 127 NaN payloads
    for s in _scales(40):
        ours = e4m3.quantize(bits, s)
        ref = _torch_encode(x / np.float32(s))
        bad = np.nonzero(ours != ref)[0]
        assert len(bad) == 0, (float(s), bits[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_unit_scale_identity_on_grid():
    """Scale 1.0: a BF16 value that is an E4M3 grid point stores exactly its code."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3.decode(codes).astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(e4m3.bf16_bits_to_f32(bits), vals)  # E4M3 values are exact in BF16
    assert np.array_equal(e4m3.quantize(bits, np.float32(1.0)), codes)


@pytest.mark.parametrize("k", [-8, -5, -3, 1, 4])
def test_power_of_two_scale_round_trip(k):
    s = np.float32(2.0 ** k)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = (e4m3.decode(codes) * float(s)).astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(e4m3.bf16_bits_to_f32(bits), vals)
    assert np.array_equal(e4m3.quantize(bits, s), codes)
    assert np.array_equal(e4m3.dequantize(codes, s), vals.astype(np.float64))


def test_quantize_divides_in_float32():
    """The quotient is one IEEE fp32 division: a case where dividing in float64 first
    and rounding twice would differ is not needed; check the operation dtype and a
    value whose fp32 quotient lands exactly on a midpoint."""
    # 0.0664062500 * 0.5 / 0.5: x = 0.033203125 (exact bf16), scale 0.5 -> 0.06640625 midpoint -> 0x18
    x = np.float32(0.033203125)
    bits = np.array([x.view(np.uint32) >> 16], dtype=np.uint32).astype(np.uint16)
    assert e4m3.bf16_bits_to_f32(bits)[0] == x
    assert e4m3.quantize(bits, np.float32(0.5))[0] == 0x18
