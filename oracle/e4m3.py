"""E4M3FN codec and the scaled quantiser, from the definition.

Test infrastructure only (see the package docstring).

The pages fix the format only as "E4M3 FP8" with calibrated scalar K/V scales
("Laguna S 2.1 INT4 -- calibrated FP8 KV on Intel B70", section Contract) and
the scale direction "quantize, store FP8, scale/dequantize" ("Laguna S 2.1
KV-cache precision decision", table in "BF16 versus FP8 in concrete terms").
Readings taken where they are silent:
  * the format is OCP E4M3FN: bias 7, no infinities, S.1111.111 is NaN,
    largest finite 448 (S.1111.110);
  * quantise: y = fp32(x) / fp32(scale) with one IEEE round-to-nearest-even
    float32 division, then y is rounded to E4M3FN to nearest, ties to even,
    saturating to +-448 for |y| >= 448 (including +-inf); NaN -> 0x7F|sign;
    the sign of zero is kept;
  * dequantise: value = decode(byte) * scale.

Method: decode is the closed form of the format. Encode does NOT use bit
manipulation: it compares |y| against the exact midpoints between the 127
non-negative finite E4M3FN magnitudes (all exactly representable in float64)
and breaks exact ties toward the even code.
"""

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def decode(codes):
    """Decode E4M3FN bytes to float64 (NaN for S.1111.111).

    Closed form: sign s = b>>7, exponent e = (b>>3)&15, mantissa m = b&7;
    e == 0: (-1)^s * m * 2^-9 (subnormal); otherwise (-1)^s * (1 + m/8) * 2^(e-7).
    """
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = b >> 7
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


# The 127 non-negative finite magnitudes, codes 0x00..0x7E, strictly increasing.
_MAGS = decode(np.arange(0, 0x7F, dtype=np.uint8))
assert np.all(np.diff(_MAGS) > 0)
_MIDS = (_MAGS[:-1] + _MAGS[1:]) / 2.0  # exact in float64


def encode(y):
    """Round float32/float64 values to E4M3FN codes (RNE, saturating at +-448).

    y is rounded from its exact value (float32 inputs are exact in float64).
    """
    y = np.asarray(y, dtype=np.float64)
    sign = np.signbit(y).astype(np.uint8) << 7
    a = np.abs(y)
    nan = np.isnan(a)
    a_clean = np.where(nan, 0.0, a)
    # index of the first midpoint >= a: candidates lo = k, hi = k + 1
    k = np.searchsorted(_MIDS, a_clean, side="left")
    k = np.minimum(k, len(_MAGS) - 1)
    # a < mid[k] -> code k ; a == mid[k] -> even of (k, k+1) ; (a > mid[k] impossible by searchsorted except k = last)
    at_mid = (k < len(_MIDS)) & (a_clean == _MIDS[np.minimum(k, len(_MIDS) - 1)])
    code = np.where(at_mid & (k % 2 == 1), k + 1, k)
    code = np.where(a_clean >= E4M3_MAX, 0x7E, code)
    code = np.where(nan, NAN_CODE, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def bf16_bits_to_f32(bits):
    """BF16 bit patterns (uint16) to float32: the BF16 bits are the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def quantize(x_bf16_bits, scale):
    """Quantise BF16 K or V to E4M3FN codes with one per-tensor scalar scale.

    y = float32(x) / float32(scale) as one IEEE float32 division (NumPy float32
    true division rounds to nearest even), then encode(y).
    """
    x = bf16_bits_to_f32(x_bf16_bits)
    y = x / np.float32(scale)
    assert y.dtype == np.float32
    return encode(y)


def dequantize(codes, scale):
    """float64 value of stored codes: decode(code) * scale."""
    return decode(codes) * np.float64(np.float32(scale))
