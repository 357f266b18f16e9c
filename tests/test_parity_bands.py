"""CPU check of the admissible-interval helpers the GPU norm/RoPE tests use (tests/parity.py):
a float32 evaluation of the step in the kernel's documented order (include/fkv.h,
fkv_qk_norm_rope_insert: eight-dim lanes summed in dim order, then combined at distances 1, 2,
4, 8; every operation rounded once) must fall inside the intervals for every element, and the
intervals must be a single value for nearly all elements. Also checks that the intervals are
not vacuous: a one-ulp change of an exact element falls outside."""

import numpy as np

from fp8_kv_paged_amd import synth
from oracle import normrope

import parity


def _f32_kernel_order(x_bits, w_bits, eps, cos, sin):
    x = normrope.bf16_f32(x_bits)
    w = normrope.bf16_f32(w_bits)
    g = x.reshape(x.shape[:-1] + (16, 8))
    s = (g[..., 0] * g[..., 0]).astype(np.float32)
    for j in range(1, 8):
        s = (s + (g[..., j] * g[..., j]).astype(np.float32)).astype(np.float32)
    idx = np.arange(16)
    for k in (1, 2, 4, 8):
        s = (s + s[..., idx ^ k]).astype(np.float32)
    r = (np.float32(1.0) / np.sqrt((s[..., :1] / np.float32(128.0) + np.float32(eps)).astype(np.float32),
                                    dtype=np.float32)).astype(np.float32)
    y = normrope.bf16_f32(_rne_f32_to_bf16(((x * r).astype(np.float32) * w).astype(np.float32)))
    lo, hi = y[..., :64], y[..., 64:]
    c, sn = cos.astype(np.float32), sin.astype(np.float32)
    zl = ((lo * c).astype(np.float32) - (hi * sn).astype(np.float32)).astype(np.float32)
    zh = ((hi * c).astype(np.float32) + (lo * sn).astype(np.float32)).astype(np.float32)
    return _rne_f32_to_bf16(np.concatenate([zl, zh], axis=-1))


def _rne_f32_to_bf16(x):
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def test_float32_evaluation_lies_inside_the_bands():
    lay = synth.tiny_layer(531, [400, 70, 2000], num_q_heads=72, num_kv_heads=8, block_size=64, q_len=12)
    st = synth.norm_rope_step(lay)
    total = nonexact = differ = 0
    for x_bits, w_bits in ((st.q_bits, st.q_w), (st.k_bits, st.k_w)):
        valid, cos, sin = normrope.table_rows(st.cos_sin, st.positions)
        got = _f32_kernel_order(x_bits, w_bits, st.eps, cos[:, None, :], sin[:, None, :])
        got[~valid] = 0
        lo, hi, exact = parity.norm_rope_bounds(x_bits, w_bits, st.eps, st.cos_sin, st.positions)
        n, d = parity.check_bf16_within(got, lo, hi, "float32 order")
        total += got.size
        nonexact += n
        differ += d
        # not vacuous: moving an exact element by one BF16 step leaves its interval
        e = np.argwhere(exact & (lo != 0))[0]
        bumped = got.copy()
        bumped[tuple(e)] += 1
        try:
            parity.check_bf16_within(bumped, lo, hi, "bumped")
            raise AssertionError("a one-step change passed the bands")
        except AssertionError as err:
            assert "outside their admissible" in str(err)
    print(f"{total} elements, {nonexact} with two admissible values, {differ} differ from the oracle")
    assert nonexact <= total * 0.01
