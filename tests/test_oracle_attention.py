"""Pins of the oracle's decode attention against things other than itself.

- closed forms: a single key returns its V row; identical keys return that V;
  q = 0 averages the visible V; a worked two-key example with weights 1/4, 3/4;
  a dominant logit selects its V row;
- brute force on tiny inputs with an independent dense formulation (full score
  matrix, explicit visibility mask, masked softmax, one matrix product);
- invariants: sliding window == global attention over the visible tail; an
  M-row verify window == M separate single-query calls; GQA group == a
  single-KV-head call; page-table permutation; FP8 with a power-of-two scale ==
  a BF16 cache holding the dequantised values.
"""

import math

import numpy as np
import pytest

from oracle import attention, e4m3, paged
from fp8_kv_paged_amd import synth

S128 = 1.0 / math.sqrt(128)


def _rand(r, *shape):
    return r.standard_normal(shape)


def dense_reference(q, k, v, M, window_left, scale):
    """Independent formulation: all rows at once with an explicit [M, L] mask."""
    Mq, Hq, D = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    pos = (L - M + np.arange(M))[:, None]
    j = np.arange(L)[None, :]
    vis = j <= pos
    if window_left >= 0:
        vis &= j >= pos - window_left
    out = np.zeros_like(q)
    for h in range(Hq):
        K, V = k[:, h // G, :], v[:, h // G, :]
        S = scale * q[:, h, :] @ K.T               # [M, L]
        S = np.where(vis, S, -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        out[:, h, :] = P @ V
    return out


def test_single_key_returns_its_value():
    r = np.random.default_rng(0)
    q, k, v = _rand(r, 1, 4, 128), _rand(r, 1, 2, 128), _rand(r, 1, 2, 128)
    out = attention.decode_attention(q, k, v, 1, -1, S128)
    for h in range(4):
        assert np.array_equal(out[0, h], v[0, h // 2])


def test_identical_keys_and_zero_query():
    r = np.random.default_rng(1)
    L = 37
    k = np.repeat(_rand(r, 1, 1, 128), L, axis=0)
    v = _rand(r, L, 1, 128)
    q = _rand(r, 3, 3, 128)
    out = attention.decode_attention(q, k, v, 3, -1, S128)
    for i in range(3):
        mean = v[: L - 3 + i + 1, 0].mean(axis=0)
        assert np.allclose(out[i, 0], mean, rtol=0, atol=1e-13)
    # q = 0: all scores equal -> mean of the visible V rows, window respected
    q0 = np.zeros((2, 1, 128))
    k2 = _rand(r, L, 1, 128)
    out = attention.decode_attention(q0, k2, v, 2, 5, S128)
    for i in range(2):
        p = L - 2 + i
        assert np.allclose(out[i, 0], v[p - 5:p + 1, 0].mean(axis=0), rtol=0, atol=1e-13)


def test_worked_two_key_example():
    """s0 = 0 and s1 = ln 3 give softmax weights 1/4 and 3/4."""
    q = np.zeros((1, 1, 128))
    q[0, 0, 0] = 1.0
    k = np.zeros((2, 1, 128))
    k[1, 0, 0] = math.log(3.0) * math.sqrt(128)  # scale * q.k1 = ln 3
    v = np.zeros((2, 1, 128))
    v[0, 0, :] = 2.0
    v[1, 0, :] = -6.0
    out = attention.decode_attention(q, k, v, 1, -1, S128)
    assert np.allclose(out[0, 0], 0.25 * 2.0 + 0.75 * -6.0, rtol=0, atol=1e-14)
    # with a window of 0 only the key at the query's own position (j = 1) is visible
    out = attention.decode_attention(q, k, v, 1, 0, S128)
    assert np.array_equal(out[0, 0], v[1, 0])
    # negative scale direction: s1 = -ln 3 -> weights 3/4, 1/4
    out = attention.decode_attention(-q, k, v, 1, -1, S128)
    assert np.allclose(out[0, 0], 0.75 * 2.0 + 0.25 * -6.0, rtol=0, atol=1e-14)


def test_dominant_logit_selects_its_row():
    r = np.random.default_rng(2)
    L = 50
    k = _rand(r, L, 1, 128) * 0.01
    q = np.zeros((1, 1, 128))
    q[0, 0, :] = k[17, 0, :] * 1e6
    v = _rand(r, L, 1, 128)
    out = attention.decode_attention(q, k, v, 1, -1, S128)
    assert np.allclose(out[0, 0], v[17, 0], rtol=0, atol=1e-9)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    r = np.random.default_rng(100 + seed)
    for _ in range(12):
        Hkv = int(r.choice([1, 2]))
        G = int(r.choice([1, 3, 9]))
        M = int(r.choice([1, 3, 12]))
        L = int(r.integers(M, 71))
        wl = int(r.choice([-1, 0, 1, 5, 17, 511]))
        q = _rand(r, M, G * Hkv, 128)
        k = _rand(r, L, Hkv, 128) * 2
        v = _rand(r, L, Hkv, 128)
        a = attention.decode_attention(q, k, v, M, wl, S128)
        b = dense_reference(q, k, v, M, wl, S128)
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12), (Hkv, G, M, L, wl)


@pytest.mark.parametrize("seed", range(3))
def test_brute_force_long_query_windows(seed):
    """Chunked prefill: many new rows attend causally to the prefix and to each other."""
    r = np.random.default_rng(200 + seed)
    for _ in range(4):
        Hkv = int(r.choice([1, 2]))
        G = int(r.choice([1, 9]))
        M = int(r.choice([17, 33, 64, 130]))
        L = int(r.integers(M, M + 90))
        wl = int(r.choice([-1, 7, 40, 511]))
        q = _rand(r, M, G * Hkv, 128)
        k = _rand(r, L, Hkv, 128) * 2
        v = _rand(r, L, Hkv, 128)
        a = attention.decode_attention(q, k, v, M, wl, S128)
        b = dense_reference(q, k, v, M, wl, S128)
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12), (Hkv, G, M, L, wl)


def test_visible_range_convention():
    # L = 5, one query at position 4, window_left 2 -> keys 2, 3, 4
    assert attention.visible_range(5, 1, 0, 2) == (2, 4)
    assert attention.visible_range(5, 1, 0, -1) == (0, 4)
    # M = 3 rows at positions 2, 3, 4
    assert [attention.visible_range(5, 3, i, 1) for i in range(3)] == [(1, 2), (2, 3), (3, 4)]
    assert attention.visible_range(5, 3, 0, 100) == (0, 2)


def test_sliding_window_equals_global_over_tail():
    r = np.random.default_rng(3)
    L, M, W = 700, 12, 511
    q, k, v = _rand(r, M, 4, 128), _rand(r, L, 2, 128), _rand(r, L, 2, 128)
    sw = attention.decode_attention(q, k, v, M, W, S128)
    for i in range(M):
        p = L - M + i
        lo = p - W
        tail = attention.decode_attention(q[i:i + 1], k[lo:p + 1], v[lo:p + 1], 1, -1, S128)
        assert np.allclose(sw[i], tail[0], rtol=1e-13, atol=1e-13)
    # window wider than the context == global
    g = attention.decode_attention(q, k, v, M, -1, S128)
    assert np.array_equal(attention.decode_attention(q, k, v, M, L, S128), g)


def test_verify_window_equals_single_query_calls():
    r = np.random.default_rng(4)
    L, M = 300, 12
    q, k, v = _rand(r, M, 18, 128), _rand(r, L, 2, 128), _rand(r, L, 2, 128)
    for wl in (-1, 64):
        full = attention.decode_attention(q, k, v, M, wl, S128)
        for i in range(M):
            Li = L - M + i + 1
            one = attention.decode_attention(q[i:i + 1], k[:Li], v[:Li], 1, wl, S128)
            assert np.array_equal(full[i], one[0])


def test_gqa_group_equals_single_kv_head_call():
    r = np.random.default_rng(5)
    L, M, G, Hkv = 90, 3, 9, 2
    q, k, v = _rand(r, M, G * Hkv, 128), _rand(r, L, Hkv, 128), _rand(r, L, Hkv, 128)
    full = attention.decode_attention(q, k, v, M, -1, S128)
    for g in range(Hkv):
        part = attention.decode_attention(q[:, g * G:(g + 1) * G], k[:, g:g + 1], v[:, g:g + 1], M, -1, S128)
        assert np.array_equal(full[:, g * G:(g + 1) * G], part)
    # swapping the two KV heads swaps the two query groups
    sw = attention.decode_attention(np.concatenate([q[:, G:], q[:, :G]], 1), k[:, ::-1], v[:, ::-1], M, -1, S128)
    assert np.allclose(sw[:, :G], full[:, G:], rtol=0, atol=1e-14)


def _paged_run(lay, table, cache_dtype=paged.FP8):
    bs, H = lay.block_size, lay.num_kv_heads
    kp, vp = paged.new_pools(lay.num_blocks, bs, H, cache_dtype, fill=0x7F)
    for b in range(lay.num_seqs):
        L = int(lay.seq_lens[b])
        k, v = lay.kv_bits(b, 0, L)
        j = np.arange(L)
        slots = (table[b, j // bs].astype(np.int64) * bs + j % bs).astype(np.int32)
        paged.insert(kp, vp, k, v, slots, lay.k_scale, lay.v_scale, bs, H, cache_dtype)
    return attention.paged_decode(kp, vp, lay.q_bits(), table, lay.seq_lens, lay.q_len, lay.window_left,
                                  lay.softmax_scale, lay.k_scale, lay.v_scale, bs, H, cache_dtype)


def test_paged_decode_page_table_permutation_invariance():
    lay = synth.tiny_layer(9, [200, 77], num_q_heads=6, num_kv_heads=2, block_size=32, q_len=3, pool_slack=3.0)
    a = _paged_run(lay, lay.block_table)
    r = np.random.default_rng(11)
    perm = r.permutation(lay.num_blocks).astype(np.int32)
    b = _paged_run(lay, perm[lay.block_table])
    assert np.array_equal(a, b)


def test_paged_decode_matches_logical_dense():
    lay = synth.tiny_layer(10, [129], num_q_heads=18, num_kv_heads=2, block_size=64, q_len=12, window_left=40)
    out = _paged_run(lay, lay.block_table)
    k, v = lay.kv_bits(0, 0, 129)
    kd = e4m3.dequantize(e4m3.quantize(k, lay.k_scale), lay.k_scale)
    vd = e4m3.dequantize(e4m3.quantize(v, lay.v_scale), lay.v_scale)
    q = e4m3.bf16_bits_to_f32(lay.q_bits()[0]).astype(np.float64)
    ref = dense_reference(q, kd, vd, 12, 40, lay.softmax_scale)
    assert np.allclose(out[0], ref, rtol=1e-12, atol=1e-12)


def test_fp8_power_of_two_scale_equals_bf16_cache_of_dequantised_values():
    lay = synth.tiny_layer(12, [150], num_q_heads=9, num_kv_heads=1, block_size=32, q_len=12,
                           fixed_scale=2.0 ** -4)
    fp8 = _paged_run(lay, lay.block_table, paged.FP8)
    # BF16 cache fed with the dequantised values (exact in BF16 for power-of-two scales)
    bs, H, L = 32, 1, 150
    k, v = lay.kv_bits(0, 0, L)
    kd = e4m3.dequantize(e4m3.quantize(k, lay.k_scale), lay.k_scale).astype(np.float32)
    vd = e4m3.dequantize(e4m3.quantize(v, lay.v_scale), lay.v_scale).astype(np.float32)
    kb = (kd.view(np.uint32) >> 16).astype(np.uint16)
    vb = (vd.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(e4m3.bf16_bits_to_f32(kb), kd)
    kp, vp = paged.new_pools(lay.num_blocks, bs, H, paged.BF16)
    paged.insert(kp, vp, kb, vb, lay.slots(0, 0, L), 1.0, 1.0, bs, H, paged.BF16)
    bf = attention.paged_decode(kp, vp, lay.q_bits(), lay.block_table, lay.seq_lens, 12, -1, lay.softmax_scale,
                                1.0, 1.0, bs, H, paged.BF16)
    assert np.array_equal(fp8, bf)
