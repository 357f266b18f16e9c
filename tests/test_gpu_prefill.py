"""GPU parity of long query windows (chunked prefill: q_len new tokens attending causally to
the cached prefix and to each other) on the 32-row kernel against the oracle, within the
2e-3 row-normalised gate: windows just past the decode shapes up to the 4,096-token maximum,
from scratch and on long prefixes, global and sliding-window, both page sizes, ragged batches,
explicit split sizes through the combine kernel, BF16 output."""

import numpy as np
import pytest
import torch

from fp8_kv_paged_amd import fkv, synth
from fp8_kv_paged_amd.layer import PagedLayer
from oracle import attention

import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def _reference(lay, b, kv_heads=None):
    """Oracle rows of sequence b; rows at negative positions (L < q_len) see no key: zeros."""
    M, L = lay.q_len, int(lay.seq_lens[b])
    if L >= M:
        return parity.reference(lay, b, kv_heads)
    G = lay.num_q_heads // lay.num_kv_heads
    k, v = parity.logical_kv(lay, b)
    q = parity.q_f64(lay, b)
    out = np.zeros(q.shape)
    for g in range(lay.num_kv_heads):
        sl = slice(g * G, (g + 1) * G)
        out[M - L:, sl] = attention.decode_attention(q[M - L:, sl], k[:, g:g + 1], v[:, g:g + 1], L,
                                                     lay.window_left, lay.softmax_scale)
    return out


def _check(lay, out, label, kv_heads=None, tol=parity.ATTN_TOL):
    gpu = out.float().cpu().numpy()
    worst = 0.0
    for b in range(lay.num_seqs):
        worst = max(worst, float(parity.row_errors(gpu[b], _reference(lay, b, kv_heads)).max()))
    print(f"[prefill parity] {label}: max row error {worst:.3e}", flush=True)
    assert worst <= tol, (label, worst)


def _cases():
    yield "q17 global p32", lambda: synth.tiny_layer(601, [17, 500, 1500], num_q_heads=18, num_kv_heads=2,
                                                     block_size=32, q_len=17)
    yield "q64 from scratch and on 2k, p64", lambda: synth.tiny_layer(603, [64, 2100], num_q_heads=18,
                                                                      num_kv_heads=2, block_size=64, q_len=64)
    yield "q256 window 512 p64", lambda: synth.tiny_layer(605, [300, 2048], num_q_heads=18, num_kv_heads=2,
                                                          block_size=64, q_len=256, window_left=511)
    yield "q128 72/8 on 4k p64", lambda: synth.tiny_layer(607, [4096], num_q_heads=72, num_kv_heads=8,
                                                          block_size=64, q_len=128)
    yield "q13 72/8 (117 rows) p32", lambda: synth.tiny_layer(609, [3000, 13], num_q_heads=72, num_kv_heads=8,
                                                              block_size=32, q_len=13)
    yield "ragged, rows before position 0", lambda: synth.tiny_layer(611, [40, 7, 900, 100], num_q_heads=18,
                                                                     num_kv_heads=2, block_size=32, q_len=100)


@pytest.mark.parametrize("label,make", list(_cases()), ids=[c[0] for c in _cases()])
def test_long_windows_against_the_oracle(label, make):
    lay = make()
    gl = PagedLayer(lay).build()
    out = gl.decode().clone()
    out5 = PagedLayer(lay, layout=5).build().decode().clone()
    torch.cuda.synchronize()
    assert torch.equal(out, out5), label  # the automatic layout is layout 5 here
    _check(lay, out, label)


@pytest.mark.parametrize("split_tiles", [4, 8, 40])
def test_explicit_splits_through_the_combine_kernel(split_tiles):
    lay = synth.tiny_layer(613, [1800, 333], num_q_heads=18, num_kv_heads=2, block_size=64, q_len=48)
    gl = PagedLayer(lay, split_tiles=split_tiles).build()
    before = fkv.get_counters()["decode_combine_launches"]
    out = gl.decode().clone()
    torch.cuda.synchronize()
    assert fkv.get_counters()["decode_combine_launches"] == before + 1
    _check(lay, out, f"split_tiles {split_tiles}")


def test_chunk_of_512_on_an_8k_prefix_sampled_heads():
    """72/8 heads, 512 new tokens at context 8192 (4,608 packed rows per KV head); the oracle
    checks two of the eight KV heads."""
    lay = synth.tiny_layer(615, [8192], num_q_heads=72, num_kv_heads=8, block_size=64, q_len=512)
    out = PagedLayer(lay).build().decode().clone()
    torch.cuda.synchronize()
    heads = [0, 5]
    _check(lay, out, "q512 on 8k, KV heads 0 and 5", kv_heads=heads)
    assert torch.isfinite(out).all()


def test_bf16_output():
    lay = synth.tiny_layer(617, [700, 64], num_q_heads=18, num_kv_heads=2, block_size=32, q_len=64)
    o32 = PagedLayer(lay).build().decode().clone()
    o16 = PagedLayer(lay, out_bf16=True).build().decode().clone()
    torch.cuda.synchronize()
    assert torch.equal(o16.view(torch.int16), o32.to(torch.bfloat16).view(torch.int16))
    _check(lay, o16, "q64 BF16 output", tol=parity.ATTN_TOL + 2.0 ** -7)


def _sampled_rows_check(lay, out, label, kv_heads, rows):
    """Sampled rows of sequence 0 against the oracle: row i of a q_len-token window equals the
    one-query attention at seq_len L - q_len + i + 1 (the oracle's own pinned identity), so each
    sampled row is one oracle call over its visible keys."""
    M, L = lay.q_len, int(lay.seq_lens[0])
    G = lay.num_q_heads // lay.num_kv_heads
    k, v = parity.logical_kv(lay, 0, heads=kv_heads)
    q = parity.q_f64(lay, 0)
    gpu = out.float().cpu().numpy()[0]
    worst = 0.0
    for i in rows:
        n = L - M + i + 1
        for j, g in enumerate(kv_heads):
            sl = slice(g * G, (g + 1) * G)
            if n <= 0:
                assert np.all(gpu[i, sl] == 0.0), (label, i)
                continue
            ref = attention.decode_attention(q[i:i + 1, sl], k[:n, j:j + 1], v[:n, j:j + 1], 1, lay.window_left,
                                             lay.softmax_scale)
            worst = max(worst, float(parity.row_errors(gpu[i:i + 1, sl], ref).max()))
    print(f"[prefill parity] {label}: {len(rows)} sampled rows x KV heads {kv_heads}: max row error {worst:.3e}",
          flush=True)
    assert worst <= parity.ATTN_TOL, (label, worst)


@pytest.mark.parametrize("label,seed,L,q_len,hq,hkv,bs,wl,heads", [
    ("q2048 from scratch, global, 18/2, p64", 621, 2048, 2048, 18, 2, 64, -1, [0, 1]),
    ("q2048 on a 2k prefix, window 512, 18/2, p32", 623, 4100, 2048, 18, 2, 32, 511, [1]),
    ("q4096 maximum on a 2k prefix, global, 72/8, p64", 625, 6144, 4096, 72, 8, 64, -1, [0, 6]),
], ids=["q2048_scratch", "q2048_window", "q4096_72x8"])
def test_longest_windows_sampled_rows(label, seed, L, q_len, hq, hkv, bs, wl, heads):
    """The longest query windows the header allows (up to FKV_MAX_PREFILL_Q_LEN = 4,096 tokens),
    through the combine kernel, on sampled rows: the first and last rows, rows around tile and
    window boundaries, and a seeded random sample."""
    lay = synth.tiny_layer(seed, [L], num_q_heads=hq, num_kv_heads=hkv, block_size=bs, q_len=q_len, window_left=wl)
    print(f"[prefill parity] {label}: building", flush=True)
    gl = PagedLayer(lay).build()
    fkv.reset_counters()
    out = gl.decode().clone()
    torch.cuda.synchronize()
    cnt = fkv.get_counters()
    assert cnt["decode_long_windows"][0] == 1 and cnt["decode_launches"][0] == 1, cnt
    assert sum(cnt["decode_row_tiles"][0]) == 0, cnt
    assert torch.isfinite(out).all()
    rng = np.random.default_rng(seed)
    rows = {0, 1, 31, 32, 33, 511, 512, 513, q_len // 2, q_len - 2, q_len - 1}
    rows |= set(int(r) for r in rng.integers(0, q_len, 24))
    _sampled_rows_check(lay, out, label, heads, sorted(r for r in rows if r < q_len))
