"""GPU parity of the fused insert + decode entry point (fkv_insert_decode): the pool bytes
it writes equal fkv_insert's for the same tokens, its output equals fkv_decode_attn's
after that insert bit for bit, and both are checked against the oracle (row-normalised
error <= 2e-3). Cases put the new tokens across tile, page and split boundaries, below
position 0 (seq_len < q_len), in sliding windows and in every row-group split."""

import dataclasses

import numpy as np
import pytest
import torch

from fp8_kv_paged_amd import fkv, synth
from fp8_kv_paged_amd.layer import PagedLayer
from oracle import attention

import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def _reference(lay, b):
    """Oracle output of sequence b; with seq_len L < q_len the first q_len - L rows sit at
    negative positions (no visible key: zeros) and the rest are the oracle over q_len = L."""
    M, L = lay.q_len, int(lay.seq_lens[b])
    if L >= M:
        return parity.reference(lay, b)
    G = lay.num_q_heads // lay.num_kv_heads
    k, v = parity.logical_kv(lay, b)
    q = parity.q_f64(lay, b)
    out = np.zeros(q.shape)
    for g in range(lay.num_kv_heads):
        sl = slice(g * G, (g + 1) * G)
        out[M - L:, sl] = attention.decode_attention(q[M - L:, sl], k[:, g:g + 1], v[:, g:g + 1], L,
                                                     lay.window_left, lay.softmax_scale)
    return out


def _check(lay, out, label):
    gpu = out.cpu().numpy()
    worst = 0.0
    for b in range(lay.num_seqs):
        L = int(lay.seq_lens[b])
        if L < lay.q_len:
            assert np.all(gpu[b, :lay.q_len - L] == 0.0), (label, b)
        worst = max(worst, float(parity.row_errors(gpu[b], _reference(lay, b)).max()))
    print(f"[insert_decode parity] {label}: max row error {worst:.3e}", flush=True)
    assert worst <= parity.ATTN_TOL, (label, worst)


def _fused_vs_separate(lay, label, **kw):
    fused = PagedLayer(lay, **kw)
    fused.prefill()
    fused.stage_new_tokens()
    # the fused call runs the 32-row kernel; with the automatic layout a separate q1 decode
    # would run the row-group kernel, so the separate reference names layout 5
    sep_kw = dict(kw)
    if sep_kw.get("layout", 0) == 0:
        sep_kw["layout"] = 5
    sep = PagedLayer(lay, **sep_kw).build()
    before = fkv.get_counters()["insert_decode_launches"]
    out_f = fused.insert_decode().clone()
    out_s = sep.decode().clone()
    torch.cuda.synchronize()
    assert fkv.get_counters()["insert_decode_launches"] == before + 1
    assert torch.equal(fused.k_pool, sep.k_pool), f"{label}: K pool differs from fkv_insert's"
    assert torch.equal(fused.v_pool, sep.v_pool), f"{label}: V pool differs from fkv_insert's"
    assert torch.equal(out_f, out_s), f"{label}: output differs from insert + decode"
    _check(lay, out_f, label)
    return fused


def _workloads():
    yield "c1", synth.c1_layer
    yield "c2", synth.c2_layer
    yield "c3_8k_p32", lambda: synth.c3_layer(8192, 32)
    yield "c3_8k_p64", lambda: synth.c3_layer(8192, 64)
    yield "c3_32k_p64", lambda: synth.c3_layer(32768, 64)
    yield "c4_sw_layer0", lambda: synth.c4_layer(0)
    yield "c4_draft_layer48", lambda: synth.c4_layer(48)


@pytest.mark.parametrize("name,make", list(_workloads()), ids=[n for n, _ in _workloads()])
def test_workload_fused_equals_separate(name, make):
    _fused_vs_separate(make(), name)


@pytest.mark.parametrize("split_tiles", [0, 1, 2, 8, 12])
@pytest.mark.parametrize("block_size", [32, 64])
def test_ragged_boundaries(block_size, split_tiles):
    """New positions straddling 32-key tiles, pages and (split_tiles 1, 2) splits; sequences
    shorter than q_len (positions below 0 are not stored). With 8 and 12 tiles per split the
    new keys fall in the first, second or third ring step of their split (the stores must
    complete before that step is requested)."""
    lay = synth.tiny_layer(401 + block_size, [40, 70, 64, 129, 700, 12, 5, 1, 300, 1000], num_q_heads=18,
                           num_kv_heads=2, block_size=block_size, q_len=12, pool_slack=2.0, outlier_rate=0.01)
    _fused_vs_separate(lay, f"ragged p{block_size} split_tiles {split_tiles}", split_tiles=split_tiles)


@pytest.mark.parametrize("layout,row_groups", [(5, 1), (5, 2), (5, 4), (6, 0)])
def test_row_groups(layout, row_groups):
    lay = synth.tiny_layer(409, [3000, 257, 33], num_q_heads=72, num_kv_heads=8, block_size=64, q_len=12)
    _fused_vs_separate(lay, f"layout {layout} row groups {row_groups}", layout=layout, row_groups=row_groups)


@pytest.mark.parametrize("name,make", [("c3_8k_p64", lambda: synth.c3_layer(8192, 64)), ("c2", synth.c2_layer)],
                         ids=["c3_8k_p64", "c2"])
def test_layout6_fused(name, make):
    _fused_vs_separate(make(), f"{name} layout 6", layout=6)


@pytest.mark.parametrize("window_left", [0, 11, 63, 511])
def test_sliding_windows(window_left):
    lay = synth.tiny_layer(411 + window_left, [600, 40, 513], num_q_heads=18, num_kv_heads=2, block_size=64, q_len=12,
                           window_left=window_left)
    _fused_vs_separate(lay, f"window {window_left}")


@pytest.mark.parametrize("window_left", [-1, 3, 40])
def test_long_row_windows(window_left):
    """16 query heads per KV head at q_len 12 (192 packed rows): each row group's key range is
    clipped to the keys its rows can see, and every row group stores the new tokens inside its
    own range before it reads them; together they store every new token."""
    lay = synth.tiny_layer(431 + window_left, [600, 40, 513, 9], num_q_heads=32, num_kv_heads=2, block_size=64,
                           q_len=12, window_left=window_left)
    _fused_vs_separate(lay, f"long rows, window {window_left}")


def test_row_exact_mode():
    lay = synth.tiny_layer(419, [3000, 257, 12, 5], num_q_heads=18, num_kv_heads=2, block_size=64, q_len=12)
    _fused_vs_separate(lay, "row exact", split_tiles=8, row_exact=1)


def test_q1_decode_and_fused_share_one_workspace():
    """Automatic layout, one query row per sequence: fkv_decode_attn runs the row-group kernel,
    fkv_insert_decode the 32-row kernel with its in-kernel merge counters. Alternating calls on
    one workspace stay correct and leave the counters zero."""
    lay = synth.tiny_layer(421, [3000, 257], num_q_heads=18, num_kv_heads=2, block_size=64, q_len=1)
    gl = PagedLayer(lay)
    gl.prefill()
    gl.stage_new_tokens()
    nws = fkv.decode_workspace_bytes(gl.cache, gl.ddesc)
    ctl = lay.num_seqs * lay.num_kv_heads * 256
    for rep in range(3):
        out_f = gl.insert_decode().clone()
        out_d = gl.decode().clone()
        torch.cuda.synchronize()
        assert torch.count_nonzero(gl.workspace[nws - ctl:nws]).item() == 0, rep
        _check(lay, out_f, f"q1 fused {rep}")
        _check(lay, out_d, f"q1 decode {rep}")


@pytest.mark.parametrize("hq,hkv,block_size", [(14, 2, 32), (4, 4, 64)])
def test_max_query_length(hq, hkv, block_size):
    """q_len 16, the largest the fused call stages: every thread of the group holds a new-token
    chunk (112 packed rows at 7 heads per KV head; one 16-row tile at one head), with
    sequences shorter than, equal to and longer than q_len."""
    lay = synth.tiny_layer(431 + hq, [16, 9, 40, 700], num_q_heads=hq, num_kv_heads=hkv, block_size=block_size,
                           q_len=16, pool_slack=2.0, outlier_rate=0.01)
    _fused_vs_separate(lay, f"q_len 16, {hq}/{hkv} heads, page {block_size}")


def _random_case(seed):
    """A seeded random shape: 1-8 KV heads, 1-16 query heads per KV head, 1-16 new tokens,
    page 32 or 64, global or a random window, 1-12 sequences up to 3k or 9k tokens (some
    shorter than q_len), automatic layout, layout 5 or (with 33-112 packed rows) layout 6, and
    an automatic or fixed split size."""
    rng = np.random.default_rng(seed)
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.integers(1, 17))
    M = int(rng.integers(1, 17))
    bs = int(rng.choice([32, 64]))
    wl = -1 if rng.random() < 0.5 else int(rng.integers(0, 700))
    ns = int(rng.integers(1, 13))
    lens = [int(x) for x in rng.integers(0, int(rng.choice([3000, 9000])), ns)]
    if rng.random() < 0.3:
        lens[0] = int(rng.integers(0, M + 1))
    layout = int(rng.choice([0, 5, 6]))
    st = int(rng.choice([0, 0, 1, 2, 4, 8, 12, 16]))
    if layout == 6 and not 32 < G * M <= 112:
        layout = 5
    lay = synth.tiny_layer(9000 + seed, lens, num_q_heads=G * hkv, num_kv_heads=hkv, block_size=bs, q_len=M,
                           window_left=wl, pool_slack=2.0)
    return lay, dict(layout=layout, split_tiles=st)


@pytest.mark.parametrize("seed", range(200, 212))
def test_random_shapes(seed):
    lay, kw = _random_case(seed)
    _fused_vs_separate(lay, f"random shape {seed} ({lay.num_q_heads}/{lay.num_kv_heads} heads, q_len {lay.q_len}, "
                            f"page {lay.block_size}, window {lay.window_left}, {kw})", **kw)


def test_single_query():
    lay = synth.tiny_layer(413, [1, 32, 33, 300], num_q_heads=18, num_kv_heads=2, block_size=32, q_len=1)
    _fused_vs_separate(lay, "q1")


def test_repeated_steps_with_growing_sequences():
    """Three decode steps in a row on one layer: each fused call inserts at the new tail and
    attends over everything inserted so far, bitwise equal to insert + decode."""
    final = synth.tiny_layer(415, [524, 114], num_q_heads=18, num_kv_heads=2, block_size=32, q_len=12, pool_slack=2.0)
    fused, sep = PagedLayer(final), PagedLayer(final)
    for gl in (fused, sep):
        for b in range(final.num_seqs):
            gl.insert_tokens(b, 0, int(final.seq_lens[b]) - 36)
    for step in range(3):
        lay = dataclasses.replace(final, seq_lens=(final.seq_lens - 12 * (2 - step)).astype(np.int32))
        for gl in (fused, sep):
            gl.lay = lay
            gl.seq_lens.copy_(torch.from_numpy(lay.seq_lens))
        fused.stage_new_tokens()
        out_f = fused.insert_decode().clone()
        sep.stage_step()
        sep.insert_step()
        out_s = sep.decode().clone()
        torch.cuda.synchronize()
        assert torch.equal(fused.k_pool, sep.k_pool) and torch.equal(fused.v_pool, sep.v_pool), step
        assert torch.equal(out_f, out_s), step
        _check(lay, out_f, f"step {step}")


def test_rejects_other_layouts_and_bf16():
    lay = synth.tiny_layer(417, [100], num_q_heads=18, num_kv_heads=2, block_size=32, q_len=12)
    gl = PagedLayer(lay, layout=3)
    gl.prefill()
    gl.stage_new_tokens()
    with pytest.raises(fkv.FkvError) as e:
        gl.insert_decode()
    assert e.value.status == fkv.EUNSUPPORTED
    lay16 = synth.tiny_layer(417, [100], num_q_heads=18, num_kv_heads=2, block_size=32, q_len=12, cache_dtype="bf16")
    gl16 = PagedLayer(lay16)
    gl16.prefill()
    gl16.stage_new_tokens()
    with pytest.raises(fkv.FkvError) as e:
        gl16.insert_decode()
    assert e.value.status == fkv.EUNSUPPORTED
