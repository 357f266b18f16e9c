"""GPU parity of paged decode attention against the oracle (row-normalised error
<= 2e-3, fp32 output), on every workload and on edge cases: ragged and tiny
contexts, windows at their boundaries, every query-row packing, poisoned
unused slots, page-table permutation and run-to-run bitwise determinism."""

import math

import numpy as np
import pytest
import torch

from fp8_kv_paged_amd import fkv, synth
from fp8_kv_paged_amd.layer import PagedLayer, to_dev_bits

import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def _check(lay, out, seqs=None, kv_heads=None, tol=parity.ATTN_TOL, label=""):
    gpu = out.cpu().numpy()
    worst = 0.0
    for b in (range(lay.num_seqs) if seqs is None else seqs):
        ref = parity.reference(lay, b, kv_heads)
        err = parity.row_errors(gpu[b], ref)
        worst = max(worst, float(err.max()))
    print(f"[decode parity] {label or lay.name}: max row error {worst:.3e}", flush=True)
    assert worst <= tol, (label or lay.name, worst)
    return worst


def _layer(lay, **kw):
    """Built PagedLayer, or None after checking that the layout rejects the shape (layouts 5
    and 6 read FP8 caches only, and layout 6 needs at least two 32-row tiles)."""
    nt = (lay.num_q_heads // lay.num_kv_heads * lay.q_len + 15) // 16
    fp8 = lay.cache_dtype == "fp8_e4m3fn"
    if (kw.get("layout") == 5 and not fp8) or (kw.get("layout") == 6 and (not fp8 or nt < 3)):
        with pytest.raises(fkv.FkvError) as e:
            PagedLayer(lay, **kw)
        assert e.value.status == fkv.EUNSUPPORTED
        return None
    return PagedLayer(lay, **kw).build()


def _workloads():
    yield "c1", synth.c1_layer
    yield "c2", synth.c2_layer
    yield "c3_8k_p32", lambda: synth.c3_layer(8192, 32)
    yield "c3_8k_p64", lambda: synth.c3_layer(8192, 64)
    yield "c3_32k_p32", lambda: synth.c3_layer(32768, 32)
    yield "c3_32k_p64", lambda: synth.c3_layer(32768, 64)
    yield "c4_sw_layer0", lambda: synth.c4_layer(0)
    yield "c4_global_layer3", lambda: synth.c4_layer(3)
    yield "c4_draft_layer48", lambda: synth.c4_layer(48)


@pytest.mark.parametrize("layout", [0, 3, 5, 6])
@pytest.mark.parametrize("name,make", list(_workloads()), ids=[n for n, _ in _workloads()])
def test_workload_parity(name, make, layout):
    lay = make()
    print(f"[decode parity] building {name} layout {layout}", flush=True)
    gl = _layer(lay, layout=layout)
    if gl is None:
        return
    fkv.reset_counters()
    out = gl.decode()
    torch.cuda.synchronize()
    cnt = fkv.get_counters()
    nt = (lay.num_q_heads // lay.num_kv_heads * lay.q_len + 15) // 16
    assert cnt["decode_launches"][0] == 1 and cnt["decode_row_tiles"][0][nt - 1] == 1, cnt
    _check(lay, out, label=f"{name} layout {layout}")


@pytest.fixture(scope="module")
def c5_fp8():
    lay = synth.c5_layer(12)
    print(f"[decode parity] building c5 fp8 (sum L = {int(lay.seq_lens.sum())})", flush=True)
    return lay, PagedLayer(lay).build()


def _c5_samples(lay):
    """The shortest, the longest and three sequences between them."""
    order = np.argsort(lay.seq_lens)
    n = len(order)
    return sorted({int(order[0]), int(order[n // 4]), int(order[n // 2]), int(order[(3 * n) // 4]), int(order[-1])})


@pytest.mark.parametrize("q_len", [12, 1])
def test_c5_batched_parity_fp8(c5_fp8, q_len):
    lay12, gl = c5_fp8
    lay = synth.c5_layer(q_len)
    assert np.array_equal(lay.block_table, lay12.block_table) and lay.k_scale == lay12.k_scale
    ddesc = fkv.make_decode_desc(lay.num_seqs, q_len, 72, lay.max_blocks, int(lay.seq_lens.max()))
    q = to_dev_bits(lay.q_bits(), "cuda")
    out = torch.empty((lay.num_seqs, q_len, 72, 128), dtype=torch.float32, device="cuda")
    ws = torch.zeros((max(16, fkv.decode_workspace_bytes(gl.cache, ddesc)),), dtype=torch.uint8, device="cuda")
    fkv.decode_attn(gl.cache, ddesc, q, gl.block_table, gl.seq_lens, gl.k_scale, gl.v_scale, out, ws)
    torch.cuda.synchronize()
    _check(lay, out, seqs=_c5_samples(lay), kv_heads=[0, 3, 7], label=f"c5 fp8 M={q_len}")


@pytest.mark.parametrize("q_len", [12, 1])
def test_c5_batched_parity_bf16_cache(q_len):
    lay = synth.c5_layer(q_len, cache_dtype="bf16")
    print(f"[decode parity] building c5 bf16 M={q_len} (sum L = {int(lay.seq_lens.sum())})", flush=True)
    gl = PagedLayer(lay).build()
    out = gl.decode()
    torch.cuda.synchronize()
    _check(lay, out, seqs=_c5_samples(lay), kv_heads=[1, 4, 7], label=f"c5 bf16 M={q_len}")


EDGE = [
    # (seq_lens, q_len, window_left, Hq, Hkv, block_size, cache_dtype)
    ([1], 1, -1, 9, 1, 32, "fp8_e4m3fn"),
    ([12], 12, -1, 18, 2, 64, "fp8_e4m3fn"),
    ([12, 13, 44], 12, 0, 18, 2, 32, "fp8_e4m3fn"),
    ([31, 32, 33, 63, 64, 65], 1, -1, 18, 2, 64, "fp8_e4m3fn"),
    ([511, 512, 513, 523, 524, 1000], 12, 511, 18, 2, 64, "fp8_e4m3fn"),
    ([700, 701], 5, 1, 9, 1, 32, "fp8_e4m3fn"),
    ([333], 2, -1, 3, 1, 32, "fp8_e4m3fn"),
    ([257, 1000], 7, -1, 16, 1, 64, "fp8_e4m3fn"),
    ([100], 3, 17, 12, 4, 32, "fp8_e4m3fn"),
    ([5000], 12, -1, 9, 1, 32, "fp8_e4m3fn"),
    ([16, 40, 300], 16, -1, 14, 2, 32, "fp8_e4m3fn"),  # q_len at its maximum, 112 packed rows
    ([16, 900], 16, 100, 4, 4, 64, "fp8_e4m3fn"),      # q_len 16 of one head per KV head: one 16-row tile
    ([12, 77, 300], 12, 64, 18, 2, 32, "bf16"),
    ([1, 33, 129], 1, -1, 18, 2, 64, "bf16"),
]


def _random_decode_case(seed):
    """A seeded random shape: 1-8 KV heads, 1-16 query heads per KV head, 1-16 query tokens
    (sometimes 17-64: a long window), page 32 or 64, global or a random window, 1-8 sequences up
    to 3k or 9k tokens, an FP8 or (a quarter of the cases) BF16 cache, layout 0, 3, 5 or 6, and an
    automatic or fixed split size."""
    rng = np.random.default_rng(seed)
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.integers(1, 17))
    M = int(rng.integers(1, 17)) if rng.random() < 0.85 else int(rng.integers(17, 65))
    bs = int(rng.choice([32, 64]))
    wl = -1 if rng.random() < 0.5 else int(rng.integers(0, 700))
    ns = int(rng.integers(1, 9))
    lens = [int(x) for x in rng.integers(M, int(rng.choice([3000, 9000])), ns)]
    dt = "bf16" if rng.random() < 0.25 else "fp8_e4m3fn"
    layout = int(rng.choice([0, 3, 5, 6]))
    st = int(rng.choice([0, 0, 1, 2, 4, 8, 12, 16]))
    lay = synth.tiny_layer(7000 + seed, lens, num_q_heads=G * hkv, num_kv_heads=hkv, block_size=bs, q_len=M,
                           window_left=wl, cache_dtype=dt, pool_slack=2.0)
    return lay, dict(layout=layout, split_tiles=st)


def _supported(lay, layout):
    """The documented shape rules: long windows (more than 16 query tokens or 112 packed rows)
    on FP8 caches with layout 0 or 5 only; layouts 5 and 6 read FP8 caches; layout 6 needs 33 to
    112 packed rows; layout 3 at most 112."""
    rows = lay.num_q_heads // lay.num_kv_heads * lay.q_len
    fp8 = lay.cache_dtype == "fp8_e4m3fn"
    long_rows = rows > 112 or lay.q_len > 16
    if long_rows:
        return fp8 and layout in (0, 5)
    if layout in (5, 6) and not fp8:
        return False
    return not (layout == 6 and rows <= 32)


@pytest.mark.parametrize("seed", range(300, 314))
def test_random_decode_shapes(seed):
    lay, kw = _random_decode_case(seed)
    label = (f"random decode {seed} ({lay.num_q_heads}/{lay.num_kv_heads} heads, q_len {lay.q_len}, page "
             f"{lay.block_size}, window {lay.window_left}, {lay.cache_dtype}, {kw})")
    if not _supported(lay, kw["layout"]):
        with pytest.raises(fkv.FkvError) as e:
            PagedLayer(lay, **kw)
        assert e.value.status == fkv.EUNSUPPORTED, label
        return
    gl = PagedLayer(lay, **kw).build()
    out = gl.decode().clone()
    torch.cuda.synchronize()
    _check(lay, out, label=label)


@pytest.mark.parametrize("layout", [3, 5])
@pytest.mark.parametrize("case", EDGE, ids=[f"L{c[0]}-M{c[1]}-w{c[2]}-{c[3]}x{c[4]}-p{c[5]}-{c[6][:4]}" for c in EDGE])
def test_edge_cases(case, layout):
    seq_lens, M, wl, hq, hkv, bs, dt = case
    lay = synth.tiny_layer(500 + len(seq_lens) * 7 + M, seq_lens, num_q_heads=hq, num_kv_heads=hkv, block_size=bs,
                           q_len=M, window_left=wl, cache_dtype=dt, pool_slack=2.0, outlier_rate=0.01)
    gl = _layer(lay, layout=layout)
    if gl is None:
        return
    out = gl.decode()
    torch.cuda.synchronize()
    _check(lay, out, label=f"{case} layout {layout}")


@pytest.mark.parametrize("layout", [3, 5, 6])
@pytest.mark.parametrize("split_tiles", [1, 2, 3, 8, 128])
def test_split_granularity(split_tiles, layout):
    lay = synth.tiny_layer(77, [2000, 64, 900], num_q_heads=18, num_kv_heads=2, block_size=32, q_len=12)
    gl = PagedLayer(lay, split_tiles=split_tiles, layout=layout).build()
    out = gl.decode()
    torch.cuda.synchronize()
    _check(lay, out, label=f"split_tiles={split_tiles} layout {layout}")


def test_page_table_permutation_is_bitwise_invariant_and_runs_are_deterministic():
    lay = synth.tiny_layer(91, [1500, 300], num_q_heads=18, num_kv_heads=2, block_size=32, q_len=12, pool_slack=3.0)
    a = PagedLayer(lay).build()
    out_a = a.decode().clone()
    out_a2 = a.decode().clone()
    perm = np.random.default_rng(3).permutation(lay.num_blocks).astype(np.int32)
    lay_b = synth.tiny_layer(91, [1500, 300], num_q_heads=18, num_kv_heads=2, block_size=32, q_len=12, pool_slack=3.0)
    lay_b.block_table = perm[lay.block_table]
    out_b = PagedLayer(lay_b).build().decode().clone()
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_a2)
    assert torch.equal(out_a, out_b)
    _check(lay, out_a, label="permutation")


def test_verify_rows_match_single_query_calls():
    """Row i of an M=12 call vs a q1 call at seq_len L-M+i+1 (reported; both gated at 2e-3)."""
    L, M = 777, 12
    lay = synth.tiny_layer(93, [L], num_q_heads=18, num_kv_heads=2, block_size=64, q_len=M)
    gl = PagedLayer(lay).build()
    out = gl.decode().cpu().numpy()
    worst = 0.0
    for i in range(M):
        d1 = fkv.make_decode_desc(1, 1, 18, lay.max_blocks, L - M + i + 1)
        q1 = to_dev_bits(lay.q_bits()[:, i:i + 1], "cuda")
        o1 = torch.empty((1, 1, 18, 128), dtype=torch.float32, device="cuda")
        sl = torch.tensor([L - M + i + 1], dtype=torch.int32, device="cuda")
        ws = torch.zeros((max(16, fkv.decode_workspace_bytes(gl.cache, d1)),), dtype=torch.uint8, device="cuda")
        fkv.decode_attn(gl.cache, d1, q1, gl.block_table, sl, gl.k_scale, gl.v_scale, o1, ws)
        worst = max(worst, float(np.abs(o1.cpu().numpy()[0, 0] - out[0, i]).max()))
    print(f"[decode] M12 row vs q1 call max abs difference {worst:.3e}", flush=True)
    _check(lay, torch.from_numpy(out), label="m12 vs q1")


def test_rows_without_visible_keys_are_zero():
    """seq_len below q_len: rows at negative positions see nothing and are written as 0."""
    lay = synth.tiny_layer(95, [12], num_q_heads=18, num_kv_heads=2, block_size=32, q_len=12)
    gl = PagedLayer(lay).build()
    gl.seq_lens.fill_(5)
    out = gl.decode().cpu().numpy()
    assert np.all(out[0, :7] == 0.0)
    assert np.all(np.isfinite(out))


def test_packing_beyond_the_decode_tiles():
    """10 query heads per KV head x 12 rows = 120 packed rows: more than the row-group kernel
    compiles (it fails closed), served by the 32-row kernel's long-window plan."""
    lay = synth.tiny_layer(97, [64, 700], num_q_heads=20, num_kv_heads=2, block_size=32, q_len=12)
    for layout in (3, 6):
        with pytest.raises(fkv.FkvError) as e:
            PagedLayer(lay, layout=layout)
        assert e.value.status == fkv.EUNSUPPORTED
    lay16 = synth.tiny_layer(97, [64], num_q_heads=20, num_kv_heads=2, block_size=32, q_len=12, cache_dtype="bf16")
    with pytest.raises(fkv.FkvError) as e:
        PagedLayer(lay16)
    assert e.value.status == fkv.EUNSUPPORTED
    out = PagedLayer(lay).build().decode().clone()
    torch.cuda.synchronize()
    _check(lay, out, label="120 packed rows")


def test_fused_split_merge_is_deterministic_and_leaves_counters_zero():
    """Layout 5 merges the splits inside the kernel when the grid fits on the chip: repeated
    calls give bitwise-identical outputs and return the workspace's counters to zero."""
    lay = synth.tiny_layer(99, [3000] * 8, num_q_heads=72, num_kv_heads=8, block_size=64, q_len=12)
    gl = PagedLayer(lay, layout=5).build()
    outs = [gl.decode().clone() for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    pairs = lay.num_seqs * lay.num_kv_heads
    nws = fkv.decode_workspace_bytes(gl.cache, gl.ddesc)
    ctl_bytes = pairs * 256
    assert torch.count_nonzero(gl.workspace[nws - ctl_bytes:nws]).item() == 0
    _check(lay, outs[0], label="fused split merge")


@pytest.mark.parametrize("row_groups", [1, 2, 4])
@pytest.mark.parametrize("name,make", [("c2", synth.c2_layer), ("c3_8k_p64", lambda: synth.c3_layer(8192, 64)),
                                       ("c4_sw_layer0", lambda: synth.c4_layer(0))], ids=["c2", "c3_8k_p64", "c4_sw"])
def test_row_groups_parity(name, make, row_groups):
    """Layout 5 with the query rows of a split cut over 1, 2 or 4 work groups."""
    lay = make()
    gl = PagedLayer(lay, layout=5, row_groups=row_groups).build()
    out = gl.decode()
    torch.cuda.synchronize()
    _check(lay, out, label=f"{name} layout 5 row groups {row_groups}")


@pytest.mark.parametrize("name,make,q_len", [
    ("c2", synth.c2_layer, 12), ("c3_8k_p64", lambda: synth.c3_layer(8192, 64), 12),
    ("c4_sw_layer0", lambda: synth.c4_layer(0), 12),
    ("ragged_m6", lambda: synth.tiny_layer(121, [3000, 40, 700], num_q_heads=18, num_kv_heads=2, block_size=32,
                                            q_len=6, outlier_rate=0.01), 6),
    ("ragged_m12_p64", lambda: synth.tiny_layer(123, [5000, 13, 12, 257], num_q_heads=72, num_kv_heads=8,
                                                block_size=64, q_len=12), 12)],
    ids=["c2", "c3_8k_p64", "c4_sw", "ragged_m6", "ragged_m12_p64"])
@pytest.mark.parametrize("split_tiles", [0, 4])
def test_two_row_tiles_per_wave_is_bitwise_layout5(name, make, q_len, split_tiles):
    """Layout 6 (four waves, each holding two row tiles) does per row tile exactly the
    arithmetic of layout 5 with two row tiles per work group: outputs are bitwise equal."""
    lay = make()
    rows = lay.num_q_heads // lay.num_kv_heads * q_len
    rt_total = 1 if rows <= 32 else (2 if rows <= 64 else 4)
    out6 = PagedLayer(lay, layout=6, split_tiles=split_tiles).build().decode().clone()
    out5 = PagedLayer(lay, layout=5, row_groups=rt_total // 2, split_tiles=split_tiles).build().decode().clone()
    torch.cuda.synchronize()
    assert torch.equal(out5, out6), name
    _check(lay, out6, label=f"{name} layout 6 split_tiles {split_tiles}")


@pytest.mark.parametrize("window_left,L", [(-1, 3000), (511, 2000), (63, 700), (-1, 40)])
@pytest.mark.parametrize("split_tiles", [4, 8])
def test_row_exact_rows_equal_single_query_calls(window_left, L, split_tiles):
    """Row-exact mode: row i of an M=12 call is bitwise equal to a q1 call at seq_len
    L - 12 + i + 1 (same cache, same split_tiles)."""
    M = 12
    lay = synth.tiny_layer(131 + L + window_left, [L], num_q_heads=18, num_kv_heads=2, block_size=64, q_len=M,
                           window_left=window_left, outlier_rate=0.01)
    gl = PagedLayer(lay, split_tiles=split_tiles, row_exact=1).build()
    out = gl.decode().clone()
    for i in range(M):
        d1 = fkv.make_decode_desc(1, 1, 18, lay.max_blocks, L, window_left, lay.softmax_scale,
                                  split_tiles=split_tiles, row_exact=1)
        q1 = to_dev_bits(lay.q_bits()[:, i:i + 1], "cuda")
        o1 = torch.empty((1, 1, 18, 128), dtype=torch.float32, device="cuda")
        sl = torch.tensor([L - M + i + 1], dtype=torch.int32, device="cuda")
        ws = torch.zeros((max(16, fkv.decode_workspace_bytes(gl.cache, d1)),), dtype=torch.uint8, device="cuda")
        fkv.decode_attn(gl.cache, d1, q1, gl.block_table, sl, gl.k_scale, gl.v_scale, o1, ws)
        torch.cuda.synchronize()
        assert torch.equal(o1[0, 0], out[0, i]), (i, float((o1[0, 0] - out[0, i]).abs().max()))
    _check(lay, out, label=f"row exact L {L} window {window_left} split_tiles {split_tiles}")


def test_row_exact_full_layer():
    """Row-exact mode on the 72/8-head layer at 8k (two row tiles per work group, four key lanes)."""
    lay = synth.c3_layer(8192, 64)
    gl = PagedLayer(lay, split_tiles=16, row_exact=1).build()
    out = gl.decode()
    torch.cuda.synchronize()
    _check(lay, out, label="c3_8k_p64 row exact")


def test_cross_xcd_split_merge_alternating_inputs():
    """18 query / 2 KV heads at 8k (two (sequence, KV head) pairs): the splits of a pair run on
    different XCDs and merge inside the kernel. Two different query tensors alternate on one
    workspace for 1,000 calls; every output must equal bit for bit the first output computed
    for the same input, so a partial left from the previous call (a stale read across XCDs)
    would show. Bounded: the comparison runs after the calls, up to the first mismatch."""
    lay = synth.c4_layer(3)
    assert lay.window_left < 0 and lay.num_kv_heads == 2
    gl = PagedLayer(lay, layout=5).build()
    plan_fused = fkv.decode_workspace_bytes(gl.cache, gl.ddesc) > 0
    assert plan_fused
    q_a = gl.q.clone()
    rng = np.random.default_rng(17)
    q_b = to_dev_bits(synth.f32_to_bf16_bits(rng.standard_normal(tuple(gl.q.shape)).astype(np.float32)), "cuda")
    n = 1000
    hist = torch.empty((n,) + tuple(gl.out.shape), dtype=torch.float32, device="cuda")
    fkv.reset_counters()
    for i in range(n):
        gl.q = q_a if i % 2 == 0 else q_b
        gl.decode()
        hist[i].copy_(gl.out)
    torch.cuda.synchronize()
    cnt = fkv.get_counters()
    assert cnt["decode_launches"][0] == n and cnt["decode_combine_launches"] == 0, cnt  # merged in-kernel
    assert not torch.equal(hist[0], hist[1])
    for i in range(2, n):
        assert torch.equal(hist[i], hist[i % 2]), f"call {i} differs from the first call with the same input"
    print(f"[decode] cross-XCD merge: {n} alternating calls bitwise stable", flush=True)
    _check(lay, hist[0], label="alternating inputs, first call")
    nws = fkv.decode_workspace_bytes(gl.cache, gl.ddesc)
    assert torch.count_nonzero(gl.workspace[nws - 2 * 256:nws]).item() == 0
