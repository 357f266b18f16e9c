"""Host-only checks of the C ABI: the library loads, exports every entry point the
header declares, sizes match the pages' payload figures, and invalid calls fail
closed with the documented codes before any HIP call (no GPU needed)."""

import ctypes
import json
import os
import re

import pytest

from fp8_kv_paged_amd import fkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fkv.h")
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "payload.json")))


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(fkv_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) == 12, names
    L = fkv.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code in (fkv.OK, fkv.EINVAL, fkv.EUNSUPPORTED, fkv.EWORKSPACE, fkv.EHIP):
        assert fkv.status_string(code)
    assert fkv.status_string(99) == "unknown status"


def test_cache_bytes_matches_payload_pins():
    for dt, key in (("fp8_e4m3fn", "fp8_e4m3fn"), ("bf16", "bf16")):
        for bs in (32, 64):
            k, v = fkv.cache_bytes(fkv.make_cache_desc(10, bs, 8, dt))
            assert k == v
            per_token = (k + v) // (10 * bs)
            assert per_token == GOLD["bytes_per_token_layer"][key]


@pytest.mark.parametrize("field,value,code", [
    ("block_size", 16, fkv.EUNSUPPORTED), ("block_size", 128, fkv.EUNSUPPORTED), ("head_dim", 64, fkv.EUNSUPPORTED),
    ("cache_dtype", 7, fkv.EUNSUPPORTED), ("num_blocks", 0, fkv.EINVAL), ("num_kv_heads", 0, fkv.EINVAL),
    ("block_size", 0, fkv.EINVAL),
])
def test_bad_cache_desc(field, value, code):
    d = fkv.make_cache_desc(4, 32, 2)
    setattr(d, field, value)
    with pytest.raises(fkv.FkvError) as e:
        fkv.cache_bytes(d)
    assert e.value.status == code


def _fake_cache(num_blocks=8, bs=32, hkv=2, dt="fp8_e4m3fn"):
    """A handle over fake aligned addresses: valid for host-only calls, never launched."""
    d = fkv.make_cache_desc(num_blocks, bs, hkv, dt)
    c = fkv.Cache()
    rc = fkv.lib().fkv_init_cache(ctypes.byref(d), ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.byref(c))
    assert rc == fkv.OK
    return c


def test_init_cache_rejects_null_and_misaligned_pools():
    d = fkv.make_cache_desc(8, 32, 2)
    c = fkv.Cache()
    L = fkv.lib()
    assert L.fkv_init_cache(ctypes.byref(d), None, ctypes.c_void_p(0x1000), ctypes.byref(c)) == fkv.EINVAL
    assert L.fkv_init_cache(ctypes.byref(d), ctypes.c_void_p(0x1001), ctypes.c_void_p(0x1000), ctypes.byref(c)) == fkv.EINVAL
    assert L.fkv_init_cache(ctypes.byref(d), ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), None) == fkv.EINVAL


def _ws(c, **kw):
    args = dict(num_seqs=1, q_len=12, num_q_heads=18, max_blocks_per_seq=8, max_seq_len=256)
    args.update(kw)
    return fkv.decode_workspace_bytes(c, fkv.make_decode_desc(**args))


def test_decode_validation_codes():
    c = _fake_cache()
    assert _ws(c) >= 0
    bad = [
        (dict(q_len=0), fkv.EINVAL), (dict(q_len=4097), fkv.EUNSUPPORTED), (dict(num_q_heads=17), fkv.EINVAL),
        (dict(q_len=17, layout=3), fkv.EUNSUPPORTED),  # long windows: the 32-row kernel only
        (dict(num_q_heads=20, q_len=12, layout=3), fkv.EUNSUPPORTED),  # 10 heads per KV head x 12 rows > 112
        (dict(layout=1), fkv.EINVAL), (dict(layout=2), fkv.EINVAL), (dict(layout=4), fkv.EINVAL),  # no such layouts
        (dict(max_seq_len=257), fkv.EINVAL),  # beyond max_blocks_per_seq * block_size
        (dict(max_blocks_per_seq=0), fkv.EINVAL), (dict(num_seqs=-1), fkv.EINVAL),
        (dict(window_left=-2), fkv.EINVAL), (dict(softmax_scale=0.0), fkv.EINVAL),
        (dict(softmax_scale=float("nan")), fkv.EINVAL), (dict(split_tiles=-1), fkv.EINVAL),
    ]
    for kw, code in bad:
        with pytest.raises(fkv.FkvError) as e:
            _ws(c, **kw)
        assert e.value.status == code, kw


def test_workspace_zero_for_single_split_and_sized_for_many():
    c = _fake_cache(num_blocks=4096, bs=64, hkv=8)
    for layout in (0, 3, 5):
        one = _ws(c, num_q_heads=72, max_blocks_per_seq=64, max_seq_len=4096, split_tiles=128, layout=layout)
        assert one == 0, layout
    # every work group stages at most 128 page-table entries per split
    for layout in (3, 5):
        with pytest.raises(fkv.FkvError) as e:
            _ws(c, num_q_heads=72, max_blocks_per_seq=128, max_seq_len=8192, split_tiles=256, layout=layout)
        assert e.value.status == fkv.EUNSUPPORTED
    many = _ws(c, num_q_heads=72, max_blocks_per_seq=128, max_seq_len=8192, split_tiles=8, layout=3)
    # 32 splits x 8 KV heads x 128 padded rows (four row groups of two 16-row tiles) x (128 + 2) fp32
    assert many == 32 * 8 * 128 * 130 * 4
    # the 32-row kernel: 128 padded rows per partial, plus 256 bytes of merge counters per pair
    m32 = _ws(c, num_q_heads=72, max_blocks_per_seq=128, max_seq_len=8192, split_tiles=8, layout=5)
    assert m32 == 32 * 8 * 128 * 130 * 4 + 8 * 256


def test_calls_fail_closed_without_touching_the_gpu():
    L = fkv.lib()
    c = _fake_cache()
    d = fkv.make_decode_desc(1, 12, 18, 8, 256)
    dev = ctypes.c_void_p(0x300000)
    # missing workspace for a multi-split plan
    d.split_tiles = 1
    rc = L.fkv_decode_attn(ctypes.byref(c), ctypes.byref(d), dev, dev, dev, dev, dev, dev, None, 0, None)
    assert rc == fkv.EWORKSPACE
    # null q
    rc = L.fkv_decode_attn(ctypes.byref(c), ctypes.byref(d), None, dev, dev, dev, dev, dev, dev, 1 << 30, None)
    assert rc == fkv.EINVAL
    # misaligned out
    rc = L.fkv_decode_attn(ctypes.byref(c), ctypes.byref(d), dev, dev, dev, dev, dev, ctypes.c_void_p(0x300004), dev,
                           1 << 30, None)
    assert rc == fkv.EINVAL
    # insert: negative count, null slots, misaligned k
    assert L.fkv_insert(ctypes.byref(c), dev, dev, dev, -1, dev, dev, None) == fkv.EINVAL
    assert L.fkv_insert(ctypes.byref(c), dev, dev, None, 4, dev, dev, None) == fkv.EINVAL
    assert L.fkv_insert(ctypes.byref(c), ctypes.c_void_p(0x300002), dev, dev, 4, dev, dev, None) == fkv.EINVAL
    # zero tokens / zero sequences are no-ops that succeed without a launch
    assert L.fkv_insert(ctypes.byref(c), None, None, None, 0, None, None, None) == fkv.OK
    d0 = fkv.make_decode_desc(0, 12, 18, 8, 256)
    assert L.fkv_decode_attn(ctypes.byref(c), ctypes.byref(d0), None, None, None, None, None, None, None, 0, None) == fkv.OK
    # a tampered handle is rejected
    c.pool_bytes += 1
    assert L.fkv_insert(ctypes.byref(c), dev, dev, dev, 4, dev, dev, None) == fkv.EINVAL


def test_layout6_plan_rules():
    """Layout 6 (two row tiles per wave): FP8 cache, at least two 32-row tiles, row groups
    fixed at half the row tiles; its workspace equals layout 5's with the same row groups."""
    c = _fake_cache(num_blocks=4096, bs=64, hkv=8)
    kw = dict(num_q_heads=72, max_blocks_per_seq=128, max_seq_len=8192)
    assert _ws(c, layout=6, **kw) == _ws(c, layout=5, row_groups=2, **kw)
    assert _ws(c, layout=6, q_len=6, **kw) == _ws(c, layout=5, row_groups=1, q_len=6, **kw)
    for bad in (dict(layout=6, q_len=1), dict(layout=6, row_groups=1), dict(layout=6, row_groups=4)):
        with pytest.raises(fkv.FkvError) as e:
            _ws(c, **kw, **bad)
        assert e.value.status == fkv.EUNSUPPORTED, bad
    with pytest.raises(fkv.FkvError) as e:
        _ws(_fake_cache(num_blocks=4096, bs=64, hkv=8, dt="bf16"), layout=6, **kw)
    assert e.value.status == fkv.EUNSUPPORTED
    with pytest.raises(fkv.FkvError) as e:
        _ws(c, layout=7, **kw)
    assert e.value.status == fkv.EINVAL


def test_row_exact_plan_rules():
    """Row-exact mode: explicit split_tiles (a multiple of 4), FP8 cache, layout 0 or 5, at most two
    row tiles per work group."""
    c = _fake_cache(num_blocks=4096, bs=64, hkv=8)
    kw = dict(num_q_heads=72, max_blocks_per_seq=128, max_seq_len=8192)
    assert _ws(c, row_exact=1, split_tiles=16, **kw) == _ws(c, row_groups=2, split_tiles=16, **kw)
    assert _ws(c, row_exact=1, split_tiles=16, q_len=1, **kw) > 0
    for bad, code in ((dict(split_tiles=0), fkv.EINVAL), (dict(split_tiles=6), fkv.EINVAL),
                      (dict(split_tiles=8, layout=3), fkv.EUNSUPPORTED),
                      (dict(split_tiles=8, layout=6), fkv.EUNSUPPORTED),
                      (dict(split_tiles=8, row_groups=1), fkv.EUNSUPPORTED)):
        with pytest.raises(fkv.FkvError) as e:
            _ws(c, row_exact=1, **kw, **bad)
        assert e.value.status == code, bad
    with pytest.raises(fkv.FkvError) as e:
        _ws(_fake_cache(num_blocks=4096, bs=64, hkv=8, dt="bf16"), row_exact=1, split_tiles=8, **kw)
    assert e.value.status == fkv.EUNSUPPORTED
    # sliding windows: aligned splits may straddle one more boundary
    # (5 -> 6 splits of partials; the 256 bytes of merge counters per pair do not scale)
    ctl = 8 * 256
    sw = _ws(c, row_exact=1, split_tiles=4, window_left=511, **kw)
    assert sw - ctl == (_ws(c, row_groups=2, split_tiles=4, window_left=511, **kw) - ctl) * 6 // 5


def test_automatic_q1_workspace_covers_both_kernels():
    """Automatic layout, FP8, one 16-row tile (q1 at 9 heads per KV head): fkv_decode_attn runs the
    row-group kernel and fkv_insert_decode the 32-row kernel on the same workspace, so its size is
    the larger partial region of the two plus the 32-row kernel's merge counters."""
    c = _fake_cache(num_blocks=4096, bs=64, hkv=8)
    for ctx, nseq in ((8192, 1), (32768, 1), (2048, 4)):
        kw = dict(num_seqs=nseq, num_q_heads=72, max_blocks_per_seq=(ctx + 63) // 64, max_seq_len=ctx, q_len=1)
        ctl = (nseq * 8 * 256 + 255) // 256 * 256
        rows = _ws(c, layout=3, **kw)
        m32 = _ws(c, layout=5, **kw)
        assert _ws(c, **kw) == max(rows, m32 - ctl) + ctl, (ctx, nseq)
    # more rows, row-exact mode and BF16 caches keep their single plan
    kw = dict(num_q_heads=72, max_blocks_per_seq=128, max_seq_len=8192)
    assert _ws(c, q_len=2, **kw) == _ws(c, q_len=2, layout=5, **kw)
    assert _ws(c, q_len=1, row_exact=1, split_tiles=16, **kw) == _ws(c, q_len=1, layout=5, row_exact=1,
                                                                     split_tiles=16, **kw)
    c16 = _fake_cache(num_blocks=4096, bs=64, hkv=8, dt="bf16")
    assert _ws(c16, q_len=1, **kw) == _ws(c16, q_len=1, layout=3, **kw)


def test_bf16_output_plan_rules():
    """BF16 output: every layout (0, 3, 5, 6) writes it with the same plan and workspace as
    fp32; unknown output types fail closed."""
    c = _fake_cache(num_blocks=4096, bs=64, hkv=8)
    kw = dict(num_q_heads=72, max_blocks_per_seq=128, max_seq_len=8192)
    for layout in (0, 3, 5, 6):
        for q_len in (1, 12):
            if layout == 6 and q_len == 1:
                continue
            assert (_ws(c, layout=layout, q_len=q_len, out_dtype=fkv.OUT_BF16, **kw)
                    == _ws(c, layout=layout, q_len=q_len, **kw)), (layout, q_len)
    for bad in (dict(out_dtype=0), dict(out_dtype=3)):
        with pytest.raises(fkv.FkvError) as e:
            _ws(c, **kw, **bad)
        assert e.value.status == fkv.EUNSUPPORTED, bad


def test_long_query_window_plan_rules():
    """Chunked prefill (q_len > 16, or more than 112 packed rows): FP8 cache, layout 0 or 5,
    automatic row groups, no row-exact mode; ceil(rows / 64) work groups of 64 rows per split,
    merged by the combine kernel."""
    c = _fake_cache(num_blocks=4096, bs=64, hkv=8)
    kw = dict(num_q_heads=72, max_blocks_per_seq=256, max_seq_len=16384)
    for q_len in (13, 17, 128, 512, 4096):
        n = _ws(c, q_len=q_len, **kw)
        assert n == _ws(c, q_len=q_len, layout=5, **kw)
        rows_pad = (9 * q_len + 63) // 64 * 64
        ctl = 8 * 256
        parts = (n - ctl) // (rows_pad * 130 * 4)   # fp32 partial rows plus (m, l) per row
        assert n == 0 or (parts >= 1 and n - ctl >= parts * rows_pad * 130 * 4), q_len
    for bad in (dict(layout=3), dict(layout=6), dict(row_groups=2), dict(row_exact=1, split_tiles=8)):
        with pytest.raises(fkv.FkvError) as e:
            _ws(c, q_len=64, **kw, **bad)
        assert e.value.status == fkv.EUNSUPPORTED, bad
    with pytest.raises(fkv.FkvError) as e:
        _ws(_fake_cache(num_blocks=4096, bs=64, hkv=8, dt="bf16"), q_len=64, **kw)
    assert e.value.status == fkv.EUNSUPPORTED
    # the fused insert stages at most 16 tokens
    L = fkv.lib()
    dev = ctypes.c_void_p(0x300000)
    d = fkv.make_decode_desc(1, 17, 72, 256, 16384)
    assert L.fkv_insert_decode(ctypes.byref(c), ctypes.byref(d), dev, dev, dev, dev, dev, dev, dev, dev, dev, 1 << 30,
                               None) == fkv.EUNSUPPORTED


def test_insert_decode_fails_closed_without_touching_the_gpu():
    L = fkv.lib()
    c = _fake_cache()
    d = fkv.make_decode_desc(1, 12, 18, 8, 256)
    dev = ctypes.c_void_p(0x300000)
    call = lambda cache, desc, kn, vn, ws=dev, nws=1 << 30: L.fkv_insert_decode(
        ctypes.byref(cache), ctypes.byref(desc), dev, kn, vn, dev, dev, dev, dev, dev, ws, nws, None)
    assert call(c, d, None, dev) == fkv.EINVAL                     # no new keys
    assert call(c, d, dev, None) == fkv.EINVAL                     # no new values
    assert call(c, d, ctypes.c_void_p(0x300002), dev) == fkv.EINVAL  # misaligned
    d.layout = 3                                                   # only the 32-row kernel fuses the insert
    assert call(c, d, dev, dev) == fkv.EUNSUPPORTED
    d.layout = 5
    d.split_tiles = 1
    assert call(c, d, dev, dev, ws=None, nws=0) == fkv.EWORKSPACE
    c16 = _fake_cache(dt="bf16")
    assert call(c16, fkv.make_decode_desc(1, 12, 18, 8, 256), dev, dev) == fkv.EUNSUPPORTED
    assert call(c, fkv.make_decode_desc(0, 12, 18, 8, 256), dev, dev) == fkv.OK  # no sequences: no launch


def test_norm_rope_insert_fails_closed_without_touching_the_gpu():
    L = fkv.lib()
    c = _fake_cache(hkv=2)
    dev = ctypes.c_void_p(0x300000)

    def call(T=4, Hq=18, eps=1e-6, rows=64, q=dev, ks=dev, cache=c):
        return L.fkv_qk_norm_rope_insert(ctypes.byref(cache), T, Hq, q, dev, dev, dev, dev, ctypes.c_float(eps), dev,
                                         rows, dev, dev, ks, dev, dev, None)
    assert call(T=-1) == fkv.EINVAL
    assert call(Hq=0) == fkv.EINVAL
    assert call(Hq=17) == fkv.EINVAL                      # not a multiple of the KV heads
    assert call(rows=0) == fkv.EINVAL
    assert call(eps=-1.0) == fkv.EINVAL
    assert call(eps=float("nan")) == fkv.EINVAL
    assert call(q=None) == fkv.EINVAL
    assert call(q=ctypes.c_void_p(0x300008)) == fkv.EINVAL  # 16-byte alignment
    assert call(ks=None) == fkv.EINVAL                     # FP8 cache needs the scales
    assert call(T=0) == fkv.OK                             # nothing to do: no launch


def test_norm_rope_insert_decode_fails_closed_without_touching_the_gpu():
    L = fkv.lib()
    c = _fake_cache()
    dev = ctypes.c_void_p(0x300000)

    def call(d, qw=dev, eps=1e-6, rows=256, cache=c):
        return L.fkv_norm_rope_insert_decode(ctypes.byref(cache), ctypes.byref(d), dev, dev, dev, qw, dev,
                                             ctypes.c_float(eps), dev, rows, dev, dev, dev, dev, dev, dev, 1 << 30,
                                             None)
    d = fkv.make_decode_desc(1, 12, 18, 8, 256)
    assert call(d, qw=None) == fkv.EINVAL
    assert call(d, qw=ctypes.c_void_p(0x300004)) == fkv.EINVAL
    assert call(d, eps=-1.0) == fkv.EINVAL
    assert call(d, rows=255) == fkv.EINVAL          # a position without a table row
    d.layout = 3
    assert call(d) == fkv.EUNSUPPORTED               # the 32-row kernel only
    assert call(fkv.make_decode_desc(1, 12, 18, 8, 256), cache=_fake_cache(dt="bf16")) == fkv.EUNSUPPORTED
    assert call(fkv.make_decode_desc(0, 12, 18, 8, 256)) == fkv.OK  # no sequences: no launch


def test_counters_record_rejections():
    fkv.reset_counters()
    c = _fake_cache()
    with pytest.raises(fkv.FkvError):
        _ws(c, q_len=0)
    cnt = fkv.get_counters()
    assert cnt["rejected_calls"] >= 1
    assert sum(cnt["insert_launches"]) == 0
