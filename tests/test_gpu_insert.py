"""GPU parity of cache insertion: the pools written by the HIP kernel equal the
oracle's bytes exactly (FP8 E4M3FN and BF16 caches), including every BF16 bit
pattern under many scales, skipped slots and untouched (poisoned) bytes."""

import numpy as np
import pytest
import torch

from fp8_kv_paged_amd import fkv, synth
from fp8_kv_paged_amd.layer import PagedLayer, to_dev_bits
from oracle import e4m3, paged

import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def _pool_bytes(t, cache_dtype):
    a = t.cpu().numpy()
    return a if cache_dtype == paged.FP8 else a.view(np.uint16)


def _scales():
    r = np.random.default_rng(77)
    s = list(r.uniform(0.01, 0.1, size=24).astype(np.float32))
    # the ends of the reciprocal-correction range, an all-ones significand, and scales outside
    # that range (IEEE division): tiny, huge, negative
    edge = (2.0 ** -32, 2.0 ** 32, np.nextafter(np.float32(2.0), np.float32(0.0)), 1e-12, 1e12, -0.05)
    return s + [np.float32(x) for x in (1.0, 0.5, 2.0 ** -6, 0.0625, 3.0, 1e-3) + edge]


def test_every_bf16_pattern_under_many_scales():
    """All 65,536 BF16 patterns (512 tokens x 128, one KV head) through the FP8 insert."""
    bs, H, T = 32, 1, 512
    nb = T // bs
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    k_bits = pats.reshape(T, H, 128)
    v_bits = pats[::-1].copy().reshape(T, H, 128)
    slots = np.random.default_rng(5).permutation(T).astype(np.int32)
    nan_k = np.isnan(e4m3.bf16_bits_to_f32(k_bits))
    nan_v = np.isnan(e4m3.bf16_bits_to_f32(v_bits))
    desc = fkv.make_cache_desc(nb, bs, H, "fp8_e4m3fn")
    nbytes = fkv.cache_bytes(desc)[0]
    kd, vd, sd = to_dev_bits(k_bits, "cuda"), to_dev_bits(v_bits, "cuda"), torch.from_numpy(slots).cuda()
    for s in _scales():
        kp = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device="cuda")
        vp = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device="cuda")
        cache = fkv.init_cache(desc, kp, vp)
        ks = torch.tensor([float(s)], dtype=torch.float32, device="cuda")
        fkv.insert(cache, kd, vd, sd, ks, ks)
        okp, ovp = paged.new_pools(nb, bs, H, paged.FP8, fill=0x7F)
        paged.insert(okp, ovp, k_bits, v_bits, slots, s, s, bs, H, paged.FP8)
        gk, gv = kp.cpu().numpy(), vp.cpu().numpy()
        # NaN inputs: only NaN-ness is defined (0x7F or 0xFF)
        for g, o, nanmask, which in ((gk, okp, nan_k, "k"), (gv, ovp, nan_v, "v")):
            idx_nan = np.zeros(g.shape, bool)
            j = np.arange(T)
            blk, off = (slots[j] // bs)[:, None], (slots[j] % bs)[:, None]
            d = np.arange(128)[None, :]
            fn = paged.k_index if which == "k" else paged.v_index
            pos = fn(blk, 0, off, d, bs, H)
            idx_nan[pos[nanmask[:, 0, :]]] = True
            assert np.all((g[idx_nan] & 0x7F) == 0x7F)
            bad = np.nonzero((g != o) & ~idx_nan)[0]
            assert len(bad) == 0, (float(s), which, bad[:8], g[bad[:8]], o[bad[:8]])


@pytest.mark.parametrize("cache_dtype", ["fp8_e4m3fn", "bf16"])
def test_skipped_and_out_of_range_slots(cache_dtype):
    bs, H = 64, 2
    lay = synth.tiny_layer(41, [200], num_q_heads=2, num_kv_heads=H, block_size=bs, cache_dtype=cache_dtype)
    gl = PagedLayer(lay)
    k, v = lay.kv_bits(0, 0, 6)
    nslots = lay.num_blocks * bs
    slots = np.array([5, -1, nslots, 77, -100, nslots + 5], np.int32)
    fkv.insert(gl.cache, to_dev_bits(k, "cuda"), to_dev_bits(v, "cuda"), torch.from_numpy(slots).cuda(),
               gl.k_scale, gl.v_scale)
    okp, ovp = paged.new_pools(lay.num_blocks, bs, H, cache_dtype, fill=parity.POISON[cache_dtype])
    keep = slots.copy()
    keep[keep >= nslots] = -1
    paged.insert(okp, ovp, k, v, keep, lay.k_scale, lay.v_scale, bs, H, cache_dtype)
    assert np.array_equal(_pool_bytes(gl.k_pool, cache_dtype), okp)
    assert np.array_equal(_pool_bytes(gl.v_pool, cache_dtype), ovp)


def _layers():
    yield "c1", synth.c1_layer()
    yield "c2", synth.c2_layer()
    yield "c3_8k_p32", synth.c3_layer(8192, 32)
    yield "c3_8k_p64", synth.c3_layer(8192, 64)
    yield "c3_32k_p64", synth.c3_layer(32768, 64)
    yield "c4_sw", synth.c4_layer(0)
    yield "c4_global", synth.c4_layer(3)
    yield "c4_draft", synth.c4_layer(50)
    yield "c2_bf16", synth.make_layer("c2_bf16", 1002, 0, 18, 2, 64, 12, 511, [2048], outlier_rate=0.01,
                                      cache_dtype="bf16")


@pytest.mark.parametrize("name,lay", list(_layers()), ids=[n for n, _ in _layers()])
def test_pools_bit_exact(name, lay):
    print(f"[insert parity] {name}", flush=True)
    gl = PagedLayer(lay).build()
    torch.cuda.synchronize()
    okp, ovp = parity.oracle_pools(lay)
    gk, gv = _pool_bytes(gl.k_pool, lay.cache_dtype), _pool_bytes(gl.v_pool, lay.cache_dtype)
    assert np.array_equal(gk, okp), np.nonzero(gk != okp)[0][:10]
    assert np.array_equal(gv, ovp), np.nonzero(gv != ovp)[0][:10]
    cnt = fkv.get_counters()
    assert cnt["insert_launches"][0 if lay.cache_dtype == "fp8_e4m3fn" else 1] > 0


def test_c5_sampled_sequences_bit_exact():
    """Shared interleaved pool of 32 sequences: every block of three sampled sequences."""
    lay = synth.c5_layer(12)
    gl = PagedLayer(lay).build()
    torch.cuda.synchronize()
    gk, gv = gl.k_pool.cpu().numpy(), gl.v_pool.cpu().numpy()
    order = np.argsort(lay.seq_lens)
    for b in (int(order[0]), int(order[len(order) // 2]), int(order[-1])):
        L = int(lay.seq_lens[b])
        print(f"[insert parity] c5 sequence {b} L={L}", flush=True)
        k, v = lay.kv_bits(b, 0, L)
        assert np.array_equal(paged.gather(gk, "k", lay.block_table[b], L, 32, 8), e4m3.quantize(k, lay.k_scale))
        assert np.array_equal(paged.gather(gv, "v", lay.block_table[b], L, 32, 8), e4m3.quantize(v, lay.v_scale))
