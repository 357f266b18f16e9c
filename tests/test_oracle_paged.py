"""Pins of the oracle's cache sizes, byte layout, insertion and gather.

- the pages' printed payload arithmetic and the exactly-2x capacity figure
  (tests/golden/payload.json);
- hand-worked byte offsets of the documented pool layout;
- invariants: gather(insert(x)) equals the quantised tokens in logical order
  for any page-table permutation; negative slots are skipped; untouched slots
  keep their previous bytes.
"""

import json
import os

import numpy as np
import pytest

from oracle import e4m3, paged
from fp8_kv_paged_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "payload.json")))


def test_payload_figures_from_pages():
    H, D = GOLD["num_kv_heads"], GOLD["head_dim"]
    assert 2 * H * D == GOLD["values_per_token_layer"]
    for dt, key in ((paged.BF16, "bf16"), (paged.FP8, "fp8_e4m3fn")):
        per = paged.payload_bytes_per_token(H, dt)
        assert per == GOLD["bytes_per_token_layer"][key]
        assert per * GOLD["target_layers"] == GOLD["kib_per_token_target"][key] * 1024
        total = per * (GOLD["target_layers"] + GOLD["draft_layers"])
        assert total == GOLD["kib_per_token_with_draft"][key] * 1024
        # clean KV-head sharding over 4 ranks: 2 KV heads per rank
        per_rank = paged.payload_bytes_per_token(H // GOLD["tp_ranks"], dt) * (GOLD["target_layers"] + GOLD["draft_layers"])
        assert per_rank == GOLD["kib_per_token_per_rank_with_draft"][key] * 1024


def test_same_budget_holds_exactly_twice_the_tokens():
    bf, fp = GOLD["cache_tokens_per_card"]["bf16"], GOLD["cache_tokens_per_card"]["fp8_e4m3fn"]
    assert fp == 2 * bf
    budget = bf * paged.payload_bytes_per_token(8, paged.BF16)
    assert budget // paged.payload_bytes_per_token(8, paged.FP8) == fp
    for bs in (32, 64):
        nb_bf = budget // (paged.pool_bytes(1, bs, 8, paged.BF16) * 2)
        nb_fp = budget // (paged.pool_bytes(1, bs, 8, paged.FP8) * 2)
        assert nb_fp in (2 * nb_bf, 2 * nb_bf + 1)


def test_layout_hand_worked_offsets():
    # K: ((blk*Hkv + h)*bs + o)*128 + d
    #   blk 3, h 1, o 5, d 7, bs 32, Hkv 2: ((3*2+1)*32+5)*128+7 = (224+5)*128+7 = 29319
    assert paged.k_index(3, 1, 5, 7, 32, 2) == 29319
    #   blk 0, h 0, o 63, d 127, bs 64, Hkv 8: 63*128+127 = 8191 (last byte of the first slab)
    assert paged.k_index(0, 0, 63, 127, 64, 8) == 8191
    # V: (blk*Hkv + h)*bs*128 + (o//8)*1024 + d*8 + o%8
    #   blk 3, h 1, o 13, d 2, bs 32, Hkv 2: 7*4096 + 1*1024 + 16 + 5 = 28672+1045 = 29717
    assert paged.v_index(3, 1, 13, 2, 32, 2) == 29717
    #   blk 1, h 0, o 0, d 1, bs 64, Hkv 2: 2*8192 + 0 + 8 + 0 = 16392
    assert paged.v_index(1, 0, 0, 1, 64, 2) == 16392
    # each slab is a permutation of its own bs*128 elements
    for bs in (32, 64):
        o, d = np.meshgrid(np.arange(bs), np.arange(128), indexing="ij")
        for fn in (paged.k_index, paged.v_index):
            idx = fn(2, 1, o, d, bs, 3)
            base = (2 * 3 + 1) * bs * 128
            assert np.array_equal(np.sort(idx.ravel()), base + np.arange(bs * 128))


@pytest.mark.parametrize("cache_dtype", [paged.FP8, paged.BF16])
@pytest.mark.parametrize("bs", [32, 64])
def test_gather_of_insert_is_logical_quantised_tokens(cache_dtype, bs):
    lay = synth.tiny_layer(31 + bs, [bs * 3 + 7, 5, bs], num_q_heads=6, num_kv_heads=2, block_size=bs,
                           cache_dtype=cache_dtype, pool_slack=2.0)
    kp, vp = paged.new_pools(lay.num_blocks, bs, 2, cache_dtype, fill=0x7F)
    for b in range(lay.num_seqs):
        L = int(lay.seq_lens[b])
        k, v = lay.kv_bits(b, 0, L)
        paged.insert(kp, vp, k, v, lay.slots(b, 0, L), lay.k_scale, lay.v_scale, bs, 2, cache_dtype)
    for b in range(lay.num_seqs):
        L = int(lay.seq_lens[b])
        k, v = lay.kv_bits(b, 0, L)
        gk = paged.gather(kp, "k", lay.block_table[b], L, bs, 2)
        gv = paged.gather(vp, "v", lay.block_table[b], L, bs, 2)
        if cache_dtype == paged.FP8:
            assert np.array_equal(gk, e4m3.quantize(k, lay.k_scale))
            assert np.array_equal(gv, e4m3.quantize(v, lay.v_scale))
        else:
            assert np.array_equal(gk, k) and np.array_equal(gv, v)


def test_negative_slots_skipped_and_untouched_bytes_kept():
    bs, H = 32, 2
    kp, vp = paged.new_pools(4, bs, H, paged.FP8, fill=0x7F)
    r = np.random.default_rng(3)
    k = synth.f32_to_bf16_bits(r.standard_normal((5, H, 128), dtype=np.float32))
    v = synth.f32_to_bf16_bits(r.standard_normal((5, H, 128), dtype=np.float32))
    slots = np.array([3, -1, 40, -7, 127], np.int32)
    paged.insert(kp, vp, k, v, slots, np.float32(0.05), np.float32(0.07), bs, H, paged.FP8)
    written = np.zeros(kp.shape, bool)
    writtenv = np.zeros(vp.shape, bool)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, o = s // bs, s % bs
        for h in range(H):
            d = np.arange(128)
            ik = paged.k_index(blk, h, o, d, bs, H)
            iv = paged.v_index(blk, h, o, d, bs, H)
            assert np.array_equal(kp[ik], e4m3.quantize(k[t, h], np.float32(0.05)))
            assert np.array_equal(vp[iv], e4m3.quantize(v[t, h], np.float32(0.07)))
            written[ik] = True
            writtenv[iv] = True
    assert np.all(kp[~written] == 0x7F) and np.all(vp[~writtenv] == 0x7F)


def test_gather_permutation_invariance():
    """Two different page tables holding the same logical tokens gather identically."""
    bs, H, L = 32, 2, 150
    r = np.random.default_rng(5)
    k = synth.f32_to_bf16_bits(r.standard_normal((L, H, 128), dtype=np.float32))
    v = synth.f32_to_bf16_bits(r.standard_normal((L, H, 128), dtype=np.float32))
    nb = (L + bs - 1) // bs
    outs = []
    for perm_seed in (0, 1, 2):
        table = np.random.default_rng(perm_seed).permutation(12)[:nb].astype(np.int32)
        kp, vp = paged.new_pools(12, bs, H, paged.FP8)
        j = np.arange(L)
        slots = (table[j // bs] * bs + j % bs).astype(np.int32)
        paged.insert(kp, vp, k, v, slots, np.float32(0.03), np.float32(0.09), bs, H, paged.FP8)
        outs.append((paged.gather(kp, "k", table, L, bs, H), paged.gather(vp, "v", table, L, bs, H)))
    for a in outs[1:]:
        assert np.array_equal(a[0], outs[0][0]) and np.array_equal(a[1], outs[0][1])
