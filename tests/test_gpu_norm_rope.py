"""GPU parity of fkv_qk_norm_rope_insert against the oracle (the plain float64 RMSNorm and
rotate-half RoPE, each rounded once to BF16): the normalised, rotated Q bits and the K' pool
codes bit for bit wherever the float64 value is not within the float32 error band of a
rounding boundary, and one of the two neighbouring roundings where it is (tests/parity.py,
norm_rope_bounds); every other pool byte, and V, bit for bit. On the workloads' shapes, ragged
and padded batches, both page sizes, both cache types and in place; then decode attention
over the result within the 2e-3 gate, and the in-launch form bitwise equal to the two-launch
form."""

import dataclasses

import numpy as np
import pytest
import torch

from fp8_kv_paged_amd import fkv, synth
from fp8_kv_paged_amd.layer import PagedLayer, to_dev_bits
from oracle import attention, normrope, paged

import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def _oracle_prefilled(lay):
    """Oracle pools holding every token before the q_len new ones (poisoned elsewhere)."""
    kp, vp = paged.new_pools(lay.num_blocks, lay.block_size, lay.num_kv_heads, lay.cache_dtype,
                             fill=parity.POISON[lay.cache_dtype])
    for b in range(lay.num_seqs):
        L = int(lay.seq_lens[b])
        n = max(0, L - lay.q_len)
        if n:
            k, v = lay.kv_bits(b, 0, n)
            paged.insert(kp, vp, k, v, lay.slots(b, 0, n), lay.k_scale, lay.v_scale, lay.block_size,
                         lay.num_kv_heads, lay.cache_dtype)
    return kp, vp


def _run(lay, st, inplace=False):
    gl = PagedLayer(lay)
    gl.prefill()
    dev = gl.device
    q = to_dev_bits(st.q_bits, dev)
    k, v = to_dev_bits(st.k_bits, dev), to_dev_bits(st.v_bits, dev)
    qw, kw = to_dev_bits(st.q_w, dev), to_dev_bits(st.k_w, dev)
    cs = torch.from_numpy(st.cos_sin).to(dev)
    pos = torch.from_numpy(st.positions).to(dev)
    slots = torch.from_numpy(st.slot_mapping).to(dev)
    q_out = q if inplace else torch.full_like(q, float("nan"))
    before = fkv.get_counters()["norm_rope_insert_launches"]
    fkv.qk_norm_rope_insert(gl.cache, q, k, v, qw, kw, st.eps, cs, pos, slots, gl.k_scale, gl.v_scale, q_out)
    torch.cuda.synchronize()
    after = fkv.get_counters()["norm_rope_insert_launches"]
    which = 0 if lay.cache_dtype == "fp8_e4m3fn" else 1
    assert after[which] == before[which] + 1

    kp, vp = _oracle_prefilled(lay)
    st = dataclasses.replace(st, slot_mapping=np.where(st.slot_mapping < lay.num_blocks * lay.block_size,
                                                      st.slot_mapping, -1).astype(np.int32))  # past the pool: skipped
    q_ref = normrope.norm_rope_insert(kp, vp, st.q_bits, st.k_bits, st.v_bits, st.q_w, st.k_w, st.eps, st.cos_sin,
                                      st.positions, st.slot_mapping, lay.k_scale, lay.v_scale, lay.block_size,
                                      lay.num_kv_heads, lay.cache_dtype)
    got_q = q_out.view(torch.int16).cpu().numpy().view(np.uint16)
    q_lo, q_hi, _ = parity.norm_rope_bounds(st.q_bits, st.q_w, st.eps, st.cos_sin, st.positions)
    nq_two, nq_diff = parity.check_bf16_within(got_q, q_lo, q_hi, f"{lay.name} Q'")
    dt = np.uint8 if lay.cache_dtype == "fp8_e4m3fn" else np.uint16
    gk = gl.k_pool.cpu().numpy().view(dt)
    gv = gl.v_pool.cpu().numpy().view(dt)
    assert np.array_equal(gv, vp), f"{lay.name}: {(gv != vp).sum()} V pool elements differ"
    k_lo, k_hi, _ = parity.norm_rope_bounds(st.k_bits, st.k_w, st.eps, st.cos_sin, st.positions)
    nk_two, nk_diff = parity.check_norm_rope_k_pool(gk, kp, lay, st, k_lo, k_hi, lay.name)
    print(f"[norm_rope_insert parity] {lay.name}: {st.positions.shape[0]} tokens; Q' {got_q.size} elements, "
          f"{nq_two} near a rounding boundary, {nq_diff} differ from the oracle; K' {nk_two} near, {nk_diff} differ; "
          f"V and every other pool byte bit-exact", flush=True)
    return gl, q_out, kp, vp, q_ref


def _cases():
    yield "c1 q1 page 32", synth.c1_layer
    yield "c2 window 512 page 64", synth.c2_layer
    yield "c3 8k page 64", lambda: synth.c3_layer(8192, 64)
    yield "c3 8k page 32", lambda: synth.c3_layer(8192, 32)
    yield "ragged, rows before position 0, page 32", \
        lambda: synth.tiny_layer(511, [40, 5, 700, 12, 1], num_q_heads=18, num_kv_heads=2, block_size=32, q_len=12)
    yield "q1 batch of 40", lambda: synth.tiny_layer(513, list(range(1, 1000, 25)), num_q_heads=72, num_kv_heads=8,
                                                      block_size=64, q_len=1)
    yield "BF16 cache", lambda: synth.tiny_layer(515, [900, 33], num_q_heads=18, num_kv_heads=2, block_size=64,
                                                 q_len=12, cache_dtype="bf16")


@pytest.mark.parametrize("label,make", list(_cases()), ids=[c[0] for c in _cases()])
def test_against_the_oracle(label, make):
    lay = make()
    _run(lay, synth.norm_rope_step(lay))


def test_padding_tokens_and_in_place():
    lay = synth.tiny_layer(517, [300, 90], num_q_heads=18, num_kv_heads=2, block_size=64, q_len=12)
    st = synth.norm_rope_step(lay)
    st.positions = st.positions.copy()
    st.slot_mapping = st.slot_mapping.copy()
    st.positions[2] = st.cos_sin.shape[0]      # outside the table: zero Q row, no insert
    st.positions[14] = -3
    st.slot_mapping[7] = -1                     # skip the insert only
    st.slot_mapping[20] = lay.num_blocks * lay.block_size  # past the pool: skipped
    _, q_out, _, _, _ = _run(lay, st, inplace=True)
    got = q_out.view(torch.int16).cpu().numpy()
    assert np.all(got[2] == 0) and np.all(got[14] == 0)


@pytest.mark.parametrize("label,make", [("c3 8k page 64", lambda: synth.c3_layer(8192, 64)),
                                        ("c2 window 512", synth.c2_layer),
                                        ("BF16 cache", lambda: synth.tiny_layer(519, [700, 64], num_q_heads=18,
                                                                               num_kv_heads=2, block_size=32,
                                                                               q_len=12, cache_dtype="bf16"))],
                         ids=["c3_8k_p64", "c2", "bf16"])
def test_decode_attention_after_the_step(label, make):
    """The step feeds decode: attention with Q' over the cache the step updated, against the
    oracle's attention with its own Q' and pools."""
    lay = make()
    gl, q_out, kp, vp, q_ref = _run(lay, synth.norm_rope_step(lay))
    gl.q = q_out.view(lay.num_seqs, lay.q_len, lay.num_q_heads, 128)
    out = gl.decode().clone()
    torch.cuda.synchronize()
    ref = attention.paged_decode(kp, vp, q_ref.reshape(lay.num_seqs, lay.q_len, lay.num_q_heads, 128),
                                 lay.block_table, lay.seq_lens, lay.q_len, lay.window_left, lay.softmax_scale,
                                 lay.k_scale, lay.v_scale, lay.block_size, lay.num_kv_heads, lay.cache_dtype)
    worst = float(parity.row_errors(out.cpu().numpy(), ref).max())
    print(f"[norm_rope_insert + decode] {label}: max row error {worst:.3e}", flush=True)
    assert worst <= parity.ATTN_TOL, (label, worst)


def _fused_cases():
    yield "c3 8k page 64", lambda: synth.c3_layer(8192, 64), {}
    yield "c2 window 512", synth.c2_layer, {}
    yield "ragged, rows before position 0", \
        lambda: synth.tiny_layer(521, [40, 5, 700, 12], num_q_heads=18, num_kv_heads=2, block_size=32, q_len=12), {}
    yield "q1 batch of 24, 72/8", lambda: synth.tiny_layer(523, list(range(1, 1200, 50)), num_q_heads=72,
                                                            num_kv_heads=8, block_size=64, q_len=1), {}
    yield "c3 8k page 64, layout 6", lambda: synth.c3_layer(8192, 64), {"layout": 6}
    yield "q_len 16, 14/2", lambda: synth.tiny_layer(525, [16, 9, 500], num_q_heads=14, num_kv_heads=2,
                                                      block_size=32, q_len=16), {}


@pytest.mark.parametrize("label,make,kw", list(_fused_cases()), ids=[c[0] for c in _fused_cases()])
def test_norm_rope_inside_the_attention_launch(label, make, kw):
    """fkv_norm_rope_insert_decode equals fkv_qk_norm_rope_insert followed by fkv_decode_attn with
    the rotated Q (same layout; layout 5 for the automatic one) bit for bit: pools and output."""
    lay = make()
    st = synth.norm_rope_step(lay)
    dev = "cuda"
    q, k, v = (to_dev_bits(x, dev) for x in (st.q_bits, st.k_bits, st.v_bits))
    qw, kw_ = to_dev_bits(st.q_w, dev), to_dev_bits(st.k_w, dev)
    cs = torch.from_numpy(st.cos_sin).to(dev)

    fused = PagedLayer(lay, **kw)
    fused.prefill()
    before = fkv.get_counters()
    fkv.norm_rope_insert_decode(fused.cache, fused.ddesc, q, k, v, qw, kw_, st.eps, cs, fused.block_table,
                                fused.seq_lens, fused.k_scale, fused.v_scale, fused.out, fused.workspace)
    out_f = fused.out.clone()

    sep = PagedLayer(lay, layout=kw.get("layout", 5))
    sep.prefill()
    q_rot = torch.empty_like(q)
    fkv.qk_norm_rope_insert(sep.cache, q, k, v, qw, kw_, st.eps, cs, torch.from_numpy(st.positions).to(dev),
                            torch.from_numpy(st.slot_mapping).to(dev), sep.k_scale, sep.v_scale, q_rot)
    sep.q = q_rot.view(lay.num_seqs, lay.q_len, lay.num_q_heads, 128)
    out_s = sep.decode().clone()
    torch.cuda.synchronize()
    after = fkv.get_counters()
    assert after["norm_rope_insert_decode_launches"] == before["norm_rope_insert_decode_launches"] + 1
    assert torch.equal(fused.k_pool, sep.k_pool), f"{label}: K pool differs"
    assert torch.equal(fused.v_pool, sep.v_pool), f"{label}: V pool differs"
    assert torch.equal(out_f, out_s), f"{label}: output differs from the two-launch path"
    print(f"[norm_rope_insert_decode] {label}: bitwise equal to norm_rope_insert + decode", flush=True)


def test_norm_rope_inside_the_attention_launch_against_the_oracle():
    lay = synth.c2_layer()
    st = synth.norm_rope_step(lay)
    dev = "cuda"
    gl = PagedLayer(lay)
    gl.prefill()
    fkv.norm_rope_insert_decode(gl.cache, gl.ddesc, *(to_dev_bits(x, dev) for x in (st.q_bits, st.k_bits, st.v_bits)),
                                to_dev_bits(st.q_w, dev), to_dev_bits(st.k_w, dev), st.eps,
                                torch.from_numpy(st.cos_sin).to(dev), gl.block_table, gl.seq_lens, gl.k_scale,
                                gl.v_scale, gl.out, gl.workspace)
    out = gl.out.clone()
    torch.cuda.synchronize()
    kp, vp = _oracle_prefilled(lay)
    q_ref = normrope.norm_rope_insert(kp, vp, st.q_bits, st.k_bits, st.v_bits, st.q_w, st.k_w, st.eps, st.cos_sin,
                                      st.positions, st.slot_mapping, lay.k_scale, lay.v_scale, lay.block_size,
                                      lay.num_kv_heads)
    assert np.array_equal(gl.v_pool.cpu().numpy(), vp)
    k_lo, k_hi, _ = parity.norm_rope_bounds(st.k_bits, st.k_w, st.eps, st.cos_sin, st.positions)
    parity.check_norm_rope_k_pool(gl.k_pool.cpu().numpy(), kp, lay, st, k_lo, k_hi, "c2 in-launch")
    ref = attention.paged_decode(kp, vp, q_ref.reshape(lay.num_seqs, lay.q_len, lay.num_q_heads, 128),
                                 lay.block_table, lay.seq_lens, lay.q_len, lay.window_left, lay.softmax_scale,
                                 lay.k_scale, lay.v_scale, lay.block_size, lay.num_kv_heads, lay.cache_dtype)
    worst = float(parity.row_errors(out.cpu().numpy(), ref).max())
    print(f"[norm_rope_insert_decode] c2 against the oracle: max row error {worst:.3e}", flush=True)
    assert worst <= parity.ATTN_TOL
