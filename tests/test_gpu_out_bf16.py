"""BF16 output (out_dtype FKV_OUT_BF16): every kernel and merge path that writes BF16 gives
bitwise the round-to-nearest-even BF16 of its own fp32 result, and stays within the oracle
gate widened by one BF16 ulp at the row's largest value (2e-3 + 2^-7, row-normalised)."""

import numpy as np
import pytest
import torch

from fp8_kv_paged_amd import fkv, synth
from fp8_kv_paged_amd.layer import PagedLayer

import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

BF16_TOL = parity.ATTN_TOL + 2.0 ** -7


def _check(lay, out, label):
    gpu = out.float().cpu().numpy()
    worst = 0.0
    for b in range(lay.num_seqs):
        M, L = lay.q_len, int(lay.seq_lens[b])
        if L < M:
            assert np.all(gpu[b, :M - L] == 0.0), (label, b)
            continue  # partly empty windows are covered with fp32 output elsewhere
        worst = max(worst, float(parity.row_errors(gpu[b], parity.reference(lay, b)).max()))
    print(f"[bf16 out] {label}: max row error {worst:.3e}", flush=True)
    assert worst <= BF16_TOL, (label, worst)


def _same_bits(o16, o32, label):
    assert o16.dtype == torch.bfloat16 and o32.dtype == torch.float32
    want = o32.to(torch.bfloat16)  # round to nearest even
    diff = (o16.view(torch.int16) != want.view(torch.int16)).sum().item()
    assert diff == 0, f"{label}: {diff} elements differ from the RNE BF16 of the fp32 output"


def _cases():
    yield "c1 q1 (automatic: row-group kernel)", synth.c1_layer, {}
    yield "c2 window 512", synth.c2_layer, {}
    yield "c3 8k p64 (in-kernel split merge)", lambda: synth.c3_layer(8192, 64), {}
    yield "c3 8k p64 layout 6", lambda: synth.c3_layer(8192, 64), {"layout": 6}
    yield "c3 8k p64 layout 3 (combine kernel)", lambda: synth.c3_layer(8192, 64), {"layout": 3}
    yield "ragged, rows before position 0", \
        lambda: synth.tiny_layer(431, [5, 12, 700, 64], num_q_heads=18, num_kv_heads=2, block_size=32, q_len=12), {}
    yield "40 sequences, grid beyond the chip (combine kernel)", \
        lambda: synth.tiny_layer(433, list(range(450, 850, 10)), num_q_heads=18, num_kv_heads=2, block_size=64,
                                 q_len=12), {"layout": 5, "split_tiles": 4}
    yield "BF16 cache", lambda: synth.tiny_layer(435, [900, 33], num_q_heads=18, num_kv_heads=2, block_size=64,
                                                 q_len=12, cache_dtype="bf16"), {}


@pytest.mark.parametrize("label,make,kw", list(_cases()), ids=[c[0] for c in _cases()])
def test_bf16_output_is_the_rounded_fp32_output(label, make, kw):
    lay = make()
    o32 = PagedLayer(lay, **kw).build().decode().clone()
    g16 = PagedLayer(lay, out_bf16=True, **kw).build()
    before = fkv.get_counters()["decode_combine_launches"]
    o16 = g16.decode().clone()
    torch.cuda.synchronize()
    if "combine kernel" in label:
        assert fkv.get_counters()["decode_combine_launches"] == before + 1, label
    _same_bits(o16, o32, label)
    _check(lay, o16, label)


def test_fused_insert_with_bf16_output():
    lay = synth.tiny_layer(437, [3000, 257, 9], num_q_heads=72, num_kv_heads=8, block_size=64, q_len=12)
    ref = PagedLayer(lay).build().decode().clone()
    gl = PagedLayer(lay, out_bf16=True)
    gl.prefill()
    gl.stage_new_tokens()
    o16 = gl.insert_decode().clone()
    torch.cuda.synchronize()
    _same_bits(o16, ref, "fused insert")
    _check(lay, o16, "fused insert")


def test_binding_checks_the_output_element_size():
    lay = synth.c1_layer()
    gl = PagedLayer(lay, out_bf16=True).build()
    wrong = torch.empty(gl.out.shape, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        fkv.decode_attn(gl.cache, gl.ddesc, gl.q, gl.block_table, gl.seq_lens, gl.k_scale, gl.v_scale, wrong,
                        gl.workspace)
