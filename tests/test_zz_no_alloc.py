"""fkv_decode_attn_noalloc (the library's static scratch instead of a caller workspace) against
fkv_decode_attn with a workspace, through the C ABI: bitwise equal outputs on consecutive calls
whose inputs shrink (the 72/8-head layer at 8k, then an 18/2-head layer whose two pairs merge
their splits inside the kernel on fewer partials, then a q1 batch through the row-group kernel
and the combine kernel), the first input again, a call captured in a HIP graph, and a plan
beyond the scratch rejected with FKV_EWORKSPACE."""

import numpy as np
import pytest
import torch

from fp8_kv_paged_amd import fkv, synth
from fp8_kv_paged_amd.layer import PagedLayer

import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def _both(gl, label):
    ref = gl.decode().clone()
    out = torch.full_like(gl.out, float("nan"))
    fkv.decode_attn_noalloc(gl.cache, gl.ddesc, gl.q, gl.block_table, gl.seq_lens, gl.k_scale, gl.v_scale, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), f"{label}: noalloc output differs from fkv_decode_attn"
    print(f"[noalloc] {label}: bitwise equal to fkv_decode_attn (workspace {gl.workspace.numel()} B)", flush=True)
    return out


def test_noalloc_matches_the_workspace_call_on_shrinking_inputs():
    big = PagedLayer(synth.c3_layer(8192, 64)).build()
    small = PagedLayer(synth.c4_layer(3)).build()
    q1 = PagedLayer(synth.tiny_layer(701, [300, 1500, 64], num_q_heads=72, num_kv_heads=8, block_size=32,
                                     q_len=1)).build()
    assert big.workspace.numel() > small.workspace.numel() > 16
    o_big = _both(big, "72/8 8k M12 (8 pairs)")
    _both(small, "18/2 8k M12 global (2 pairs, in-kernel merge)")
    _both(q1, "q1 batch of 3, 72/8 (row-group kernel + combine)")
    o_again = _both(big, "72/8 8k M12 again")
    assert torch.equal(o_big, o_again)
    worst = float(parity.row_errors(o_again.cpu().numpy()[0], parity.reference(big.lay, 0, [0, 7])).max())
    assert worst <= parity.ATTN_TOL, worst


def test_noalloc_inside_a_captured_graph():
    gl = PagedLayer(synth.c4_layer(0)).build()
    ref = gl.decode().clone()
    out = torch.zeros_like(gl.out)
    s = torch.cuda.Stream()
    fkv.decode_attn_noalloc(gl.cache, gl.ddesc, gl.q, gl.block_table, gl.seq_lens, gl.k_scale, gl.v_scale, out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fkv.decode_attn_noalloc(gl.cache, gl.ddesc, gl.q, gl.block_table, gl.seq_lens, gl.k_scale, gl.v_scale, out)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        gl.decode()  # eager work on the same data between replays
        torch.cuda.synchronize()


def test_noalloc_rejects_plans_beyond_its_scratch():
    lay = synth.c5_layer(12)
    gl = PagedLayer(lay)  # no prefill needed: the call fails before any launch
    need = fkv.decode_workspace_bytes(gl.cache, gl.ddesc)
    assert need > (32 << 20)
    before = fkv.get_counters()["rejected_calls"]
    with pytest.raises(fkv.FkvError) as e:
        fkv.decode_attn_noalloc(gl.cache, gl.ddesc, gl.q, gl.block_table, gl.seq_lens, gl.k_scale, gl.v_scale, gl.out)
    assert e.value.status == fkv.EWORKSPACE
    assert fkv.get_counters()["rejected_calls"] == before + 1
