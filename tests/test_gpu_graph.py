"""Graph capture of a multi-layer decode cycle: every entry point is capturable (device
scalars, caller-owned workspaces, no allocation, no host synchronisation), each replay
reproduces the eager outputs bit for bit, the inserted cache bytes stay those of the eager
insert, and the launch counters count the captured launches once (at capture) and nothing
per replay."""

import dataclasses

import numpy as np
import pytest
import torch

from fp8_kv_paged_amd import fkv, synth
from fp8_kv_paged_amd.layer import PagedLayer

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def _cycle_layers():
    """Sliding-window, global and draft layers of the 48 (+6) layer cycle (context 8192)."""
    ids = [0, 1, 3, 7, 48, 53]
    layers = []
    for i in ids:
        gl = PagedLayer(synth.c4_layer(i))
        gl.prefill()
        gl.stage_new_tokens()
        layers.append(gl)
    return layers


def test_cycle_graph_replays_match_eager():
    layers = _cycle_layers()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for gl in layers:
            gl.insert_decode(stream)
    stream.synchronize()
    ref_out = [gl.out.clone() for gl in layers]
    ref_k = [gl.k_pool.clone() for gl in layers]
    ref_v = [gl.v_pool.clone() for gl in layers]
    before = fkv.get_counters()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for gl in layers:
            gl.insert_decode()
    torch.cuda.synchronize()
    mid = fkv.get_counters()
    assert mid["insert_decode_launches"] == before["insert_decode_launches"] + len(layers)
    for rep in range(3):
        for gl in layers:
            gl.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, gl in enumerate(layers):
            assert torch.equal(gl.out, ref_out[j]), (rep, j)
            assert torch.equal(gl.k_pool, ref_k[j]) and torch.equal(gl.v_pool, ref_v[j]), (rep, j)
        # eager work between replays (another layer's decode on the side stream)
        with torch.cuda.stream(stream):
            layers[0].decode(stream)
        stream.synchronize()
    after = fkv.get_counters()
    assert after["insert_decode_launches"] == mid["insert_decode_launches"]  # replays bypass the host
    print(f"[graph] {len(layers)}-layer cycle: 3 replays equal to eager", flush=True)


def test_decode_graph_with_split_merge_counters():
    """A captured decode whose splits merge inside the kernel: the workspace counters return
    to zero at the end of every replay, so replays stay equal to the eager call."""
    lay = synth.c3_layer(8192, 64)
    gl = PagedLayer(lay).build()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        gl.decode(stream)
    stream.synchronize()
    ref = gl.out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        gl.decode()
    torch.cuda.synchronize()
    nws = fkv.decode_workspace_bytes(gl.cache, gl.ddesc)
    ctl = lay.num_seqs * lay.num_kv_heads * 256
    for rep in range(4):
        gl.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(gl.out, ref), rep
        assert torch.count_nonzero(gl.workspace[nws - ctl:nws]).item() == 0, rep


def test_fused_steps_replayed_with_metadata_refreshed_in_place():
    """Three decode steps of one layer from a single captured fkv_insert_decode: before each replay
    the sequence lengths and the new tokens are rewritten in place in the captured buffers (the
    block table already holds the final capacity, the descriptor's max_seq_len the final length).
    Every replay equals the eager fused call of the same step bit for bit (pools and output) and
    the oracle, and launches nothing from the host."""
    final = synth.tiny_layer(661, [524, 114, 3000], num_q_heads=18, num_kv_heads=2, block_size=32, q_len=12,
                             pool_slack=2.0)
    graphed, eager = PagedLayer(final), PagedLayer(final)
    for gl in (graphed, eager):
        for b in range(final.num_seqs):
            gl.insert_tokens(b, 0, int(final.seq_lens[b]) - 36)

    def at_step(step):
        return dataclasses.replace(final, seq_lens=(final.seq_lens - 12 * (2 - step)).astype(np.int32))

    def refresh(gl, lay):
        gl.lay = lay
        gl.seq_lens.copy_(torch.from_numpy(lay.seq_lens))
        k, v = gl.new_k, gl.new_v
        gl.stage_new_tokens()
        if k is not None:  # keep the captured buffers, rewrite their contents
            k.copy_(gl.new_k)
            v.copy_(gl.new_v)
            gl.new_k, gl.new_v = k, v

    import parity

    refresh(graphed, at_step(0))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        graphed.insert_decode()
    torch.cuda.synchronize()
    for step in range(3):
        lay = at_step(step)
        refresh(graphed, lay)
        torch.cuda.synchronize()
        before = fkv.get_counters()["insert_decode_launches"]
        g.replay()
        torch.cuda.synchronize()
        assert fkv.get_counters()["insert_decode_launches"] == before, step  # no host launch
        refresh(eager, lay)
        out_e = eager.insert_decode().clone()
        torch.cuda.synchronize()
        assert torch.equal(graphed.k_pool, eager.k_pool) and torch.equal(graphed.v_pool, eager.v_pool), step
        assert torch.equal(graphed.out, out_e), step
        gpu = graphed.out.cpu().numpy()
        worst = max(float(parity.row_errors(gpu[b], parity.reference(lay, b)).max()) for b in range(lay.num_seqs))
        print(f"[graph] fused step {step} replayed with refreshed metadata: max row error {worst:.3e}", flush=True)
        assert worst <= parity.ATTN_TOL, (step, worst)


def test_norm_rope_paths_in_a_graph():
    """The Q/K norm + RoPE entry points captured in one graph per layer: the standalone step
    followed by decode on one layer, the step inside the attention launch on another. Each
    replay (with eager work and synchronisations in between) reproduces the eager outputs,
    rotated Q and pool bytes bit for bit."""
    from fp8_kv_paged_amd.layer import to_dev_bits
    lay = synth.c4_layer(3)
    st = synth.norm_rope_step(lay)
    d = "cuda"
    q, k, v = (to_dev_bits(x, d) for x in (st.q_bits, st.k_bits, st.v_bits))
    qw, kw = to_dev_bits(st.q_w, d), to_dev_bits(st.k_w, d)
    cs = torch.from_numpy(st.cos_sin).to(d)
    pos, sl = torch.from_numpy(st.positions).to(d), torch.from_numpy(st.slot_mapping).to(d)
    two, one = PagedLayer(lay, layout=5), PagedLayer(lay)
    for gl in (two, one):
        gl.prefill()
    q_rot = torch.empty_like(q)
    two.q = q_rot.view(lay.num_seqs, lay.q_len, lay.num_q_heads, 128)
    stream = torch.cuda.Stream()

    def step(s):
        fkv.qk_norm_rope_insert(two.cache, q, k, v, qw, kw, st.eps, cs, pos, sl, two.k_scale, two.v_scale, q_rot, s)
        two.decode(s)
        fkv.norm_rope_insert_decode(one.cache, one.ddesc, q, k, v, qw, kw, st.eps, cs, one.block_table, one.seq_lens,
                                    one.k_scale, one.v_scale, one.out, one.workspace, s)
    with torch.cuda.stream(stream):
        step(stream)
    stream.synchronize()
    ref = [two.out.clone(), one.out.clone(), q_rot.clone(), two.k_pool.clone(), one.k_pool.clone(),
           one.v_pool.clone()]
    assert torch.equal(ref[0], ref[1]) and torch.equal(ref[3], ref[4])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step(stream)
    torch.cuda.synchronize()
    nws = fkv.decode_workspace_bytes(one.cache, one.ddesc)
    ctl = lay.num_seqs * lay.num_kv_heads * 256
    for rep in range(3):
        for t in (two.out, one.out, q_rot):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [two.out, one.out, q_rot, two.k_pool, one.k_pool, one.v_pool]
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), rep
        assert torch.count_nonzero(one.workspace[nws - ctl:nws]).item() == 0, rep
    print("[graph] norm/RoPE paths: 3 replays equal to eager", flush=True)


def test_full_54_layer_cycle_in_one_graph_against_the_oracle():
    """The whole decode cycle at context 8192 ("Laguna S 2.1 B70 campaign transfer ledger",
    section "Graph/topology lessons": whole-cycle graph coverage): 36 window-512 layers, 12
    global layers (each with its own k/v scales) and 6 draft layers at scale 1.0, one
    fkv_insert_decode launch per layer, captured in ONE HIP graph. Capture records 54 launches,
    a replay makes none on the host; every replay's output of every layer is within 2e-3 of the
    oracle and equal to the first replay bit for bit, and every pool equals the oracle's insert
    of all 8,192 tokens bit for bit."""
    import parity
    n = synth.C4_LAYERS + synth.C4_DRAFT_LAYERS
    lays = [synth.c4_layer(i) for i in range(n)]
    assert sum(1 for l in lays[:synth.C4_LAYERS] if l.window_left < 0) == 12
    assert len({(float(l.k_scale), float(l.v_scale)) for l in lays[:synth.C4_LAYERS]}) == 48
    assert all(l.k_scale == 1.0 and l.v_scale == 1.0 for l in lays[synth.C4_LAYERS:])
    layers = []
    for lay in lays:
        gl = PagedLayer(lay)
        gl.prefill()          # the 8,180 earlier tokens; the 12 new ones are inserted by the cycle
        gl.stage_new_tokens()
        layers.append(gl)
    torch.cuda.synchronize()
    print(f"[graph] {n}-layer cycle built", flush=True)
    stream = torch.cuda.Stream()
    before = fkv.get_counters()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for gl in layers:
            gl.insert_decode()
    torch.cuda.synchronize()
    mid = fkv.get_counters()
    assert mid["insert_decode_launches"] - before["insert_decode_launches"] == n
    assert mid["decode_launches"][0] - before["decode_launches"][0] == n
    assert mid["decode_combine_launches"] == before["decode_combine_launches"]  # merged inside each kernel
    first = None
    for rep in range(3):
        for gl in layers:
            gl.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        outs = [gl.out.clone() for gl in layers]
        if first is None:
            first = outs
        else:
            assert all(torch.equal(a, b) for a, b in zip(outs, first)), rep
        with torch.cuda.stream(stream):   # eager work between replays
            layers[rep].decode(stream)
        stream.synchronize()
    after = fkv.get_counters()
    assert after["insert_decode_launches"] == mid["insert_decode_launches"]  # no host launch per replay
    worst = 0.0
    for j, (lay, gl) in enumerate(zip(lays, layers)):
        kp, vp = parity.oracle_pools(lay)
        assert np.array_equal(gl.k_pool.cpu().numpy(), kp), f"layer {j}: K pool differs from the oracle"
        assert np.array_equal(gl.v_pool.cpu().numpy(), vp), f"layer {j}: V pool differs from the oracle"
        err = float(parity.row_errors(first[j].cpu().numpy()[0], parity.reference(lay, 0)).max())
        assert err <= parity.ATTN_TOL, (j, err)
        worst = max(worst, err)
    print(f"[graph] {n}-layer cycle in one graph: 3 replays, pools bit-exact, max row error {worst:.3e}", flush=True)
