"""Benchmark of the calibrated-FP8 paged KV hot path on one MI355X.

One step = one layer call of the full path on the 72-query / 8-KV-head layer at
context 8,192 with a 12-token causal verify window (M=12), global attention, page
64: the 12 new BF16 K/V tokens inserted into the FP8 cache (E4M3 with per-tensor
scales) and paged GQA decode attention over the FP8 pages, in one
fkv_insert_decode launch (split partials merged inside the kernel). The timed steps
are replayed from one captured HIP graph and checked bit for bit against the eager
steps; every timed step uses its own layer copy (different pools, identical
contents) and the copies together exceed the 256 MB Infinity Cache, so K/V comes
from HBM. Insert and decode as two launches are timed beside it.

Prints ONE JSON line. `value` is K/V-read throughput of the whole step
(algorithmic K/V bytes / step time); `roofline` is that kernel's HBM roofline
(achieved bandwidth from HIP events on its launch stream, traffic from the
committed rocprofv3 counter summary when it was taken on this source);
`cpu_baseline` times the NumPy oracle on host cores (all threads, and one thread).
Further keys, each measured in the same run: the 32k-context step, the page-32 vs
page-64 A/B at 8k and 32k, the q1 fused step at 8k and 32k, the 32-sequence batch
with FP8 and BF16 caches, the
attainable read bandwidth of the box (a stream-read probe), and the MFMA busy share
from the committed counter profile of this source.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--context", type=int, default=8192)
    p.add_argument("--block-size", type=int, default=64)
    p.add_argument("--q-len", type=int, default=12)
    p.add_argument("--copies", type=int, default=0, help="layer copies to rotate over (0 = enough for 1 GiB)")
    p.add_argument("--split-tiles", type=int, default=0)
    p.add_argument("--layout", type=int, default=0, help="decode work-group layout (0 = automatic)")
    p.add_argument("--row-groups", type=int, default=0, help="layout 5: row groups per split (0 = automatic)")
    p.add_argument("--cache-dtype", default="fp8_e4m3fn")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=8.0, help="seconds of oracle work per thread setting")
    p.add_argument("--headline-only", action="store_true",
                   help="only the headline step (no 32k, A/B, batch, probe or CPU sections; for profilers)")
    p.add_argument("--suite", action="store_true",
                   help="also time the other workloads (C1, C2, the C4 cycle eager and as a HIP graph, C5, "
                        "the Q/K norm + RoPE step and a 512-token prefill chunk); no CPU baseline")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run device-to-device copies of MIB MiB (scales the HBM byte counters)")
    return p.parse_args()


def algorithmic_bytes(context, q_len, hq, hkv, block_size, elem):
    kv = context * hkv * 2 * 128 * elem          # every visible key and value once
    q = q_len * hq * 128 * 2
    out = q_len * hq * 128 * 4
    meta = ((context + block_size - 1) // block_size) * 4 + 4
    return kv, q + out + meta


def insert_bytes(q_len, hkv, elem):
    """BF16 K and V of the new tokens in, the cache's bytes out."""
    return q_len * hkv * 128 * 2 * (2 + elem)


def run_gpu(args, context, block_size, cache_dtype, steps, warmup, separate=True):
    import torch
    from fp8_kv_paged_amd import fkv, synth
    from fp8_kv_paged_amd.layer import PagedLayer

    lay = synth.make_layer(f"c3_m{args.q_len}_{context}_p{block_size}", 1003, 0, 72, 8, block_size, args.q_len, -1,
                           [context], cache_dtype=cache_dtype)
    base = PagedLayer(lay, split_tiles=args.split_tiles, layout=args.layout, row_groups=args.row_groups).build()
    kv_bytes, other = algorithmic_bytes(context, args.q_len, 72, 8, block_size, 1 if cache_dtype == "fp8_e4m3fn" else 2)
    pool_total = 2 * base.k_pool.numel()
    # each step (warm-up and timed) gets its own copy until the copies hold 1 GiB of K/V
    copies = args.copies or min(warmup + steps, max(2, math.ceil((1 << 30) / kv_bytes)))
    layers = [base]
    for _ in range(copies - 1):
        c = PagedLayer(lay, poison=False, split_tiles=args.split_tiles, layout=args.layout, row_groups=args.row_groups)
        c.k_pool.copy_(base.k_pool)
        c.v_pool.copy_(base.v_pool)
        c.step_k, c.step_v, c.step_slots = base.step_k, base.step_v, base.step_slots
        layers.append(c)
    torch.cuda.synchronize()

    fused_ok = cache_dtype == "fp8_e4m3fn" and args.layout in (0, 5, 6)
    if fused_ok:
        base.stage_new_tokens()
        for c in layers[1:]:
            c.new_k, c.new_v = base.new_k, base.new_v
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    mean = lambda xs: sum(xs) / len(xs)
    med = lambda xs: sorted(xs)[len(xs) // 2]
    fkv.reset_counters()
    touched = len({(warmup + i) % copies for i in range(steps)})  # copies the timed steps read
    res = dict(kv_bytes=kv_bytes, other_bytes=other, copies=copies, copies_timed=touched,
               working_set=touched * kv_bytes, plan_ws=base.workspace.numel(), fused_insert=fused_ok)
    with torch.cuda.stream(stream):
        # the decode step as one launch: the new tokens' insert fused into the attention call
        if fused_ok:
            for i in range(warmup):
                layers[i % copies].insert_decode(stream)
            stream.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                e0, e1 = ev[i]
                e0.record(stream)
                layers[(warmup + i) % copies].insert_decode(stream)
                e1.record(stream)
            stream.synchronize()
            res["fused_wall_ms_per_step"] = (time.perf_counter() - t0) * 1e3 / steps
            f_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
            res["fused_ms"], res["fused_ms_median"] = mean(f_ms), med(f_ms)
            # The timed whole job: the same K steps captured in one HIP graph (host launch cost
            # out of the loop), replayed between two synchronizations. Every layer copy computes
            # the same output; each replay is checked bit for bit against the eager result.
            ref = base.out.clone()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(steps):
                    layers[(warmup + i) % copies].insert_decode()
            torch.cuda.synchronize()

            def replay_checked(timed):
                for c in layers:
                    c.out.fill_(float("nan"))
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                t0 = time.perf_counter()
                e0.record(stream)
                g.replay()
                e1.record(stream)
                stream.synchronize()
                wall = time.perf_counter() - t0
                used = {(warmup + i) % copies for i in range(steps)}
                assert all(torch.equal(layers[k].out, ref) for k in used), "graph replay differs from eager"
                return e0.elapsed_time(e1), wall

            replay_checked(False)
            gms, gwall = replay_checked(True)
            res["graph_ms_per_step"] = gms / steps
            res["graph_wall_ms_per_step"] = gwall * 1e3 / steps
            # Hot, labelled apart: the same K steps on one layer copy, whose K/V stays resident
            # in the 256 MB Infinity Cache between steps (not the headline)
            gh = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gh, stream=stream):
                for i in range(steps):
                    base.insert_decode()
            torch.cuda.synchronize()
            hot = []
            for _ in range(2):
                base.out.fill_(float("nan"))
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                gh.replay()
                e1.record(stream)
                stream.synchronize()
                assert torch.equal(base.out, ref), "hot graph replay differs from eager"
                hot.append(e0.elapsed_time(e1) / steps)
            res["hot_graph_ms_per_step"] = hot[-1]
        if not separate:
            return res
        # the same step as two launches: insert, then decode
        for i in range(warmup):
            L = layers[i % copies]
            L.insert_step(stream)
            L.decode(stream)
        stream.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            L = layers[(warmup + i) % copies]
            e0, e1, e2 = ev[i]
            e0.record(stream)
            L.insert_step(stream)
            e1.record(stream)
            L.decode(stream)
            e2.record(stream)
        stream.synchronize()
        torch.cuda.synchronize()
        res["wall_ms_per_step"] = (time.perf_counter() - t0) * 1e3 / steps
    step_ms = [ev[i][0].elapsed_time(ev[i][2]) for i in range(steps)]
    ins_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(steps)]
    dec_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(steps)]
    cnt = fkv.get_counters()
    nt = (72 // 8 * args.q_len + 15) // 16
    fused_calls = 3 * steps + warmup if fused_ok else 0  # eager steps, then the two captured graphs
    calls = steps + warmup + fused_calls
    assert cnt["decode_row_tiles"][0 if cache_dtype == "fp8_e4m3fn" else 1][nt - 1] == calls, cnt
    assert cnt["insert_decode_launches"] == fused_calls, cnt
    res.update(step_ms=mean(step_ms), insert_ms=mean(ins_ms), decode_ms=mean(dec_ms), decode_ms_median=med(dec_ms),
               combine=cnt["decode_combine_launches"] > 0, fused=cnt["decode_combine_launches"] == 0)
    return res


def _time_calls(fn, stream, iters, warmup):
    """Median and mean event time (ms) of fn() on stream."""
    import torch
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            fn()
        stream.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        stream.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    return t[len(t) // 2], sum(t) / len(t)


def _visible_kv_bytes(lay, elem):
    """Algorithmic K/V bytes of one decode call: every key visible to some row, once."""
    tot = 0
    for L in lay.seq_lens:
        L = int(L)
        lo = 0 if lay.window_left < 0 else max(0, L - lay.q_len - lay.window_left)
        tot += (L - lo) * lay.num_kv_heads * 2 * 128 * elem
    return tot


def run_suite(iters):
    """The other workloads of the scope table, timed with HIP events (median): the Q/K norm +
    RoPE + insert step and a 512-token prefill chunk of the 72/8 layer, C1 / C2 single layers,
    the 54-layer C4 cycle eager and as a captured HIP graph, and the 32-sequence C5 batch with
    FP8 and BF16 caches at M = 1 and 12. Each section prints a progress line on stderr."""
    import torch
    from fp8_kv_paged_amd import synth
    from fp8_kv_paged_amd.layer import PagedLayer
    stream = torch.cuda.Stream()
    out = {}

    def layer_step(lay, fused=True, layout=0):
        gl = PagedLayer(lay, layout=layout)
        gl.prefill()
        gl.stage_step()
        if fused:
            gl.stage_new_tokens()
        return gl

    # Q/K RMSNorm + RoPE + insert of one step's new tokens (72/8 heads): the 8k layer's 12
    # tokens and the 32-sequence batch's 384. Bytes: raw Q, K, V and the table rows read,
    # rotated Q and the FP8 K/V written.
    def progress(msg):
        print(f"[suite] {msg}", file=sys.stderr, flush=True)

    for name, lay in (("norm_rope_insert_c3_m12", synth.c3_layer(8192, 64)),):
        progress(name)
        gl = PagedLayer(lay)
        gl.stage_norm_rope(synth.norm_rope_step(lay))
        nm, _ = _time_calls(lambda: gl.norm_rope_insert(stream), stream, iters, 20)
        T = lay.num_seqs * lay.q_len
        nbytes = T * (lay.num_q_heads * 128 * 2 * 2 + lay.num_kv_heads * 128 * (2 + 2 + 1 + 1) + 128 * 4 + 8)
        out[name] = {"us": round(nm * 1e3, 3), "tokens": T, "bytes": nbytes,
                     "gbs": round(nbytes / (nm * 1e-3) / 1e9, 1)}
        del gl
        torch.cuda.empty_cache()

    # Chunked prefill on the 32-row kernel: 512 new tokens of a 72/8 layer attending to an
    # 8k prefix and causally to each other (4,608 packed rows per KV head). Algorithmic work:
    # 4 flops per (row, visible key, dim) for QK^T and PV.
    for name, M, L in (("prefill_q512_ctx8192", 512, 8192),):
        progress(name)
        lay = synth.tiny_layer(1006, [L], num_q_heads=72, num_kv_heads=8, block_size=64, q_len=M)
        gl = PagedLayer(lay).build()
        pm, _ = _time_calls(lambda: gl.decode(stream), stream, max(10, iters // 10), 3)
        vis = sum(L - M + i + 1 for i in range(M))
        flops = 4 * 128 * lay.num_q_heads * vis
        out[name] = {"us": round(pm * 1e3, 2), "q_len": M, "context": L, "flops": flops,
                     "tflops": round(flops / (pm * 1e-3) / 1e12, 1),
                     "mfma_bf16_frac": round(flops / (pm * 1e-3) / 2.5e15, 3)}
        del gl
        torch.cuda.empty_cache()

    for name, make in (("c1", synth.c1_layer), ("c2", synth.c2_layer)):
        progress(name)
        lay = make()
        gl = layer_step(lay)
        fm, _ = _time_calls(lambda: gl.insert_decode(stream), stream, iters, 20)
        dm, _ = _time_calls(lambda: gl.decode(stream), stream, iters, 20)
        im, _ = _time_calls(lambda: gl.insert_step(stream), stream, iters, 20)
        kv = _visible_kv_bytes(lay, 1)
        out[name] = {"fused_step_us": round(fm * 1e3, 3), "decode_us": round(dm * 1e3, 3),
                     "insert_us": round(im * 1e3, 3), "kv_bytes": kv}

    # C4: 48 target layers (36 sliding-window, 12 global) + 6 draft layers at context 8192;
    # one cycle = one fused insert + decode call per layer. Two copies of the cycle's layers
    # are alternated so consecutive cycles do not find the K/V in the 256 MB Infinity Cache.
    progress("c4 cycle")
    layers = [synth.c4_layer(i) for i in range(synth.C4_LAYERS + synth.C4_DRAFT_LAYERS)]
    copies = [[layer_step(lay) for lay in layers] for _ in range(2)]
    kv54 = sum(_visible_kv_bytes(lay, 1) for lay in layers)
    kv48 = sum(_visible_kv_bytes(lay, 1) for lay in layers[:synth.C4_LAYERS])
    which = [0]

    def cycle_eager():
        c = copies[which[0] % 2]
        which[0] += 1
        for gl in c:
            gl.insert_decode(stream)

    em, _ = _time_calls(cycle_eager, stream, max(20, iters // 4), 4)
    graphs = []
    for c in copies:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for gl in c:
                gl.insert_decode()
        graphs.append(g)
    torch.cuda.synchronize()
    # every replay must reproduce the eager outputs bit for bit (eager work in between)
    for c, g in zip(copies, graphs):
        with torch.cuda.stream(stream):
            for gl in c:
                gl.insert_decode(stream)
        stream.synchronize()
        ref = [gl.out.clone() for gl in c]
        for _ in range(3):
            for gl in c:
                gl.out.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert all(torch.equal(gl.out, r) for gl, r in zip(c, ref)), "graph replay differs from eager"
            with torch.cuda.stream(stream):
                c[0].decode(stream)
            stream.synchronize()
    def cycle_graph():
        which[0] += 1
        graphs[which[0] % 2].replay()

    gm, _ = _time_calls(cycle_graph, stream, max(20, iters // 4), 4)
    out["c4_cycle"] = {"layers": len(layers), "eager_us": round(em * 1e3, 2), "graph_us": round(gm * 1e3, 2),
                       "graph_us_per_layer": round(gm * 1e3 / len(layers), 3), "kv_bytes_54_layers": kv54,
                       "kv_bytes_48_layers": kv48, "graph_kv_gbs": round(kv54 / (gm * 1e-3) / 1e9, 1),
                       "replays_checked": 6}
    del copies, graphs
    torch.cuda.empty_cache()

    # C5: 32 sequences, 72/8 heads, contexts log-uniform in [1k, 128k], page 32, one pool
    for q_len in (12, 1):
        progress(f"c5 q_len {q_len}")
        for dt in ("fp8_e4m3fn", "bf16"):
            lay = synth.c5_layer(q_len=q_len, cache_dtype=dt)
            fp8 = dt == "fp8_e4m3fn"
            gl = layer_step(lay, fused=fp8)
            dm, _ = _time_calls(lambda: gl.decode(stream), stream, max(20, iters // 4), 5)
            kv = _visible_kv_bytes(lay, 1 if fp8 else 2)
            rec = {"decode_us": round(dm * 1e3, 2), "kv_bytes": kv, "decode_kv_gbs": round(kv / (dm * 1e-3) / 1e9, 1),
                   "layout": ("5 (32-row kernel)" if fp8 and q_len > 1 else "3 (row-group kernel)")}
            if fp8:
                fm, _ = _time_calls(lambda: gl.insert_decode(stream), stream, max(20, iters // 4), 5)
                rec["fused_step_us"] = round(fm * 1e3, 2)
                rec["fused_kv_gbs"] = round(kv / (fm * 1e-3) / 1e9, 1)
            out[f"c5_m{q_len}_{'fp8' if fp8 else 'bf16'}"] = rec
            del gl
            torch.cuda.empty_cache()
            if fp8:
                # the FP8 cache through the BF16 cache's kernel (layout 3): the same-kernel comparison
                gl = layer_step(lay, fused=False, layout=3)
                dm, _ = _time_calls(lambda: gl.decode(stream), stream, max(20, iters // 4), 5)
                out[f"c5_m{q_len}_fp8_layout3"] = {"decode_us": round(dm * 1e3, 2), "kv_bytes": kv,
                                                   "decode_kv_gbs": round(kv / (dm * 1e-3) / 1e9, 1)}
                del gl
                torch.cuda.empty_cache()
    return out


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_steps(seconds):
    """The NumPy oracle (as it stands) on the host: insert 12 tokens + paged decode of the 8k
    layer, repeated until about `seconds` of CPU work. Returns (steps, elapsed seconds)."""
    from fp8_kv_paged_amd import synth
    from oracle import attention, paged
    lay = synth.c3_layer(8192, 64)
    kp, vp = paged.new_pools(lay.num_blocks, 64, 8, paged.FP8)
    L = int(lay.seq_lens[0])
    k, v = lay.kv_bits(0, 0, L - 12)
    paged.insert(kp, vp, k, v, lay.slots(0, 0, L - 12), lay.k_scale, lay.v_scale, 64, 8, paged.FP8)
    ks, vs = lay.kv_bits(0, L - 12, L)
    sl = lay.slots(0, L - 12, L)
    q = lay.q_bits()
    n, t0 = 0, time.perf_counter()
    while True:
        paged.insert(kp, vp, ks, vs, sl, lay.k_scale, lay.v_scale, 64, 8, paged.FP8)
        attention.paged_decode(kp, vp, q, lay.block_table, lay.seq_lens, 12, -1, lay.softmax_scale,
                               lay.k_scale, lay.v_scale, 64, 8, paged.FP8)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return n, el


def cpu_baseline(seconds):
    """The oracle timed with the BLAS pool at all its threads, then at one thread (about
    `seconds` each). `value` is the all-threads figure in the metric's unit (K/V GB/s)."""
    import threadpoolctl
    kv_bytes = 8192 * 8 * 256
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    n, el = _oracle_steps(seconds)
    with threadpoolctl.threadpool_limits(limits=1):
        n1, el1 = _oracle_steps(seconds)
    sample = "oracle steps (12-token insert + paged decode, 72/8 heads, context 8192, M=12, page 64)"
    return {"value": round(kv_bytes * n / el / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} {sample}, {el:.1f} s, {el / n * 1e3:.1f} ms/step",
            "us_per_layer": round(el / n * 1e6, 1),
            "single_thread": {"value": round(kv_bytes * n1 / el1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "us_per_layer": round(el1 / n1 * 1e6, 1), "sample": f"{n1} {sample}, {el1:.1f} s"},
            "cpu_model": _cpu_model(), "os_cpu_count": os.cpu_count(),
            "affinity_cores": len(os.sched_getaffinity(0)), "blas": [i.get("internal_api") for i in info]}


# ---- further sections of the default run ---------------------------------------------------

def device_prefill(gl, seed):
    """Fills a layer's cache with N(0, 1) BF16 K/V drawn on the GPU (seeded) through fkv_insert,
    in 32k-token chunks: timing needs the pages' sizes and value distribution, not the host
    draws the parity tests compare (generating 860k tokens on the host takes minutes)."""
    import torch
    from fp8_kv_paged_amd import fkv
    lay = gl.lay
    g = torch.Generator(device=gl.device).manual_seed(seed)
    H = lay.num_kv_heads
    for b in range(lay.num_seqs):
        L = int(lay.seq_lens[b])
        for c0 in range(0, L, 32768):
            c1 = min(L, c0 + 32768)
            k = torch.randn((c1 - c0, H, 128), generator=g, device=gl.device).to(torch.bfloat16)
            v = torch.randn((c1 - c0, H, 128), generator=g, device=gl.device).to(torch.bfloat16)
            slots = torch.from_numpy(lay.slots(b, c0, c1)).to(gl.device)
            fkv.insert(gl.cache, k, v, slots, gl.k_scale, gl.v_scale)
    torch.cuda.synchronize()


def run_batch(iters):
    """The 32-sequence batch (72/8 heads, contexts log-uniform in [1k, 128k], page 32, one shared
    interleaved pool), FP8 against BF16 caches at M = 12 and M = 1: the automatic kernel of each
    cache, and the FP8 cache through the BF16 cache's kernel (layout 3: the same code reading
    half the bytes). Decode calls timed with HIP events (median)."""
    import torch
    from fp8_kv_paged_amd import synth
    from fp8_kv_paged_amd.layer import PagedLayer
    stream = torch.cuda.Stream()
    out = {}
    for dt in ("fp8_e4m3fn", "bf16"):
        fp8 = dt == "fp8_e4m3fn"
        base = synth.c5_layer(12, cache_dtype=dt)
        kv = _visible_kv_bytes(base, 1 if fp8 else 2)
        gl = PagedLayer(base)
        device_prefill(gl, 1005)
        for q_len in (12, 1):
            lay = synth.c5_layer(q_len, cache_dtype=dt)
            for layout in ((0, 3) if fp8 else (0,)):
                g2 = PagedLayer(lay, layout=layout, poison=False) if (q_len, layout) != (12, 0) else gl
                if g2 is not gl:
                    g2.k_pool, g2.v_pool, g2.cache = gl.k_pool, gl.v_pool, gl.cache
                med, _ = _time_calls(lambda: g2.decode(stream), stream, iters, 3)
                key = f"m{q_len}_{'fp8' if fp8 else 'bf16'}" + ("_layout3" if layout == 3 else "")
                out[key] = {"decode_us": round(med * 1e3, 2), "kv_bytes": kv,
                            "kv_gbs": round(kv / (med * 1e-3) / 1e9, 1),
                            "kv_pct_of_peak": round(100 * kv / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                            "kernel": "decode_rows_kernel (layout 3)" if (layout == 3 or not fp8 or q_len == 1)
                            else "decode_m32_kernel (layout 5)"}
                if g2 is not gl:
                    del g2
        del gl
        torch.cuda.empty_cache()
    for m in (12, 1):
        f, b16 = out[f"m{m}_fp8_layout3"]["decode_us"], out[f"m{m}_bf16"]["decode_us"]
        out[f"m{m}_fp8_over_bf16_time_same_kernel"] = round(f / b16, 3)
        out[f"m{m}_fp8_over_bf16_time_automatic"] = round(out[f"m{m}_fp8"]["decode_us"] / b16, 3)
    out["workload"] = ("32 sequences, 72 Q / 8 KV heads, contexts log-uniform in [1,024, 131,072] (sum "
                       f"{int(synth.c5_seq_lens().sum())} tokens), global, page 32; decode only")
    return out


def stream_probe():
    """Attainable read bandwidth of the box: one pass of the stream-read probe over 16 MiB,
    64 MiB and 2 GiB buffers (median of 20 passes each; the two small buffers fit in the 256 MB
    Infinity Cache and are labelled so)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "fp8_kv_paged_amd", "libfkv_probe.so"))
    lib.fkv_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_void_p]
    stream = torch.cuda.Stream()
    blocks = 256 * 8
    sink = torch.empty((blocks,), dtype=torch.int32, device="cuda")
    out = {}
    for name, nbytes in (("16MiB_cache_resident", 16 << 20), ("64MiB_cache_resident", 64 << 20), ("2GiB", 2 << 30)):
        buf = torch.ones((nbytes // 4,), dtype=torch.int32, device="cuda")

        def fn():
            rc = lib.fkv_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                           blocks, ctypes.c_void_p(stream.cuda_stream))
            assert rc == 0, rc
        med, _ = _time_calls(fn, stream, 20, 3)
        out[name] = {"gbs": round(nbytes / (med * 1e-3) / 1e9, 1), "us": round(med * 1e3, 2)}
        del buf
    torch.cuda.empty_cache()
    out["kernel"] = ("stream_read_kernel: 2,048 work groups x 256 threads, one contiguous chunk per work group, "
                     "16-byte nontemporal loads, 8 in flight per thread")
    return out


def counter_profile(src_hash):
    """MFMA busy share and VALU instructions per MFMA of the decode kernel from the committed
    rocprofv3 SQ counter summary, when it was taken on this source (else None)."""
    p = os.path.join(ROOT, "profiles", "decode_sq_counters.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != src_hash:
        return None
    return d.get("configs")


# split kernel each decode layout launches (layout 0, the automatic choice, is the 32-row kernel for FP8)
DECODE_KERNELS = {0: "decode_m32_kernel", 3: "decode_rows_kernel", 5: "decode_m32_kernel", 6: "decode_m32_kernel"}


def source_hash():
    """Hash of the library's kernel and host sources (csrc/*, not the benchmark's probe)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "fp8_kv_paged_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if os.path.isfile(os.path.join(d, f)):
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(src_hash, cfg_name):
    """HBM bytes per decode call from the committed PMC summary, if it was taken on this source."""
    p = os.path.join(ROOT, "profiles", "decode_pmc_traffic.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != src_hash or cfg_name not in d.get("configs", {}):
        return None
    return d["configs"][cfg_name].get("hbm_bytes_per_call")


def copy_calibration(mib, steps):
    """Plain device-to-device copies of a known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = mib << 20
    src = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "copies": steps}),
          flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one MI355X: --gpus {args.gpus} is not supported (the path runs on one GPU; "
              "see the sharding note in DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(1, min(args.steps, 10)))
        return
    r = run_gpu(args, args.context, args.block_size, args.cache_dtype, args.steps, args.warmup)
    kv = r["kv_bytes"]
    ins_bytes = insert_bytes(args.q_len, 8, 1 if args.cache_dtype == "fp8_e4m3fn" else 2)
    if r["fused_insert"]:
        # one launch per step, K steps replayed from one HIP graph: the roofline covers the
        # whole step (decode and insert bytes)
        step_ms = r["graph_ms_per_step"]
        alg = kv + r["other_bytes"] + ins_bytes
        kernel = "decode_m32_kernel (insert fused into decode, one launch per step)"
        kernel_ms = r["graph_ms_per_step"]
    else:
        step_ms = r["step_ms"]
        alg = kv + r["other_bytes"]
        kernel = f"{DECODE_KERNELS[args.layout]}" + ("" if r["fused"] else " + decode_combine_kernel") + " (one decode call)"
        kernel_ms = r["decode_ms"]
    value = kv / (step_ms * 1e-3) / 1e9
    achieved = alg / (kernel_ms * 1e-3) / 1e9
    src = source_hash()
    cfg_name = f"c3_m{args.q_len}_{args.context}_p{args.block_size}_{args.cache_dtype}"
    line = {
        "metric": "decode-attn µs/layer and KV-read HBM GB/s (% of peak) at M=12, 8k ctx",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3fn KV, bf16 Q, f32 accumulate" if args.cache_dtype == "fp8_e4m3fn" else "bf16",
        "data": "synthetic",
        "config": {"workload": f"full layer, 72 Q / 8 KV heads, head 128, context {args.context}, M={args.q_len} "
                               f"causal, global, page {args.block_size}, {args.cache_dtype} cache; one step = insert "
                               f"the {args.q_len} new tokens + decode attention",
                   "context": args.context, "q_len": args.q_len, "block_size": args.block_size,
                   "layer_copies": r["copies"], "layer_copies_timed": r["copies_timed"],
                   "working_set_bytes": r["working_set"], "split_tiles": args.split_tiles},
        "us_per_layer": round(step_ms * 1e3, 3),
        "step_launches": 1 if r["fused_insert"] else 2,
        "separate_launches": {"step_us": round(r["step_ms"] * 1e3, 3), "insert_us": round(r["insert_ms"] * 1e3, 3),
                              "decode_us": round(r["decode_ms"] * 1e3, 3),
                              "decode_us_median": round(r["decode_ms_median"] * 1e3, 3)},
        "decode_us_per_layer": round(r["decode_ms"] * 1e3, 3),
        "kv_read_pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile(src, cfg_name),
                     "kernel": kernel, "algorithmic_bytes": alg},
        "source_hash": src,
    }
    if r["fused_insert"]:
        line["config"]["launch"] = (f"the {args.steps} timed steps replayed from one captured HIP graph, "
                                    "outputs checked bitwise against eager")
        line["graph_wall_us_per_step"] = round(r["graph_wall_ms_per_step"] * 1e3, 3)
        line["hot_mall_resident_us_per_step"] = round(r["hot_graph_ms_per_step"] * 1e3, 3)
        line["eager_fused"] = {"event_us_per_step": round(r["fused_ms"] * 1e3, 3),
                               "event_us_median": round(r["fused_ms_median"] * 1e3, 3),
                               "wall_us_per_step": round(r["fused_wall_ms_per_step"] * 1e3, 3)}
    line["separate_launches"]["wall_us_per_step"] = round(r["wall_ms_per_step"] * 1e3, 3)
    if not args.headline_only:
        progress = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)
        progress("32k step")
        r32 = run_gpu(args, 32768, args.block_size, args.cache_dtype, args.steps, args.warmup, separate=False)
        alg32 = r32["kv_bytes"] + r32["other_bytes"] + ins_bytes
        ms32 = r32["graph_ms_per_step"]
        line["c3_32k"] = {"us_per_layer": round(ms32 * 1e3, 3),
                          "kv_gbs": round(r32["kv_bytes"] / (ms32 * 1e-3) / 1e9, 1),
                          "kv_pct_of_peak": round(100 * r32["kv_bytes"] / (ms32 * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                          "roofline_frac": round(alg32 / (ms32 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "eager_event_us": round(r32["fused_ms"] * 1e3, 3),
                          "hot_mall_resident_us": round(r32["hot_graph_ms_per_step"] * 1e3, 3),
                          "layer_copies_timed": r32["copies_timed"],
                          "working_set_bytes": r32["working_set"],
                          "workload": "72/8 heads, context 32768, M=12, global, page 64; one graph-replayed "
                                      "fkv_insert_decode step"}
        progress("page 32 vs 64")
        ab = {}
        for ctx in (8192, 32768):
            for bs in (32, 64):
                rr = r if (ctx, bs) == (args.context, args.block_size) else (
                    r32 if (ctx, bs) == (32768, args.block_size) else
                    run_gpu(args, ctx, bs, args.cache_dtype, args.steps, args.warmup, separate=False))
                ms = rr["graph_ms_per_step"]
                ab[f"{ctx}_p{bs}"] = {"us_per_layer": round(ms * 1e3, 3),
                                      "kv_gbs": round(rr["kv_bytes"] / (ms * 1e-3) / 1e9, 1)}
        for ctx in (8192, 32768):
            ab[f"{ctx}_p32_over_p64_time"] = round(ab[f"{ctx}_p32"]["us_per_layer"] / ab[f"{ctx}_p64"]["us_per_layer"], 3)
        ab["workload"] = "72/8 heads, M=12, global; graph-replayed fkv_insert_decode steps, same source"
        line["page_ab"] = ab
        progress("q1 steps")
        a1 = argparse.Namespace(**{**vars(args), "q_len": 1})
        q1 = {}
        for ctx in (8192, 32768):
            rq = run_gpu(a1, ctx, args.block_size, args.cache_dtype, args.steps, args.warmup, separate=False)
            ms = rq["graph_ms_per_step"]
            q1[str(ctx)] = {"us_per_layer": round(ms * 1e3, 3),
                            "kv_gbs": round(rq["kv_bytes"] / (ms * 1e-3) / 1e9, 1),
                            "hot_mall_resident_us": round(rq["hot_graph_ms_per_step"] * 1e3, 3)}
        q1["workload"] = "72/8 heads, q_len 1, global, page 64; graph-replayed fkv_insert_decode steps"
        line["q1_steps"] = q1
        progress("32-sequence batch, FP8 and BF16 caches")
        line["batch_fp8_vs_bf16"] = run_batch(max(10, args.steps))
        progress("stream-read probe")
        line["attainable_read_bw"] = stream_probe()
        line["kv_read_pct_of_attainable"] = round(100 * value / line["attainable_read_bw"]["2GiB"]["gbs"], 2)
        line["counters"] = counter_profile(src)
    if args.suite:
        line["suite"] = run_suite(args.steps)
    # the CPU baseline belongs to the headline line; the suite's line omits it
    if not args.no_cpu_baseline and not args.suite and not args.headline_only:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
