"""Sliding-window layers whose pool stops growing: a sequence of a window-512 layer keeps
only the pages its window (plus the verify rows) can see, reusing R physical blocks in a
ring (page j of the sequence -> block ring[j % R]). The decode reads only the visible
pages, so the same kernels serve it; older pages' table entries point at recycled blocks
that hold newer tokens and are never visible. Checked against the oracle on the logical
sequence (fused insert + decode, and insert then decode)."""

import dataclasses
import math

import numpy as np
import pytest
import torch

from fp8_kv_paged_amd import synth
from fp8_kv_paged_amd.layer import PagedLayer

import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def _ring_layer(seq_lens, window_left, block_size, q_len=12, seed=431):
    """A sliding-window layer whose sequences each own a ring of R blocks."""
    base = synth.tiny_layer(seed, seq_lens, num_q_heads=18, num_kv_heads=2, block_size=block_size, q_len=q_len,
                            window_left=window_left, outlier_rate=0.01)
    R = math.ceil((window_left + 1 + q_len) / block_size) + 1
    B = len(seq_lens)
    rng = np.random.default_rng(seed)
    phys = rng.permutation(B * R + 3).astype(np.int32)  # a few blocks never used
    table = np.zeros_like(base.block_table)
    for b in range(B):
        ring = phys[b * R:(b + 1) * R]
        table[b] = ring[np.arange(table.shape[1]) % R]
    return dataclasses.replace(base, block_table=table, num_blocks=B * R + 3), R


def _fill(gl, lay, R, upto):
    """Insert tokens [0, upto(b)) of every sequence one ring generation per call, so a call
    never holds two tokens for one slot and later generations overwrite earlier ones."""
    gen = R * lay.block_size
    for b in range(lay.num_seqs):
        end = upto(b)
        for c0 in range(0, end, gen):
            gl.insert_tokens(b, c0, min(end, c0 + gen), chunk=gen)


def _check(lay, out, label):
    gpu = out.cpu().numpy()
    worst = max(float(parity.row_errors(gpu[b], parity.reference(lay, b)).max()) for b in range(lay.num_seqs))
    print(f"[window ring] {label}: max row error {worst:.3e}", flush=True)
    assert worst <= parity.ATTN_TOL, (label, worst)


@pytest.mark.parametrize("block_size", [32, 64])
@pytest.mark.parametrize("fused", [False, True])
def test_window_ring_decode(block_size, fused):
    lay, R = _ring_layer([4000, 700, 2049, 530], 511, block_size)
    pages = [math.ceil(int(L) / block_size) for L in lay.seq_lens]
    assert lay.num_blocks < sum(pages)  # the pool is smaller than the sequences' pages
    gl = PagedLayer(lay)
    M = lay.q_len
    _fill(gl, lay, R, lambda b: int(lay.seq_lens[b]) - M)
    if fused:
        gl.stage_new_tokens()
        out = gl.insert_decode()
    else:
        gl.stage_step()
        gl.insert_step()
        out = gl.decode()
    torch.cuda.synchronize()
    _check(lay, out, f"page {block_size} {'fused' if fused else 'insert + decode'}, {R} blocks per sequence")


def test_window_ring_steps():
    """Decode steps past several ring wraps: each step inserts 12 tokens into recycled blocks."""
    final, R = _ring_layer([1500, 900], 511, 64, seed=433)
    gl = PagedLayer(final)
    M = final.q_len
    steps = 4
    _fill(gl, final, R, lambda b: int(final.seq_lens[b]) - M * steps)
    for step in range(steps):
        lay = dataclasses.replace(final, seq_lens=(final.seq_lens - M * (steps - 1 - step)).astype(np.int32))
        gl.lay = lay
        gl.seq_lens.copy_(torch.from_numpy(lay.seq_lens))
        gl.stage_new_tokens()
        out = gl.insert_decode()
        torch.cuda.synchronize()
        _check(lay, out, f"step {step}")
