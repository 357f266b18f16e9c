"""Seeded synthetic workloads for the FP8 paged KV path.

This module only draws inputs: random BF16 Q/K/V, per-layer scalar scales,
sequence lengths, page tables and slot mappings. It holds none of the method's
arithmetic (no quantisation, no attention) and imports neither the HIP binding
nor the oracle; tests, the bench and the smoke check feed the same draws to both.

Workload shapes follow the pages: q=18 / kv=2 per TP4 rank, head 128, page 32
and 64, global and sliding windows ("Laguna FP8 KV -- replicated embedding win,
page-32 build, and host boundary", section "Page-32 attention experiment"); the
full 8-KV-head layer and the 36 sliding (512) + 12 global layer mix ("Laguna S
2.1 KV-cache precision decision", section "BF16 versus FP8 in concrete terms");
width-12 verify windows and six unit-scale draft cache layers ("Laguna S 2.1
INT4 -- calibrated FP8 KV on Intel B70", section Contract).

Value recipe: every float is drawn in float32 from numpy's PCG64 and rounded to
BF16 with round-to-nearest-even. Seeds are 1000 + workload number; each
sequence / tensor / 4096-token chunk has its own child stream so any slice of a
long context can be regenerated alone.
"""

from dataclasses import dataclass, field
import math

import numpy as np

HEAD_DIM = 128
CHUNK = 4096  # tokens per independently seeded chunk of context K/V


def f32_to_bf16_bits(x):
    """Round float32 to BF16 (nearest, ties to even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _rng(*key):
    return np.random.default_rng([int(k) for k in key])


@dataclass
class Layer:
    """One attention layer's synthetic state for a batch of sequences."""
    name: str
    seed: int
    layer_id: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    block_size: int
    q_len: int
    window_left: int
    seq_lens: np.ndarray            # int32 [B], cached tokens after the q_len new ones
    block_table: np.ndarray         # int32 [B, max_blocks]
    num_blocks: int                 # physical blocks in the pool
    k_scale: np.float32
    v_scale: np.float32
    kv_std: float = 1.0
    outlier_rate: float = 0.0       # fraction of channels scaled x8
    cache_dtype: str = "fp8_e4m3fn"
    softmax_scale: float = 1.0 / math.sqrt(HEAD_DIM)
    _q: np.ndarray = field(default=None, repr=False)

    @property
    def max_blocks(self):
        return self.block_table.shape[1]

    def _outlier_mask(self, which, heads):
        if self.outlier_rate <= 0:
            return None
        r = _rng(self.seed, self.layer_id, 7, which)
        return np.where(r.random((heads, HEAD_DIM)) < self.outlier_rate, 8.0, 1.0).astype(np.float32)

    def q_bits(self):
        """BF16 queries [B, M, Hq, 128]."""
        if self._q is None:
            r = _rng(self.seed, self.layer_id, 1)
            q = r.standard_normal((self.num_seqs, self.q_len, self.num_q_heads, HEAD_DIM), dtype=np.float32)
            m = self._outlier_mask(2, self.num_q_heads)
            if m is not None:
                q = q * m[None, None]
            self._q = f32_to_bf16_bits(q)
        return self._q

    def kv_bits(self, b, t0, t1):
        """BF16 K and V [t1 - t0, Hkv, 128] for tokens [t0, t1) of sequence b."""
        ks, vs = [], []
        c0, c1 = t0 // CHUNK, (t1 + CHUNK - 1) // CHUNK
        mk = self._outlier_mask(3, self.num_kv_heads)
        mv = self._outlier_mask(4, self.num_kv_heads)
        for c in range(c0, c1):
            lo, hi = max(t0, c * CHUNK), min(t1, (c + 1) * CHUNK)
            r = _rng(self.seed, self.layer_id, 5, b, c)
            k = r.standard_normal((CHUNK, self.num_kv_heads, HEAD_DIM), dtype=np.float32)
            v = r.standard_normal((CHUNK, self.num_kv_heads, HEAD_DIM), dtype=np.float32)
            sl = slice(lo - c * CHUNK, hi - c * CHUNK)
            k, v = k[sl] * np.float32(self.kv_std), v[sl] * np.float32(self.kv_std)
            if mk is not None:
                k, v = k * mk[None], v * mv[None]
            ks.append(k)
            vs.append(v)
        if not ks:
            z = np.zeros((0, self.num_kv_heads, HEAD_DIM), np.float32)
            return f32_to_bf16_bits(z), f32_to_bf16_bits(z)
        return f32_to_bf16_bits(np.concatenate(ks)), f32_to_bf16_bits(np.concatenate(vs))

    def slots(self, b, t0, t1):
        """int32 slot mapping for tokens [t0, t1) of sequence b through its page table."""
        j = np.arange(t0, t1, dtype=np.int64)
        return (self.block_table[b, j // self.block_size].astype(np.int64) * self.block_size
                + j % self.block_size).astype(np.int32)


def _table_from_perm(perm, seq_lens, block_size):
    nb = [(int(L) + block_size - 1) // block_size for L in seq_lens]
    width = max(1, max(nb) if nb else 1)
    table = np.zeros((len(seq_lens), width), dtype=np.int32)
    off = 0
    for b, n in enumerate(nb):
        table[b, :n] = perm[off:off + n]
        off += n
    return table


def make_layer(name, seed, layer_id, num_q_heads, num_kv_heads, block_size, q_len, window_left, seq_lens,
               scale_range=(0.01, 0.1), fixed_scale=None, kv_std=1.0, outlier_rate=0.0, pool_slack=2.0,
               cache_dtype="fp8_e4m3fn"):
    """A layer whose sequences get blocks from one random permutation of a pool.

    pool_slack > 1 leaves unused physical blocks so the table is non-contiguous
    and does not cover the pool.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    need = int(sum((int(L) + block_size - 1) // block_size for L in seq_lens))
    num_blocks = max(1, int(math.ceil(need * pool_slack)))
    r = _rng(seed, layer_id, 0)
    perm = r.permutation(num_blocks)[:need].astype(np.int32)
    table = _table_from_perm(perm, seq_lens, block_size)
    if fixed_scale is not None:
        ks = vs = np.float32(fixed_scale)
    else:
        ks, vs = r.uniform(scale_range[0], scale_range[1], size=2).astype(np.float32)
    return Layer(name=name, seed=seed, layer_id=layer_id, num_seqs=len(seq_lens), num_q_heads=num_q_heads,
                 num_kv_heads=num_kv_heads, block_size=block_size, q_len=q_len, window_left=window_left,
                 seq_lens=seq_lens, block_table=table, num_blocks=num_blocks, k_scale=np.float32(ks),
                 v_scale=np.float32(vs), kv_std=kv_std, outlier_rate=outlier_rate, cache_dtype=cache_dtype)


# ---- the five workloads -------------------------------------------------------------------

def c1_layer():
    """1 seq, 18 Q / 2 KV heads, context 256, page 32, M=1, global; N(0,1); scales U(0.01, 0.1)."""
    return make_layer("c1_q1_256_p32", 1001, 0, 18, 2, 32, 1, -1, [256], pool_slack=1.0)


def c2_layer():
    """1 seq, 18/2, page 64, context 2048, 512-token sliding window, M=12, 1% x8 outlier channels."""
    return make_layer("c2_m12_2048_sw512_p64", 1002, 0, 18, 2, 64, 12, 511, [2048], outlier_rate=0.01)


def c3_layer(context=8192, block_size=64, layer_id=0):
    """Full layer: 72 Q / 8 KV heads, global, M=12, contexts 8k or 32k, page 32 or 64."""
    return make_layer(f"c3_m12_{context}_p{block_size}", 1003, layer_id, 72, 8, block_size, 12, -1, [context])


C4_LAYERS = 48
C4_DRAFT_LAYERS = 6


def c4_is_global(layer_id):
    """36 sliding-window + 12 global target layers: every fourth layer (3, 7, ..., 47) is global.

    The pages give only the counts; the interleave is this module's reading.
    """
    return layer_id % 4 == 3


def c4_layer(layer_id):
    """Layer of the 48-layer (+6 draft) cycle at context 8192, 18/2, page 64, M=12.

    Target layers 0..47: their own U(0.01, 0.1) scales; window 512 unless global.
    Draft layers 48..53: scale 1.0, K/V ~ N(0, 0.5^2), global.
    """
    if layer_id < C4_LAYERS:
        wl = -1 if c4_is_global(layer_id) else 511
        return make_layer(f"c4_layer{layer_id}", 1004, layer_id, 18, 2, 64, 12, wl, [8192])
    return make_layer(f"c4_draft{layer_id - C4_LAYERS}", 1004, layer_id, 18, 2, 64, 12, -1, [8192],
                      fixed_scale=1.0, kv_std=0.5)


def c5_seq_lens(num_seqs=32, lo=1024, hi=131072, seed=1005):
    """Per-sequence contexts, log-uniform in [lo, hi], rounded to the nearest integer."""
    r = _rng(seed, 99)
    return np.rint(np.exp(r.uniform(math.log(lo), math.log(hi), size=num_seqs))).astype(np.int32)


def c5_layer(q_len=12, cache_dtype="fp8_e4m3fn", num_seqs=32):
    """32 sequences, 72/8, global, page 32, one shared pool with interleaved blocks."""
    return make_layer(f"c5_m{q_len}_{cache_dtype}", 1005, 0, 72, 8, 32, q_len, -1, c5_seq_lens(num_seqs),
                      pool_slack=1.0, cache_dtype=cache_dtype)


def tiny_layer(seed, seq_lens, num_q_heads=18, num_kv_heads=2, block_size=32, q_len=1, window_left=-1,
               cache_dtype="fp8_e4m3fn", pool_slack=1.5, outlier_rate=0.0, fixed_scale=None):
    return make_layer(f"tiny{seed}", seed, 0, num_q_heads, num_kv_heads, block_size, q_len, window_left, seq_lens,
                      cache_dtype=cache_dtype, pool_slack=pool_slack, outlier_rate=outlier_rate,
                      fixed_scale=fixed_scale)


# ---- inputs of the Q/K RMSNorm + RoPE + insert step -------------------------------------

ROPE_BASE = 1.0e6  # rotary base of the synthetic table (the method takes the table as given)


def rope_table(num_positions, base=ROPE_BASE):
    """float32 [P, 128]: row p holds cos(p * f_i) for i < 64, then sin(p * f_i), with
    f_i = base^(-i / 64); computed in float64, then rounded to float32."""
    p = np.arange(num_positions, dtype=np.float64)[:, None]
    f = base ** (-np.arange(HEAD_DIM // 2, dtype=np.float64) / (HEAD_DIM // 2))
    ang = p * f[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


@dataclass
class NormRopeStep:
    """T new tokens before the norm/RoPE/insert step: raw BF16 Q, K, V, the norm weights,
    positions and slots (into a layer's pool) and the scales."""
    q_bits: np.ndarray          # uint16 [T, Hq, 128]
    k_bits: np.ndarray          # uint16 [T, Hkv, 128]
    v_bits: np.ndarray          # uint16 [T, Hkv, 128]
    q_w: np.ndarray             # uint16 [128]
    k_w: np.ndarray             # uint16 [128]
    eps: float
    cos_sin: np.ndarray         # float32 [P, 128]
    positions: np.ndarray       # int32 [T]
    slot_mapping: np.ndarray    # int32 [T]


def norm_rope_step(lay, seed=77, eps=1e-6, table_rows=None):
    """The M new tokens of every sequence of `lay` (positions L - M .. L - 1, slots through
    its block table) with raw Q/K/V ~ N(0, 1) (K, V with the layer's outlier channels, Q
    scaled by 4 so the norm does real work) and norm weights ~ U(0.5, 1.5), BF16."""
    r = _rng(seed, lay.seed, lay.layer_id)
    M, B = lay.q_len, lay.num_seqs
    T = M * B
    q = r.standard_normal((T, lay.num_q_heads, HEAD_DIM), dtype=np.float32) * np.float32(4.0)
    ks, vs, pos, slots = [], [], [], []
    for b in range(B):
        L = int(lay.seq_lens[b])
        t0 = L - M
        kb, vb = lay.kv_bits(b, max(t0, 0), L)
        pad = max(0, -t0)
        if pad:  # rows before position 0: padding tokens (any values, never inserted)
            kb = np.concatenate([np.zeros((pad,) + kb.shape[1:], np.uint16), kb])
            vb = np.concatenate([np.zeros((pad,) + vb.shape[1:], np.uint16), vb])
        ks.append(kb)
        vs.append(vb)
        p = np.arange(t0, L)
        pos.append(p)
        sl = np.full(M, -1, dtype=np.int64)
        ok = p >= 0
        sl[ok] = lay.slots(b, max(t0, 0), L)
        slots.append(sl)
    positions = np.concatenate(pos).astype(np.int32)
    P = table_rows if table_rows is not None else int(max(1, positions.max() + 1))
    w = r.uniform(0.5, 1.5, size=(2, HEAD_DIM)).astype(np.float32)
    return NormRopeStep(q_bits=f32_to_bf16_bits(q), k_bits=np.concatenate(ks), v_bits=np.concatenate(vs),
                        q_w=f32_to_bf16_bits(w[0]), k_w=f32_to_bf16_bits(w[1]), eps=float(eps),
                        cos_sin=rope_table(P), positions=positions,
                        slot_mapping=np.concatenate(slots).astype(np.int32))
