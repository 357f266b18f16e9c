"""GPU state of one attention layer driven through the C ABI.

PagedLayer owns the device buffers of one layer: the two pools, the page table,
sequence lengths, the scalar scales (kept at fixed device addresses so calls
never synchronise) and the decode output / workspace. It uploads synthetic
inputs from `synth.Layer` and issues insert / decode calls; all arithmetic
happens in libfkv.so.
"""

import numpy as np
import torch

from . import fkv
from .synth import HEAD_DIM

POISON_BYTE = {"fp8_e4m3fn": 0x7F, "bf16": 0xFF}  # E4M3 NaN / BF16 NaN bit patterns


def to_dev_bits(bits, device):
    """uint16 BF16 bit patterns (numpy) -> a bfloat16 GPU tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


class PagedLayer:
    def __init__(self, lay, device="cuda", poison=True, split_tiles=0, layout=0, row_groups=0, row_exact=0,
                 out_bf16=False):
        self.lay = lay
        self.device = device
        self.desc = fkv.make_cache_desc(lay.num_blocks, lay.block_size, lay.num_kv_heads, lay.cache_dtype)
        nbytes, _ = fkv.cache_bytes(self.desc)
        fill = POISON_BYTE[lay.cache_dtype] if poison else 0
        self.k_pool = torch.full((nbytes,), fill, dtype=torch.uint8, device=device)
        self.v_pool = torch.full((nbytes,), fill, dtype=torch.uint8, device=device)
        self.cache = fkv.init_cache(self.desc, self.k_pool, self.v_pool)
        self.k_scale = torch.tensor([float(lay.k_scale)], dtype=torch.float32, device=device)
        self.v_scale = torch.tensor([float(lay.v_scale)], dtype=torch.float32, device=device)
        self.block_table = torch.from_numpy(np.ascontiguousarray(lay.block_table)).to(device)
        self.seq_lens = torch.from_numpy(np.ascontiguousarray(lay.seq_lens)).to(device)
        self.max_seq_len = int(max(1, lay.seq_lens.max())) if lay.num_seqs else 1
        self.ddesc = fkv.make_decode_desc(lay.num_seqs, lay.q_len, lay.num_q_heads, lay.max_blocks, self.max_seq_len,
                                          lay.window_left, lay.softmax_scale, split_tiles, layout, row_groups,
                                          row_exact, fkv.OUT_BF16 if out_bf16 else fkv.OUT_F32)
        self.q = to_dev_bits(lay.q_bits(), device)
        self.out = torch.empty((lay.num_seqs, lay.q_len, lay.num_q_heads, HEAD_DIM),
                               dtype=torch.bfloat16 if out_bf16 else torch.float32, device=device)
        nws = fkv.decode_workspace_bytes(self.cache, self.ddesc)
        # zero once: the split-merge counters at its end must start at zero (calls leave them so)
        self.workspace = torch.zeros((max(nws, 16),), dtype=torch.uint8, device=device)
        self.step_k = self.step_v = self.step_slots = None
        self.new_k = self.new_v = None

    def set_split_tiles(self, split_tiles):
        self.ddesc.split_tiles = int(split_tiles)
        nws = fkv.decode_workspace_bytes(self.cache, self.ddesc)
        if nws > self.workspace.numel():
            self.workspace = torch.zeros((nws,), dtype=torch.uint8, device=self.device)

    def insert_tokens(self, b, t0, t1, chunk=32768):
        """Insert tokens [t0, t1) of sequence b (host-generated BF16) through the slot mapping."""
        for c0 in range(t0, t1, chunk):
            c1 = min(t1, c0 + chunk)
            k, v = self.lay.kv_bits(b, c0, c1)
            slots = torch.from_numpy(self.lay.slots(b, c0, c1)).to(self.device)
            fkv.insert(self.cache, to_dev_bits(k, self.device), to_dev_bits(v, self.device), slots,
                       self.k_scale, self.v_scale)

    def prefill(self):
        """Everything before the q_len new tokens of each sequence."""
        for b in range(self.lay.num_seqs):
            L = int(self.lay.seq_lens[b])
            self.insert_tokens(b, 0, max(0, L - self.lay.q_len))

    def stage_step(self):
        """Upload the q_len new tokens of every sequence (one insert call inserts them all)."""
        ks, vs, ss = [], [], []
        for b in range(self.lay.num_seqs):
            L = int(self.lay.seq_lens[b])
            t0 = max(0, L - self.lay.q_len)
            k, v = self.lay.kv_bits(b, t0, L)
            ks.append(k)
            vs.append(v)
            ss.append(self.lay.slots(b, t0, L))
        self.step_k = to_dev_bits(np.concatenate(ks), self.device)
        self.step_v = to_dev_bits(np.concatenate(vs), self.device)
        self.step_slots = torch.from_numpy(np.concatenate(ss).astype(np.int32)).to(self.device)

    def stage_new_tokens(self):
        """The q_len new tokens of every sequence as [num_seqs, q_len, Hkv, 128] BF16 (the layout of
        insert_decode); positions below 0 (seq_len < q_len) are zero rows, which are not stored."""
        M, H = self.lay.q_len, self.lay.num_kv_heads
        k = np.zeros((self.lay.num_seqs, M, H, HEAD_DIM), dtype=np.uint16)
        v = np.zeros_like(k)
        for b in range(self.lay.num_seqs):
            L = int(self.lay.seq_lens[b])
            t0 = max(0, L - M)
            kb, vb = self.lay.kv_bits(b, t0, L)
            k[b, M - (L - t0):] = kb.reshape(L - t0, H, HEAD_DIM)
            v[b, M - (L - t0):] = vb.reshape(L - t0, H, HEAD_DIM)
        self.new_k = to_dev_bits(k, self.device)
        self.new_v = to_dev_bits(v, self.device)

    def insert_decode(self, stream=None):
        """One launch: insert the staged new tokens and decode."""
        fkv.insert_decode(self.cache, self.ddesc, self.q, self.new_k, self.new_v, self.block_table, self.seq_lens,
                          self.k_scale, self.v_scale, self.out, self.workspace, stream)
        return self.out

    def stage_norm_rope(self, st):
        """Upload a synth.NormRopeStep (raw Q/K/V of the new tokens, weights, table, positions,
        slots); q_rot receives the normalised, rotated Q."""
        d = self.device
        self.nr = {"q": to_dev_bits(st.q_bits, d), "k": to_dev_bits(st.k_bits, d), "v": to_dev_bits(st.v_bits, d),
                   "q_w": to_dev_bits(st.q_w, d), "k_w": to_dev_bits(st.k_w, d), "eps": st.eps,
                   "cos_sin": torch.from_numpy(st.cos_sin).to(d), "positions": torch.from_numpy(st.positions).to(d),
                   "slots": torch.from_numpy(st.slot_mapping).to(d)}
        self.q_rot = torch.empty_like(self.nr["q"])

    def norm_rope_insert(self, stream=None):
        n = self.nr
        fkv.qk_norm_rope_insert(self.cache, n["q"], n["k"], n["v"], n["q_w"], n["k_w"], n["eps"], n["cos_sin"],
                                n["positions"], n["slots"], self.k_scale, self.v_scale, self.q_rot, stream)
        return self.q_rot

    def insert_step(self, stream=None):
        fkv.insert(self.cache, self.step_k, self.step_v, self.step_slots, self.k_scale, self.v_scale, stream)

    def decode(self, stream=None):
        fkv.decode_attn(self.cache, self.ddesc, self.q, self.block_table, self.seq_lens, self.k_scale, self.v_scale,
                        self.out, self.workspace, stream)
        return self.out

    def build(self):
        """Prefill, insert the new tokens, ready to decode."""
        self.prefill()
        self.stage_step()
        self.insert_step()
        return self
