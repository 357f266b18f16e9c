"""Python binding of libfkv.so: the C entry points of include/fkv.h, marshalled with ctypes.

Names follow the C ABI without its `fkv_` prefix (cache_bytes, init_cache, insert,
decode_workspace_bytes, decode_attn, decode_attn_noalloc, insert_decode, qk_norm_rope_insert,
norm_rope_insert_decode, status_string, get_counters, reset_counters).
Every step of the path runs in the HIP library; this module only checks tensor
placement and passes pointers, sizes and the current HIP stream. There is no
fallback: if the library is missing, loading raises.
"""

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfkv.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, 1, 2, 3, 4
FP8_E4M3FN, BF16 = 1, 2
OUT_F32 = 1
OUT_BF16 = 2
HEAD_DIM = 128
CACHE_DTYPES = {"fp8_e4m3fn": FP8_E4M3FN, "bf16": BF16}


class FkvError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("cache_dtype", ctypes.c_int32)]


class Cache(ctypes.Structure):
    _fields_ = [("desc", CacheDesc), ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("pool_bytes", ctypes.c_uint64)]


class DecodeDesc(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("q_len", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("window_left", ctypes.c_int32), ("softmax_scale", ctypes.c_float), ("out_dtype", ctypes.c_int32),
                ("split_tiles", ctypes.c_int32), ("layout", ctypes.c_int32), ("row_groups", ctypes.c_int32),
                ("row_exact", ctypes.c_int32)]


class Counters(ctypes.Structure):
    _fields_ = [("insert_launches", ctypes.c_uint64 * 2), ("decode_launches", ctypes.c_uint64 * 2),
                ("decode_row_tiles", (ctypes.c_uint64 * 7) * 2), ("decode_long_windows", ctypes.c_uint64 * 2),
                ("decode_combine_launches", ctypes.c_uint64), ("rejected_calls", ctypes.c_uint64),
                ("insert_decode_launches", ctypes.c_uint64), ("norm_rope_insert_launches", ctypes.c_uint64 * 2),
                ("norm_rope_insert_decode_launches", ctypes.c_uint64)]


_lib = None


def lib():
    """Load libfkv.so from the package directory (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(f"{LIB_PATH} is missing: build it with fp8_kv_paged_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.fkv_cache_bytes.argtypes = [ctypes.POINTER(CacheDesc), ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.fkv_init_cache.argtypes = [ctypes.POINTER(CacheDesc), vp, vp, ctypes.POINTER(Cache)]
        L.fkv_insert.argtypes = [ctypes.POINTER(Cache), vp, vp, vp, i32, vp, vp, vp]
        L.fkv_decode_workspace_bytes.argtypes = [ctypes.POINTER(Cache), ctypes.POINTER(DecodeDesc), ctypes.POINTER(sz)]
        L.fkv_decode_attn.argtypes = [ctypes.POINTER(Cache), ctypes.POINTER(DecodeDesc), vp, vp, vp, vp, vp, vp, vp,
                                      sz, vp]
        L.fkv_decode_attn_noalloc.argtypes = [ctypes.POINTER(Cache), ctypes.POINTER(DecodeDesc), vp, vp, vp, vp, vp,
                                              vp, vp]
        L.fkv_insert_decode.argtypes = [ctypes.POINTER(Cache), ctypes.POINTER(DecodeDesc), vp, vp, vp, vp, vp, vp, vp,
                                        vp, vp, sz, vp]
        L.fkv_qk_norm_rope_insert.argtypes = [ctypes.POINTER(Cache), i32, i32, vp, vp, vp, vp, vp, ctypes.c_float, vp,
                                              i32, vp, vp, vp, vp, vp, vp]
        L.fkv_norm_rope_insert_decode.argtypes = [ctypes.POINTER(Cache), ctypes.POINTER(DecodeDesc), vp, vp, vp, vp, vp,
                                                  ctypes.c_float, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.fkv_status_string.argtypes = [ctypes.c_int]
        L.fkv_status_string.restype = ctypes.c_char_p
        L.fkv_get_counters.argtypes = [ctypes.POINTER(Counters)]
        L.fkv_reset_counters.argtypes = []
        for f in ("fkv_cache_bytes", "fkv_init_cache", "fkv_insert", "fkv_decode_workspace_bytes", "fkv_decode_attn",
                  "fkv_decode_attn_noalloc", "fkv_insert_decode", "fkv_qk_norm_rope_insert", "fkv_norm_rope_insert_decode", "fkv_get_counters", "fkv_reset_counters"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status):
    return lib().fkv_status_string(int(status)).decode()


def _check(rc, what):
    if rc != OK:
        raise FkvError(rc, what)


def _ptr(t, what, elem_size=None):
    """Device pointer of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if elem_size is not None and t.element_size() != elem_size:
        raise ValueError(f"{what} must have {elem_size}-byte elements, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_cache_desc(num_blocks, block_size, num_kv_heads, cache_dtype="fp8_e4m3fn", head_dim=HEAD_DIM):
    dt = CACHE_DTYPES.get(cache_dtype, cache_dtype)
    return CacheDesc(int(num_blocks), int(block_size), int(num_kv_heads), int(head_dim), int(dt))


def cache_bytes(desc):
    k, v = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().fkv_cache_bytes(ctypes.byref(desc), ctypes.byref(k), ctypes.byref(v)), "fkv_cache_bytes")
    return k.value, v.value


def init_cache(desc, k_pool, v_pool):
    """Cache handle over two caller-owned GPU pools of cache_bytes(desc) bytes each."""
    nbytes = cache_bytes(desc)[0]
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool)):
        if t.numel() * t.element_size() != nbytes:
            raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, expected {nbytes}")
    out = Cache()
    _check(lib().fkv_init_cache(ctypes.byref(desc), _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool"), ctypes.byref(out)),
           "fkv_init_cache")
    out._keep = (k_pool, v_pool)  # the pools must outlive the handle
    return out


def insert(cache, k, v, slot_mapping, k_scale, v_scale, stream=None):
    """k, v: BF16 [T, Hkv, 128]; slot_mapping int32 [T]; scales: 1-element fp32 GPU tensors."""
    T = int(slot_mapping.numel())
    for name, t in (("k", k), ("v", v)):
        if t.numel() != T * cache.desc.num_kv_heads * HEAD_DIM:
            raise ValueError(f"{name} has {t.numel()} elements, expected {T} x {cache.desc.num_kv_heads} x 128")
    _check(lib().fkv_insert(ctypes.byref(cache), _ptr(k, "k", 2), _ptr(v, "v", 2), _ptr(slot_mapping, "slot_mapping", 4),
                            T, _ptr(k_scale, "k_scale", 4), _ptr(v_scale, "v_scale", 4), _stream(stream)),
           "fkv_insert")


def make_decode_desc(num_seqs, q_len, num_q_heads, max_blocks_per_seq, max_seq_len, window_left=-1,
                     softmax_scale=1.0 / math.sqrt(HEAD_DIM), split_tiles=0, layout=0, row_groups=0, row_exact=0,
                     out_dtype=OUT_F32):
    return DecodeDesc(int(num_seqs), int(q_len), int(num_q_heads), int(max_blocks_per_seq), int(max_seq_len),
                      int(window_left), float(softmax_scale), int(out_dtype), int(split_tiles), int(layout),
                      int(row_groups), int(row_exact))


def _out_size(desc):
    return 2 if desc.out_dtype == OUT_BF16 else 4


def decode_workspace_bytes(cache, desc):
    n = ctypes.c_size_t()
    _check(lib().fkv_decode_workspace_bytes(ctypes.byref(cache), ctypes.byref(desc), ctypes.byref(n)),
           "fkv_decode_workspace_bytes")
    return n.value


def decode_attn(cache, desc, q, block_table, seq_lens, k_scale, v_scale, out, workspace=None, stream=None):
    """q BF16 [B, M, Hq, 128]; block_table int32 [B, max_blocks]; seq_lens int32 [B]; out fp32 [B, M, Hq, 128]
    (BF16 when desc.out_dtype is OUT_BF16)."""
    B, M, Hq = desc.num_seqs, desc.q_len, desc.num_q_heads
    if q.numel() != B * M * Hq * HEAD_DIM or out.numel() != B * M * Hq * HEAD_DIM:
        raise ValueError("q / out do not match the decode descriptor")
    if block_table.numel() != B * desc.max_blocks_per_seq or seq_lens.numel() != B:
        raise ValueError("block_table / seq_lens do not match the decode descriptor")
    ws = _ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().fkv_decode_attn(ctypes.byref(cache), ctypes.byref(desc), _ptr(q, "q", 2),
                                 _ptr(block_table, "block_table", 4), _ptr(seq_lens, "seq_lens", 4),
                                 _ptr(k_scale, "k_scale", 4), _ptr(v_scale, "v_scale", 4), _ptr(out, "out", _out_size(desc)), ws,
                                 ws_bytes, _stream(stream)),
           "fkv_decode_attn")


def decode_attn_noalloc(cache, desc, q, block_table, seq_lens, k_scale, v_scale, out, stream=None):
    """fkv_decode_attn_noalloc: decode_attn with the library's static scratch instead of a
    workspace (nothing is allocated)."""
    B, M, Hq = desc.num_seqs, desc.q_len, desc.num_q_heads
    if q.numel() != B * M * Hq * HEAD_DIM or out.numel() != B * M * Hq * HEAD_DIM:
        raise ValueError("q / out do not match the decode descriptor")
    if block_table.numel() != B * desc.max_blocks_per_seq or seq_lens.numel() != B:
        raise ValueError("block_table / seq_lens do not match the decode descriptor")
    _check(lib().fkv_decode_attn_noalloc(ctypes.byref(cache), ctypes.byref(desc), _ptr(q, "q", 2),
                                         _ptr(block_table, "block_table", 4), _ptr(seq_lens, "seq_lens", 4),
                                         _ptr(k_scale, "k_scale", 4), _ptr(v_scale, "v_scale", 4),
                                         _ptr(out, "out", _out_size(desc)), _stream(stream)),
           "fkv_decode_attn_noalloc")


def insert_decode(cache, desc, q, k_new, v_new, block_table, seq_lens, k_scale, v_scale, out, workspace=None,
                  stream=None):
    """fkv_insert_decode: k_new / v_new BF16 [B, M, Hkv, 128] (the M new tokens of each sequence, at
    positions L-M .. L-1); the other arguments as decode_attn."""
    B, M, Hq = desc.num_seqs, desc.q_len, desc.num_q_heads
    if q.numel() != B * M * Hq * HEAD_DIM or out.numel() != B * M * Hq * HEAD_DIM:
        raise ValueError("q / out do not match the decode descriptor")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t.numel() != B * M * cache.desc.num_kv_heads * HEAD_DIM:
            raise ValueError(f"{name} must hold num_seqs x q_len x num_kv_heads x 128 elements")
    if block_table.numel() != B * desc.max_blocks_per_seq or seq_lens.numel() != B:
        raise ValueError("block_table / seq_lens do not match the decode descriptor")
    ws = _ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().fkv_insert_decode(ctypes.byref(cache), ctypes.byref(desc), _ptr(q, "q", 2), _ptr(k_new, "k_new", 2),
                                   _ptr(v_new, "v_new", 2), _ptr(block_table, "block_table", 4),
                                   _ptr(seq_lens, "seq_lens", 4), _ptr(k_scale, "k_scale", 4),
                                   _ptr(v_scale, "v_scale", 4), _ptr(out, "out", _out_size(desc)), ws, ws_bytes, _stream(stream)),
           "fkv_insert_decode")


def qk_norm_rope_insert(cache, q, k, v, q_weight, k_weight, eps, cos_sin, positions, slot_mapping, k_scale, v_scale,
                        q_out, stream=None):
    """fkv_qk_norm_rope_insert: q BF16 [T, Hq, 128], k / v BF16 [T, Hkv, 128], weights BF16 [128],
    cos_sin fp32 [P, 128], positions / slot_mapping int32 [T], q_out BF16 like q (may be q)."""
    T = int(positions.numel())
    Hkv = cache.desc.num_kv_heads
    if q.dim() != 3 or q.shape[0] != T or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [num_tokens, num_q_heads, 128]")
    Hq = int(q.shape[1])
    for name, t, n in (("k", k, T * Hkv * HEAD_DIM), ("v", v, T * Hkv * HEAD_DIM), ("q_out", q_out, q.numel()),
                       ("q_weight", q_weight, HEAD_DIM), ("k_weight", k_weight, HEAD_DIM),
                       ("slot_mapping", slot_mapping, T)):
        if t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements, expected {n}")
    if cos_sin.dim() != 2 or cos_sin.shape[1] != HEAD_DIM:
        raise ValueError("cos_sin must be [rope_rows, 128]")
    _check(lib().fkv_qk_norm_rope_insert(ctypes.byref(cache), T, Hq, _ptr(q, "q", 2), _ptr(k, "k", 2),
                                         _ptr(v, "v", 2), _ptr(q_weight, "q_weight", 2),
                                         _ptr(k_weight, "k_weight", 2), float(eps), _ptr(cos_sin, "cos_sin", 4),
                                         int(cos_sin.shape[0]), _ptr(positions, "positions", 4),
                                         _ptr(slot_mapping, "slot_mapping", 4), _ptr(k_scale, "k_scale", 4),
                                         _ptr(v_scale, "v_scale", 4), _ptr(q_out, "q_out", 2), _stream(stream)),
           "fkv_qk_norm_rope_insert")


def norm_rope_insert_decode(cache, desc, q, k_new, v_new, q_weight, k_weight, eps, cos_sin, block_table, seq_lens,
                            k_scale, v_scale, out, workspace=None, stream=None):
    """fkv_norm_rope_insert_decode: insert_decode with raw q / k_new normalised and rotated in the
    kernel; weights BF16 [128], cos_sin fp32 [P, 128] with P >= desc.max_seq_len."""
    B, M, Hq = desc.num_seqs, desc.q_len, desc.num_q_heads
    if q.numel() != B * M * Hq * HEAD_DIM or out.numel() != B * M * Hq * HEAD_DIM:
        raise ValueError("q / out do not match the decode descriptor")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t.numel() != B * M * cache.desc.num_kv_heads * HEAD_DIM:
            raise ValueError(f"{name} must hold num_seqs x q_len x num_kv_heads x 128 elements")
    for name, t in (("q_weight", q_weight), ("k_weight", k_weight)):
        if t.numel() != HEAD_DIM:
            raise ValueError(f"{name} must hold 128 elements")
    if cos_sin.dim() != 2 or cos_sin.shape[1] != HEAD_DIM:
        raise ValueError("cos_sin must be [rope_rows, 128]")
    if block_table.numel() != B * desc.max_blocks_per_seq or seq_lens.numel() != B:
        raise ValueError("block_table / seq_lens do not match the decode descriptor")
    ws = _ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().fkv_norm_rope_insert_decode(ctypes.byref(cache), ctypes.byref(desc), _ptr(q, "q", 2),
                                             _ptr(k_new, "k_new", 2), _ptr(v_new, "v_new", 2),
                                             _ptr(q_weight, "q_weight", 2), _ptr(k_weight, "k_weight", 2),
                                             float(eps), _ptr(cos_sin, "cos_sin", 4), int(cos_sin.shape[0]),
                                             _ptr(block_table, "block_table", 4), _ptr(seq_lens, "seq_lens", 4),
                                             _ptr(k_scale, "k_scale", 4), _ptr(v_scale, "v_scale", 4),
                                             _ptr(out, "out", _out_size(desc)), ws, ws_bytes, _stream(stream)),
           "fkv_norm_rope_insert_decode")


def get_counters():
    c = Counters()
    _check(lib().fkv_get_counters(ctypes.byref(c)), "fkv_get_counters")
    return {"insert_launches": list(c.insert_launches),
            "decode_launches": list(c.decode_launches),
            "decode_row_tiles": [list(r) for r in c.decode_row_tiles],
            "decode_long_windows": list(c.decode_long_windows),
            "decode_combine_launches": c.decode_combine_launches,
            "insert_decode_launches": c.insert_decode_launches,
            "norm_rope_insert_launches": list(c.norm_rope_insert_launches),
            "norm_rope_insert_decode_launches": c.norm_rope_insert_decode_launches,
            "rejected_calls": c.rejected_calls}


def reset_counters():
    _check(lib().fkv_reset_counters(), "fkv_reset_counters")
