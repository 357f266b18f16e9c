// Host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fkv.h"

namespace fkv {

constexpr int kMaxSplits = 512;  // split-KV partials per (sequence, KV head) the combine can merge
constexpr int kMaxDmaSplitTiles = 128;  // 32-key tiles per split of the LDS-pipelined kernels
constexpr int kFastMergeSplits = 16;    // 32-row kernel: splits one thread merges with all loads in flight

struct InsertArgs {
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* slots;
  const float* k_scale;
  const float* v_scale;
  void* k_pool;
  void* v_pool;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t block_size;
  int64_t num_slots;  // num_blocks * block_size
};

// Plan of one decode call: split-KV tiling and workspace carve-up.
struct DecodePlan {
  int nt;              // 16-row query tiles per KV head: ceil(G*M/16)
  int layout;          // work-group layout (see split_shape)
  int rows_pad;        // rows of one split partial: 16 * nt, or every row group's rows
  int row_groups;      // work groups per (sequence, KV head, split) of the row-group kernel
  int tiles_per_split; // 32-key tiles handled by one work group
  int max_splits;      // grid x
  size_t ws_o_bytes;   // fp32 partial outputs
  size_t ws_ml_bytes;  // fp32 (m, l) per partial row
  size_t ws_ctl_bytes; // in-kernel split merge: 256 bytes of counters and claim bits per pair
  size_t ws_ctl_offset; // where those counters start (after every partial region the layout
                        // choice of the descriptor may use)
  int fused_combine;   // layout 5 with the whole grid resident: splits merged inside the kernel
  int key_lanes;       // 32-row kernel: key lanes per work group
  int align_splits;    // 32-row kernel, row-exact mode: split boundaries at absolute tile indices
  int clip_rows;       // 32-row kernel, long query windows: per-work-group key ranges
  int xcd_pairs;       // row-group kernel: each (sequence, KV head) pair's work groups on one XCD
  size_t ws_bytes;     // total, 256-byte aligned pieces
};

struct DecodeArgs {
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const uint16_t* q;
  const uint16_t* k_new;  // fused insert (32-row kernel): BF16 [num_seqs][q_len][num_kv_heads][128], or null
  const uint16_t* v_new;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const float* k_scale;
  const float* v_scale;
  float* out;
  float* ws_o;
  float* ws_ml;
  uint32_t* ws_ctl;      // 64 words per (sequence, KV head): merge counters and claim bits
  int32_t num_seqs, num_q_heads, num_kv_heads, group, q_len, block_size, max_blocks, num_blocks;
  int32_t window_left, tiles_per_split, max_splits, max_seq_len, rows_pad;
  int32_t row_groups;  // work groups per (sequence, KV head, split) sharing its query rows
  int32_t xcd_pairs;   // each (sequence, KV head) pair's work groups on one XCD
  int32_t fused_combine;  // 32-row kernel: merge the splits inside the kernel (no combine launch)
  int32_t key_lanes;      // 32-row kernel: key lanes per work group
  int32_t align_splits;   // 32-row kernel: splits start at multiples of tiles_per_split (row-exact mode)
  int32_t clip_rows;      // 32-row kernel, long query windows: each work group skips the tiles its rows cannot see
  int32_t out_bf16;       // out holds BF16 (rounded to nearest even), else fp32
  // fused insert with the Q/K RMSNorm + RoPE in front (cos_sin non-null): q and k_new are raw
  const uint16_t* q_w;    // BF16 [128]
  const uint16_t* k_w;    // BF16 [128]
  const float* cos_sin;   // fp32 [rope_rows][128], rope_rows >= max_seq_len
  float eps;
  float softmax_scale;
};

hipError_t launch_insert(const InsertArgs& a, bool fp8, hipStream_t stream);

struct NormRopeArgs {
  const uint16_t* q;        // BF16 [T][Hq][128]
  const uint16_t* k;        // BF16 [T][Hkv][128]
  const uint16_t* v;        // BF16 [T][Hkv][128]
  const uint16_t* q_w;      // BF16 [128]
  const uint16_t* k_w;      // BF16 [128]
  const float* cos_sin;     // fp32 [rope_rows][128]: 64 cosines, then 64 sines
  const int32_t* positions; // [T]
  const int32_t* slots;     // [T]
  const float* k_scale;
  const float* v_scale;
  uint16_t* q_out;          // BF16 [T][Hq][128] (may be q itself)
  void* k_pool;
  void* v_pool;
  int32_t num_tokens, num_q_heads, num_kv_heads, block_size, rope_rows;
  int64_t num_slots;
  float eps;
};
hipError_t launch_norm_rope_insert(const NormRopeArgs& a, bool fp8, hipStream_t stream);
// Work-group shape of a decode kernel: r row groups of ntw row tiles each, k key lanes per
// group, and groups_per_cu marking the kernel: 0 = the row-group kernel (layout 3; 16-row
// tiles, ntw of them per group), -2 = the 32-row kernel (layout 5; ntw = r row tiles of 32,
// k = 8 / r key lanes), -3 = the 32-row kernel with two row tiles per wave (layout 6, k = 4).
struct SplitShapeInfo {
  int ntw, r, k, groups_per_cu;
};

inline SplitShapeInfo split_shape(int nt, int layout, bool fp8 = true) {
  if (layout == 5 || layout == 6 || (layout == 0 && fp8)) {  // layout 0 (automatic) is layout 5 for FP8 caches
    const int rows = 16 * nt;
    const int rt = rows <= 32 ? 1 : (rows <= 64 ? 2 : 4);
    if (layout == 6) return {rt, rt, 4, -3};
    return {rt, rt, 8 / rt, -2};
  }
  // layout 3, and layout 0 (automatic) for BF16 caches
  const int ntw = nt >= 2 ? 2 : 1;
  return {ntw, (nt + ntw - 1) / ntw, fp8 ? 8 : 4, 0};
}

// Row-group split kernel (layout 3): ntw 16-row tiles per row group.
hipError_t launch_rows(const DecodeArgs& a, int ntw, bool fp8, hipStream_t stream);
// 32-row tile kernel: rt row tiles of 32 per work group (1, 2 or 4) and rw per wave (layout 5:
// 1; layout 6: 2 with rt = 2), FP8 cache only.
hipError_t launch_m32(const DecodeArgs& a, int rt, int rw, int kl, bool fp8, hipStream_t stream);
// Merges split partials (rows_pad rows per partial) into out.
hipError_t launch_combine(const DecodeArgs& a, bool fp8, hipStream_t stream);

// A scratch area the library owns (fkv_decode_attn_noalloc): `bytes` in all, merge counters in
// the first `ctl_bytes` (256 per (sequence, KV head) pair; zero before every call, and every
// call leaves them zero), split partials after them. acquire(stream, &status) returns the
// area's device address on the current device, setting it up on first use; it runs only
// after the call's arguments are validated.
struct FixedScratch {
  void* (*acquire)(void* stream, int* status);
  uint64_t bytes;
  uint64_t ctl_bytes;
};
// fkv_decode_attn with its workspace in a FixedScratch (validation, plan and launches shared).
int decode_attn_fixed_scratch(const fkv_cache* cache, const fkv_decode_desc* desc, const uint16_t* q,
                              const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                              const float* v_scale, void* out, const FixedScratch& scratch, void* stream);

// Returns hipErrorInvalidValue when no kernel is compiled for the shape.
hipError_t launch_decode(const DecodeArgs& a, const SplitShapeInfo& shape, bool fp8, hipStream_t stream,
                         bool* launched_combine);

}  // namespace fkv
