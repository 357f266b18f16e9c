// C ABI of libfkv.so: argument validation, split-KV planning, launches, counters.
// Every check runs on the host before any HIP call, so invalid calls fail without a GPU.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>

#include "../../include/fkv.h"
#include "fkv_internal.h"

namespace {

constexpr int kNumCUs = 256;       // MI355X compute units
constexpr int kMaxNT = 7;          // compiled query-row tiles: (Hq/Hkv) * q_len <= 112
constexpr int kMaxSplitTiles = 1 << 20;
constexpr uint64_t kAlign = 256;

std::atomic<uint64_t> g_insert[2];
std::atomic<uint64_t> g_decode[2];                // decode launches by cache type (0 = FP8, 1 = BF16)
std::atomic<uint64_t> g_decode_tiles[2][kMaxNT];  // decode shapes: [cache][query row tiles - 1]
std::atomic<uint64_t> g_long_window[2];           // long query windows (chunked prefill)
std::atomic<uint64_t> g_combine;
std::atomic<uint64_t> g_insert_decode;
std::atomic<uint64_t> g_norm_rope[2];
std::atomic<uint64_t> g_norm_rope_decode;
std::atomic<uint64_t> g_rejected;

// Counter slot of a decode launch: nt - 1 for the decode shapes (1 <= nt <= kMaxNT query row
// tiles of 16 and q_len <= FKV_MAX_Q_LEN), -1 for long query windows, which have no per-shape
// slot. Every index into g_decode_tiles comes from here.
int decode_tile_slot(int nt, int q_len) {
  return (nt >= 1 && nt <= kMaxNT && q_len >= 1 && q_len <= FKV_MAX_Q_LEN) ? nt - 1 : -1;
}

int reject(int code) {
  g_rejected.fetch_add(1, std::memory_order_relaxed);
  return code;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_desc(const fkv_cache_desc* d) {
  if (!d) return FKV_EINVAL;
  if (d->num_blocks < 1 || d->num_kv_heads < 1 || d->block_size < 1 || d->head_dim < 1) return FKV_EINVAL;
  if (d->block_size != 32 && d->block_size != 64) return FKV_EUNSUPPORTED;
  if (d->head_dim != FKV_HEAD_DIM) return FKV_EUNSUPPORTED;
  if (d->cache_dtype != FKV_FP8_E4M3FN && d->cache_dtype != FKV_BF16) return FKV_EUNSUPPORTED;
  if (d->num_kv_heads > 65535) return FKV_EUNSUPPORTED;
  return FKV_OK;
}

int pool_bytes(const fkv_cache_desc* d, uint64_t* bytes) {
  int rc = check_desc(d);
  if (rc) return rc;
  const uint64_t elem = d->cache_dtype == FKV_FP8_E4M3FN ? 1 : 2;
  const uint64_t per_block = (uint64_t)d->num_kv_heads * (uint64_t)d->block_size * FKV_HEAD_DIM * elem;
  if ((uint64_t)d->num_blocks > (UINT64_MAX / 4) / per_block) return FKV_EINVAL;
  *bytes = per_block * (uint64_t)d->num_blocks;
  return FKV_OK;
}

int check_cache(const fkv_cache* c) {
  if (!c) return FKV_EINVAL;
  uint64_t bytes = 0;
  int rc = pool_bytes(&c->desc, &bytes);
  if (rc) return rc;
  if (!c->k_pool || !c->v_pool || c->pool_bytes != bytes) return FKV_EINVAL;
  if (!aligned(c->k_pool, 16) || !aligned(c->v_pool, 16)) return FKV_EINVAL;
  return FKV_OK;
}

uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// Plan of one decode call with the given work-group layout (0: the 32-row kernel for FP8
// caches, the row-group kernel for BF16).
int plan_layout(const fkv_cache* c, const fkv_decode_desc* d, int layout, fkv::DecodePlan* p) {
  int rc = check_cache(c);
  if (rc) return rc;
  if (!d) return FKV_EINVAL;
  const int hkv = c->desc.num_kv_heads;
  if (d->num_seqs < 0 || d->q_len < 1 || d->num_q_heads < 1 || d->max_blocks_per_seq < 1 || d->max_seq_len < 1)
    return FKV_EINVAL;
  if (d->window_left < -1 || d->split_tiles < 0 || d->split_tiles > kMaxSplitTiles) return FKV_EINVAL;
  if (layout != 0 && layout != 3 && layout != 5 && layout != 6) return FKV_EINVAL;
  if (d->row_exact && (d->split_tiles == 0 || d->split_tiles % 4 != 0)) return FKV_EINVAL;
  if (!(std::isfinite(d->softmax_scale) && d->softmax_scale > 0.f)) return FKV_EINVAL;
  if (d->num_q_heads % hkv != 0) return FKV_EINVAL;
  if ((int64_t)d->max_seq_len > (int64_t)d->max_blocks_per_seq * c->desc.block_size) return FKV_EINVAL;
  if (d->q_len > FKV_MAX_PREFILL_Q_LEN) return FKV_EUNSUPPORTED;
  if (d->out_dtype != FKV_OUT_F32 && d->out_dtype != FKV_OUT_BF16) return FKV_EUNSUPPORTED;
  if (d->num_seqs > 65535) return FKV_EUNSUPPORTED;
  const int64_t group = d->num_q_heads / hkv;
  const int64_t rows = group * d->q_len;
  const int nt = (int)((rows + 15) / 16);
  // longer query windows (chunked prefill) run on the 32-row kernel only: 64-row work groups
  const bool long_rows = nt > kMaxNT || d->q_len > FKV_MAX_Q_LEN;
  if (long_rows && !(c->desc.cache_dtype == FKV_FP8_E4M3FN && (layout == 0 || layout == 5) && !d->row_exact &&
                     d->row_groups == 0))
    return FKV_EUNSUPPORTED;
  const bool fp8_cache = c->desc.cache_dtype == FKV_FP8_E4M3FN;
  if ((layout == 5 || layout == 6) && !fp8_cache) return FKV_EUNSUPPORTED;  // the 32-row kernel reads FP8 caches
  p->nt = nt;
  p->rows_pad = 16 * nt;

  // Tiles (32 keys, aligned to absolute position) that can hold visible keys at the
  // longest context: the whole context for global attention, window + verify rows
  // (plus one tile of misalignment) for sliding windows.
  const int64_t lmax = d->max_seq_len;
  int64_t tiles_max = (lmax + 31) / 32;
  if (d->window_left >= 0) tiles_max = std::min<int64_t>(tiles_max, ((int64_t)d->window_left + d->q_len + 31) / 32 + 1);
  p->layout = layout;
  const bool fp8 = c->desc.cache_dtype == FKV_FP8_E4M3FN;
  const fkv::SplitShapeInfo sh = fkv::split_shape(nt, layout, fp8);
  p->row_groups = 1;
  p->key_lanes = 0;
  p->align_splits = 0;
  p->clip_rows = long_rows ? 1 : 0;
  if (d->row_exact && (!fp8 || (layout != 0 && layout != 5))) return FKV_EUNSUPPORTED;
  int64_t tps = d->split_tiles;
  if (sh.groups_per_cu == -2 || sh.groups_per_cu == -3) {
    // 32-row kernel: the rows_pad = 32 * rt_total packed rows of a KV head are cut into RG
    // row groups of separate work groups (on one XCD, sharing K/V tiles through its L2); the
    // splits fill the chip, each key lane takes whole tiles, a split at most 128 tiles.
    // long query windows: ceil(rows / 64) work groups of two row tiles and four key lanes
    const int rt_total = long_rows ? (int)((rows + 63) / 64) * 2 : sh.r;
    p->rows_pad = 32 * rt_total;
    if (d->row_groups != 0 && d->row_groups != 1 && d->row_groups != 2 && d->row_groups != 4) return FKV_EINVAL;
    int rg = d->row_groups;
    const int64_t bg = (int64_t)std::max(d->num_seqs, 1) * hkv;
    if (rg == 0) {
      // Automatic: two row groups whenever there are two row tiles. Each split partial costs
      // 512 bytes per row written and read back, each K/V tile 8 KB per reading work group
      // (the second reader hits the XCD's L2); measured on the 72/8-head layer at M = 12,
      // two groups beat one and four at both 8k and 32k context.
      rg = rt_total >= 2 ? 2 : 1;
      if (long_rows) rg = rt_total / 2;
    }
    if (sh.groups_per_cu == -3) {
      // layout 6: two row tiles per work group (both held by each of its four waves)
      if (rt_total < 2) return FKV_EUNSUPPORTED;
      if (d->row_groups != 0 && d->row_groups != rt_total / 2) return FKV_EUNSUPPORTED;
      rg = rt_total / 2;
    }
    if (d->row_exact) {
      // row-exact mode: four key lanes whatever the rows (one or two row tiles per work group)
      if (d->row_groups == 0) rg = rt_total >= 2 ? rt_total / 2 : 1;
      if (rt_total / rg > 2) return FKV_EUNSUPPORTED;
      p->align_splits = 1;
    }
    if (rg > rt_total) return FKV_EUNSUPPORTED;
    p->row_groups = rg;
    const int kl = (sh.groups_per_cu == -3 || d->row_exact) ? 4 : 8 / (rt_total / rg);
    p->key_lanes = kl;
    if (tps == 0) {
      // Fill the chip, but with at most kFastMergeSplits splits, or up to twice that while
      // every split keeps at least four steps of kl tiles: with few (sequence, KV head) pairs
      // more splits of one step each cost more in partials and merging than they gain
      // (measured at 18/2 heads, 8k: 64 one-step splits 29.6 us, 16 four-step splits
      // 20.3 us), while 32 four-step splits beat 16 eight-step ones with the layer in HBM
      // (72/8 heads, q1, 32k: 29.8 vs 31.8-33.1 us per graph-replayed fused step).
      const int64_t cap = std::max<int64_t>(fkv::kFastMergeSplits,
                                            std::min<int64_t>(2 * fkv::kFastMergeSplits, tiles_max / (4 * kl)));
      const int64_t splits = std::max<int64_t>(1, std::min<int64_t>(kNumCUs / (bg * rg), cap));
      tps = (tiles_max + splits - 1) / splits;
      tps = (tps + kl - 1) / kl * kl;
      tps = std::min<int64_t>(tps, fkv::kMaxDmaSplitTiles);
      tps = std::max<int64_t>(tps, (tiles_max + fkv::kMaxSplits - 1) / fkv::kMaxSplits);
    }
    if (tps > fkv::kMaxDmaSplitTiles) return FKV_EUNSUPPORTED;  // the page-table window holds 128 entries
  } else {
    // row-group kernel (layout 3): one work group per CU; the row groups of a KV head
    // multiply the work groups, the splits fill the rest of the chip
    p->row_groups = sh.r;
    p->rows_pad = 16 * sh.ntw * sh.r;
    if (tps == 0) {
      const int64_t bg = (int64_t)std::max(d->num_seqs, 1) * hkv;
      const int64_t splits = std::max<int64_t>(1, kNumCUs / (bg * sh.r));
      tps = (tiles_max + splits - 1) / splits;
      tps = (tps + sh.k - 1) / sh.k * sh.k;  // whole tiles for every wave
      tps = std::min<int64_t>(tps, fkv::kMaxDmaSplitTiles);
      tps = std::max<int64_t>(tps, (tiles_max + fkv::kMaxSplits - 1) / fkv::kMaxSplits);
    }
    if (tps > fkv::kMaxDmaSplitTiles) return FKV_EUNSUPPORTED;  // its page-table window holds 128 entries
  }
  // aligned splits (row-exact mode) can straddle one more split boundary inside a window
  const int64_t max_splits = (tiles_max + tps - 1) / tps + (p->align_splits && d->window_left >= 0 ? 1 : 0);
  if (max_splits > fkv::kMaxSplits) return FKV_EUNSUPPORTED;
  if ((int64_t)std::max(d->num_seqs, 1) * hkv * max_splits * p->row_groups > 0x7FFFFFFF) return FKV_EUNSUPPORTED;
  p->tiles_per_split = (int)tps;
  p->max_splits = (int)max_splits;
  // With at least eight (sequence, KV head) pairs, each pair's work groups go to one XCD (all
  // eight XCDs stay busy); else each split's row groups share one.
  p->xcd_pairs = (int64_t)std::max(d->num_seqs, 1) * hkv >= 8 ? 1 : 0;
  p->fused_combine = 0;
  p->ws_ctl_bytes = 0;
  if (max_splits <= 1) {
    p->ws_o_bytes = p->ws_ml_bytes = p->ws_bytes = 0;
    return FKV_OK;
  }
  const uint64_t parts = (uint64_t)d->num_seqs * hkv * (uint64_t)max_splits;
  p->ws_o_bytes = round_up(parts * p->rows_pad * FKV_HEAD_DIM * sizeof(float), kAlign);
  p->ws_ml_bytes = round_up(parts * 2 * p->rows_pad * sizeof(float), kAlign);
  if (sh.groups_per_cu <= -2) {
    // 32-row kernel: when every work group of the grid fits on the chip at once (one per
    // CU), the splits of a (sequence, KV head) are merged inside the kernel
    const int64_t pairs = (int64_t)d->num_seqs * hkv;
    const int64_t per_pair = max_splits * p->row_groups;
    const int64_t grid = p->xcd_pairs ? (pairs + 7) / 8 * 8 * per_pair : pairs * per_pair;
    p->fused_combine = (grid <= kNumCUs && !long_rows) ? 1 : 0;  // long windows: the combine kernel
    p->ws_ctl_bytes = round_up((uint64_t)pairs * 256, kAlign);  // 256 bytes of counters per pair
  }
  p->ws_bytes = p->ws_o_bytes + p->ws_ml_bytes + p->ws_ctl_bytes;
  return FKV_OK;
}

}  // namespace

// Plan of a call. With the automatic layout an FP8 cache uses the 32-row kernel, except that
// one 16-row tile of query rows (q1 at 9 query heads per KV head) decodes faster with the
// row-group kernel (measured on MI355X: 431 vs 495 us on the 32-sequence batch, 23.6 vs 26.3 us
// at 32k); the fused insert exists in the 32-row kernel only. Both calls then share one
// workspace, sized for either, with the 32-row kernel's merge counters after both partial
// regions so that neither layout's partials can overwrite them.
static int plan_decode(const fkv_cache* c, const fkv_decode_desc* d, fkv::DecodePlan* p, bool fused_insert) {
  int rc = plan_layout(c, d, d ? d->layout : 0, p);
  if (rc) return rc;
  p->ws_ctl_offset = p->ws_o_bytes + p->ws_ml_bytes;
  const bool fp8 = c->desc.cache_dtype == FKV_FP8_E4M3FN;
  if (d->layout == 0 && fp8 && p->nt == 1 && !d->row_exact) {
    fkv::DecodePlan rows;
    if (plan_layout(c, d, 3, &rows) == FKV_OK) {
      const size_t off = std::max(p->ws_o_bytes + p->ws_ml_bytes, rows.ws_o_bytes + rows.ws_ml_bytes);
      const size_t total = off + p->ws_ctl_bytes;
      if (!fused_insert) *p = rows;
      p->ws_ctl_offset = off;
      p->ws_bytes = total;
    }
  }
  return FKV_OK;
}

extern "C" {

int fkv_cache_bytes(const fkv_cache_desc* desc, size_t* k_bytes, size_t* v_bytes) {
  if (!k_bytes || !v_bytes) return reject(FKV_EINVAL);
  uint64_t b = 0;
  int rc = pool_bytes(desc, &b);
  if (rc) return reject(rc);
  *k_bytes = (size_t)b;
  *v_bytes = (size_t)b;
  return FKV_OK;
}

int fkv_init_cache(const fkv_cache_desc* desc, void* k_pool, void* v_pool, fkv_cache* out) {
  if (!out) return reject(FKV_EINVAL);
  uint64_t b = 0;
  int rc = pool_bytes(desc, &b);
  if (rc) return reject(rc);
  if (!k_pool || !v_pool || !aligned(k_pool, 16) || !aligned(v_pool, 16)) return reject(FKV_EINVAL);
  std::memset(out, 0, sizeof(*out));
  out->desc = *desc;
  out->k_pool = k_pool;
  out->v_pool = v_pool;
  out->pool_bytes = b;
  return FKV_OK;
}

int fkv_insert(const fkv_cache* cache, const uint16_t* k, const uint16_t* v, const int32_t* slot_mapping,
               int32_t num_tokens, const float* k_scale, const float* v_scale, void* stream) {
  int rc = check_cache(cache);
  if (rc) return reject(rc);
  if (num_tokens < 0) return reject(FKV_EINVAL);
  if (num_tokens == 0) return FKV_OK;
  const bool fp8 = cache->desc.cache_dtype == FKV_FP8_E4M3FN;
  if (!k || !v || !slot_mapping || !aligned(k, 16) || !aligned(v, 16) || !aligned(slot_mapping, 4))
    return reject(FKV_EINVAL);
  if (fp8 && (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4))) return reject(FKV_EINVAL);
  fkv::InsertArgs a;
  a.k = k;
  a.v = v;
  a.slots = slot_mapping;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.k_pool = cache->k_pool;
  a.v_pool = cache->v_pool;
  a.num_tokens = num_tokens;
  a.num_kv_heads = cache->desc.num_kv_heads;
  a.block_size = cache->desc.block_size;
  a.num_slots = (int64_t)cache->desc.num_blocks * cache->desc.block_size;
  if (fkv::launch_insert(a, fp8, static_cast<hipStream_t>(stream)) != hipSuccess) return reject(FKV_EHIP);
  g_insert[fp8 ? 0 : 1].fetch_add(1, std::memory_order_relaxed);
  return FKV_OK;
}

int fkv_qk_norm_rope_insert(const fkv_cache* cache, int32_t num_tokens, int32_t num_q_heads, const uint16_t* q,
                            const uint16_t* k, const uint16_t* v, const uint16_t* q_weight, const uint16_t* k_weight,
                            float eps, const float* cos_sin, int32_t rope_rows, const int32_t* positions,
                            const int32_t* slot_mapping, const float* k_scale, const float* v_scale, uint16_t* q_out,
                            void* stream) {
  int rc = check_cache(cache);
  if (rc) return reject(rc);
  if (num_tokens < 0 || num_q_heads < 1 || num_q_heads % cache->desc.num_kv_heads != 0 || rope_rows < 1)
    return reject(FKV_EINVAL);
  if (!(std::isfinite(eps) && eps >= 0.f)) return reject(FKV_EINVAL);
  if (num_tokens == 0) return FKV_OK;
  const bool fp8 = cache->desc.cache_dtype == FKV_FP8_E4M3FN;
  const void* p16[] = {q, k, v, q_weight, k_weight, cos_sin, q_out};
  for (const void* ptr : p16)
    if (!ptr || !aligned(ptr, 16)) return reject(FKV_EINVAL);
  if (!positions || !slot_mapping || !aligned(positions, 4) || !aligned(slot_mapping, 4)) return reject(FKV_EINVAL);
  if (fp8 && (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4))) return reject(FKV_EINVAL);
  fkv::NormRopeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_w = q_weight;
  a.k_w = k_weight;
  a.cos_sin = cos_sin;
  a.positions = positions;
  a.slots = slot_mapping;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.q_out = q_out;
  a.k_pool = cache->k_pool;
  a.v_pool = cache->v_pool;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = cache->desc.num_kv_heads;
  a.block_size = cache->desc.block_size;
  a.rope_rows = rope_rows;
  a.num_slots = (int64_t)cache->desc.num_blocks * cache->desc.block_size;
  a.eps = eps;
  if (fkv::launch_norm_rope_insert(a, fp8, static_cast<hipStream_t>(stream)) != hipSuccess) return reject(FKV_EHIP);
  g_norm_rope[fp8 ? 0 : 1].fetch_add(1, std::memory_order_relaxed);
  return FKV_OK;
}

int fkv_decode_workspace_bytes(const fkv_cache* cache, const fkv_decode_desc* desc, size_t* bytes) {
  if (!bytes) return reject(FKV_EINVAL);
  fkv::DecodePlan p;
  int rc = plan_decode(cache, desc, &p, false);
  if (rc) return reject(rc);
  *bytes = (size_t)p.ws_bytes;
  return FKV_OK;
}

// Q/K RMSNorm + RoPE in front of the fused insert (fkv_norm_rope_insert_decode)
struct NormRopeIn {
  const uint16_t* q_w;
  const uint16_t* k_w;
  const float* cos_sin;
  int32_t rope_rows;
  float eps;
};

static int decode_call(const fkv_cache* cache, const fkv_decode_desc* desc, const uint16_t* q, const uint16_t* k_new,
                       const uint16_t* v_new, const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                       const float* v_scale, void* out, void* workspace, size_t workspace_bytes, void* stream,
                       const NormRopeIn* nr = nullptr, const fkv::FixedScratch* fixed = nullptr) {
  const bool fused_insert = k_new != nullptr;
  fkv::DecodePlan p;
  int rc = plan_decode(cache, desc, &p, fused_insert);
  if (rc) return reject(rc);
  const bool fp8 = cache->desc.cache_dtype == FKV_FP8_E4M3FN;
  // the fused insert exists in the 32-row kernel only (FP8 cache, layout 5, 6 or automatic)
  if (fused_insert && (!fp8 || fkv::split_shape(p.nt, p.layout, fp8).groups_per_cu > -2)) return reject(FKV_EUNSUPPORTED);
  if (fused_insert && desc->q_len > FKV_MAX_Q_LEN) return reject(FKV_EUNSUPPORTED);  // the kernel stages 16 tokens
  if (desc->num_seqs == 0) return FKV_OK;
  if (fused_insert && (!v_new || !aligned(k_new, 16) || !aligned(v_new, 16))) return reject(FKV_EINVAL);
  if (!q || !block_table || !seq_lens || !out) return reject(FKV_EINVAL);
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(block_table, 4) || !aligned(seq_lens, 4))
    return reject(FKV_EINVAL);
  if (fp8 && (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4))) return reject(FKV_EINVAL);
  char* ctl_base = static_cast<char*>(workspace) + p.ws_ctl_offset;
  char* part_base = static_cast<char*>(workspace);
  if (fixed) {
    // a fixed scratch area: the merge counters at its start (the same place for every call, so
    // no call's partials can land on another call's counters), the partials after them
    const uint64_t pairs = (uint64_t)desc->num_seqs * cache->desc.num_kv_heads;
    if (pairs * 256 > fixed->ctl_bytes || fixed->ctl_bytes + p.ws_o_bytes + p.ws_ml_bytes > fixed->bytes)
      return reject(FKV_EWORKSPACE);
    int status = FKV_OK;
    char* base = static_cast<char*>(fixed->acquire(stream, &status));
    if (status != FKV_OK || !base) return reject(status != FKV_OK ? status : FKV_EHIP);
    ctl_base = base;
    part_base = base + fixed->ctl_bytes;
  } else {
    if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes)) return reject(FKV_EWORKSPACE);
    if (workspace && !aligned(workspace, 16)) return reject(FKV_EINVAL);
  }

  fkv::DecodeArgs a;
  a.k_pool = static_cast<const uint8_t*>(cache->k_pool);
  a.v_pool = static_cast<const uint8_t*>(cache->v_pool);
  a.q = q;
  a.k_new = k_new;
  a.v_new = fused_insert ? v_new : nullptr;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.out = static_cast<float*>(out);
  a.out_bf16 = desc->out_dtype == FKV_OUT_BF16 ? 1 : 0;
  a.q_w = nr ? nr->q_w : nullptr;
  a.k_w = nr ? nr->k_w : nullptr;
  a.cos_sin = nr ? nr->cos_sin : nullptr;
  a.eps = nr ? nr->eps : 0.f;
  a.ws_o = p.ws_bytes ? reinterpret_cast<float*>(part_base) : nullptr;
  a.ws_ml = p.ws_bytes ? reinterpret_cast<float*>(part_base + p.ws_o_bytes) : nullptr;
  a.ws_ctl = p.ws_ctl_bytes ? reinterpret_cast<uint32_t*>(ctl_base) : nullptr;
  a.fused_combine = p.fused_combine;
  a.xcd_pairs = p.xcd_pairs;
  a.num_seqs = desc->num_seqs;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = cache->desc.num_kv_heads;
  a.group = desc->num_q_heads / cache->desc.num_kv_heads;
  a.q_len = desc->q_len;
  a.block_size = cache->desc.block_size;
  a.max_blocks = desc->max_blocks_per_seq;
  a.num_blocks = cache->desc.num_blocks;
  a.window_left = desc->window_left;
  a.tiles_per_split = p.tiles_per_split;
  a.max_splits = p.max_splits;
  a.max_seq_len = desc->max_seq_len;
  a.rows_pad = p.rows_pad;
  a.row_groups = p.row_groups;
  a.key_lanes = p.key_lanes;
  a.align_splits = p.align_splits;
  a.clip_rows = p.clip_rows;
  a.softmax_scale = desc->softmax_scale;
  bool combined = false;
  const hipError_t e = fkv::launch_decode(a, fkv::split_shape(p.nt, p.layout, fp8), fp8, static_cast<hipStream_t>(stream),
                                          &combined);
  if (e == hipErrorInvalidValue) return reject(FKV_EUNSUPPORTED);
  if (e != hipSuccess) return reject(FKV_EHIP);
  const int ci = fp8 ? 0 : 1;
  g_decode[ci].fetch_add(1, std::memory_order_relaxed);
  const int slot = decode_tile_slot(p.nt, desc->q_len);
  if (slot >= 0)
    g_decode_tiles[ci][slot].fetch_add(1, std::memory_order_relaxed);
  else
    g_long_window[ci].fetch_add(1, std::memory_order_relaxed);
  if (combined) g_combine.fetch_add(1, std::memory_order_relaxed);
  if (fused_insert) g_insert_decode.fetch_add(1, std::memory_order_relaxed);
  if (nr) g_norm_rope_decode.fetch_add(1, std::memory_order_relaxed);
  return FKV_OK;
}

int fkv_decode_attn(const fkv_cache* cache, const fkv_decode_desc* desc, const uint16_t* q,
                    const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                    const float* v_scale, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_call(cache, desc, q, nullptr, nullptr, block_table, seq_lens, k_scale, v_scale, out, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"

int fkv::decode_attn_fixed_scratch(const fkv_cache* cache, const fkv_decode_desc* desc, const uint16_t* q,
                                   const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                                   const float* v_scale, void* out, const FixedScratch& scratch, void* stream) {
  return decode_call(cache, desc, q, nullptr, nullptr, block_table, seq_lens, k_scale, v_scale, out, nullptr, 0, stream,
                     nullptr, &scratch);
}

extern "C" {

int fkv_insert_decode(const fkv_cache* cache, const fkv_decode_desc* desc, const uint16_t* q, const uint16_t* k_new,
                      const uint16_t* v_new, const int32_t* block_table, const int32_t* seq_lens,
                      const float* k_scale, const float* v_scale, void* out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (!k_new || !v_new) return reject(FKV_EINVAL);
  return decode_call(cache, desc, q, k_new, v_new, block_table, seq_lens, k_scale, v_scale, out, workspace,
                     workspace_bytes, stream);
}

int fkv_norm_rope_insert_decode(const fkv_cache* cache, const fkv_decode_desc* desc, const uint16_t* q,
                                const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q_weight,
                                const uint16_t* k_weight, float eps, const float* cos_sin, int32_t rope_rows,
                                const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                                const float* v_scale, void* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (!k_new || !v_new || !desc) return reject(FKV_EINVAL);
  if (!q_weight || !k_weight || !cos_sin || !aligned(q_weight, 16) || !aligned(k_weight, 16) || !aligned(cos_sin, 16))
    return reject(FKV_EINVAL);
  if (!(std::isfinite(eps) && eps >= 0.f) || rope_rows < desc->max_seq_len) return reject(FKV_EINVAL);
  const NormRopeIn nr{q_weight, k_weight, cos_sin, rope_rows, eps};
  return decode_call(cache, desc, q, k_new, v_new, block_table, seq_lens, k_scale, v_scale, out, workspace,
                     workspace_bytes, stream, &nr);
}

const char* fkv_status_string(int status) {
  switch (status) {
    case FKV_OK: return "ok";
    case FKV_EINVAL: return "invalid argument";
    case FKV_EUNSUPPORTED: return "unsupported shape (no compiled kernel; no fallback)";
    case FKV_EWORKSPACE: return "workspace missing or too small";
    case FKV_EHIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

int fkv_get_counters(fkv_counters* out) {
  if (!out) return FKV_EINVAL;
  std::memset(out, 0, sizeof(*out));
  for (int i = 0; i < 2; ++i) {
    out->insert_launches[i] = g_insert[i].load(std::memory_order_relaxed);
    out->decode_launches[i] = g_decode[i].load(std::memory_order_relaxed);
    for (int j = 0; j < kMaxNT; ++j) out->decode_row_tiles[i][j] = g_decode_tiles[i][j].load(std::memory_order_relaxed);
    out->decode_long_windows[i] = g_long_window[i].load(std::memory_order_relaxed);
  }
  out->decode_combine_launches = g_combine.load(std::memory_order_relaxed);
  out->insert_decode_launches = g_insert_decode.load(std::memory_order_relaxed);
  out->rejected_calls = g_rejected.load(std::memory_order_relaxed);
  for (int i = 0; i < 2; ++i) out->norm_rope_insert_launches[i] = g_norm_rope[i].load(std::memory_order_relaxed);
  out->norm_rope_insert_decode_launches = g_norm_rope_decode.load(std::memory_order_relaxed);
  return FKV_OK;
}

int fkv_reset_counters(void) {
  for (int i = 0; i < 2; ++i) {
    g_insert[i].store(0);
    g_decode[i].store(0);
    for (int j = 0; j < kMaxNT; ++j) g_decode_tiles[i][j].store(0);
    g_long_window[i].store(0);
  }
  g_combine.store(0);
  g_insert_decode.store(0);
  g_norm_rope[0].store(0);
  g_norm_rope[1].store(0);
  g_norm_rope_decode.store(0);
  g_rejected.store(0);
  return FKV_OK;
}

}  // extern "C"
