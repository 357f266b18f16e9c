/*
 * fkv.h -- C ABI of libfkv.so: calibrated-FP8 paged KV cache insertion and
 * paged GQA decode attention for AMD Instinct MI355X (gfx950).
 *
 * The problem statement comes from four pages of the b70-optimization-lab:
 *   [P1] "Laguna S 2.1 INT4 -- calibrated FP8 KV on Intel B70"
 *   [P2] "Laguna FP8 KV -- replicated embedding win, page-32 build, and host boundary"
 *   [P3] "Laguna S 2.1 B70 campaign transfer ledger"
 *   [P4] "Laguna S 2.1 KV-cache precision decision"
 *
 * Conventions shared by every call:
 *  - Every device buffer is owned by the caller. The library allocates no
 *    device memory and never synchronises the stream; its only device state is
 *    the static scratch array of fkv_decode_attn_noalloc (loaded with the library).
 *    Fixed-address buffers can therefore be refreshed in place between calls
 *    ([P3] "Result progression": persistent fixed-address attention metadata).
 *  - Pointers named "device" must be device-accessible and 16-byte aligned.
 *  - Streams are hipStream_t passed as void* (NULL = the legacy default stream).
 *    Calls are asynchronous on that stream.
 *  - Every call returns FKV_OK or an error code. Arguments are validated on the
 *    host before any HIP call; an unsupported shape returns FKV_EUNSUPPORTED and
 *    never falls back to another path ([P2] "Page-32 attention experiment" and
 *    "Transferable learnings": a fallback invalidates the result). No C++
 *    exception crosses the ABI. The calls are thread-safe.
 */
#ifndef FKV_H
#define FKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------------------------- */
#define FKV_OK 0
#define FKV_EINVAL 1        /* null pointer, bad size, misalignment, inconsistent shapes     */
#define FKV_EUNSUPPORTED 2  /* a shape no compiled kernel covers (no fallback exists)          */
#define FKV_EWORKSPACE 3    /* workspace missing or smaller than fkv_decode_workspace_bytes   */
#define FKV_EHIP 4          /* the HIP runtime reported an error at launch                    */

/* ---- cache element types ([P1] Contract: explicit E4M3 KV; [P4] BF16 as the control) ---- */
#define FKV_FP8_E4M3FN 1    /* OCP E4M3FN bytes: bias 7, max 448, S.1111.111 = NaN, no inf  */
#define FKV_BF16 2          /* BF16 bit patterns, stored unchanged                            */

/* ---- output types ------------------------------------------------------------------------ */
#define FKV_OUT_F32 1
#define FKV_OUT_BF16 2

#define FKV_HEAD_DIM 128
#define FKV_MAX_Q_LEN 16
#define FKV_MAX_PREFILL_Q_LEN 4096

/*
 * Cache geometry. [P2] "Page-32 attention experiment": page (block) sizes 32 and
 * 64, head size 128; [P4] "BF16 versus FP8 in concrete terms": 8 KV heads x 128.
 *
 * Pool layout (element = 1 byte for FP8, 2 bytes for BF16; index in elements):
 *   K pool: index(blk, h, o, d) = ((blk*num_kv_heads + h)*block_size + o)*128 + d
 *   V pool: index(blk, h, o, d) = (blk*num_kv_heads + h)*block_size*128
 *                                 + (o/8)*1024 + d*8 + (o%8)
 * for physical block blk, KV head h, offset o in the block and dimension d.
 * Each (block, head) owns one contiguous block_size*128-element slab per pool.
 * K rows are contiguous per key; in V every group of 8 keys is stored
 * dimension-major, so 8 consecutive keys of one dimension are 8 consecutive
 * elements. Key j of a sequence lives in block block_table[j / block_size] at
 * offset j % block_size.
 */
typedef struct fkv_cache_desc {
  int32_t num_blocks;    /* physical blocks in each pool, >= 1                 */
  int32_t block_size;    /* 32 or 64                                           */
  int32_t num_kv_heads;  /* >= 1                                               */
  int32_t head_dim;      /* must be 128                                        */
  int32_t cache_dtype;   /* FKV_FP8_E4M3FN or FKV_BF16                         */
} fkv_cache_desc;

/* Value handle filled by fkv_init_cache; nothing to free. */
typedef struct fkv_cache {
  fkv_cache_desc desc;
  void* k_pool;          /* device */
  void* v_pool;          /* device */
  uint64_t pool_bytes;   /* bytes of each pool */
} fkv_cache;

/*
 * Byte size of each pool: num_blocks * num_kv_heads * block_size * 128 * element
 * bytes. Per token and layer that is 2 * num_kv_heads * 128 elements for K + V:
 * 2,048 bytes in FP8 and 4,096 in BF16 at 8 KV heads ([P4] "BF16 versus FP8 in
 * concrete terms"). Pure host arithmetic. Errors: FKV_EINVAL for a null argument,
 * a non-positive size or an overflow; FKV_EUNSUPPORTED for block_size not in
 * {32, 64}, head_dim != 128 or an unknown cache_dtype.
 */
int fkv_cache_bytes(const fkv_cache_desc* desc, size_t* k_bytes, size_t* v_bytes);

/*
 * Fills *out from desc and two caller-owned device pools of fkv_cache_bytes each
 * (the paged E4M3 K and V pools of [P1] Contract and [P2] "Page-32 attention
 * experiment"; the pools stay the caller's, as the fixed-address buffers of
 * [P3] "Result progression"). No allocation and no device work: pool contents
 * stay undefined until tokens are inserted. Errors as fkv_cache_bytes, plus
 * FKV_EINVAL for null or misaligned pools.
 */
int fkv_init_cache(const fkv_cache_desc* desc, void* k_pool, void* v_pool, fkv_cache* out);

/*
 * Cache insertion ([P1] Contract: explicit E4M3 FP8 KV with the checkpoint's
 * calibrated scalar K/V scales, unit scales for uncalibrated draft layers, no
 * runtime scale calculation; [P4] "What the official checkpoint requests":
 * static, symmetric, per-tensor scales; [P1] "Initial optimization order":
 * FP8 cache update profiled on its own).
 *
 *  k, v          device BF16 [num_tokens][num_kv_heads][128]
 *  slot_mapping  device int32 [num_tokens]: token t goes to block slot/block_size,
 *                offset slot%block_size. Negative slots, and slots >= num_blocks *
 *                block_size, are skipped. Duplicate slots leave an undefined winner.
 *  k_scale, v_scale  device pointers to one fp32 each (> 0, finite); read on the
 *                device so the call needs no host sync. Ignored for a BF16 cache.
 *
 * FP8: each element is stored as E4M3FN(fp32(x) / fp32(scale)) with one
 * correctly rounded fp32 division, then round-to-nearest-even to E4M3FN,
 * saturating to +-448 for |quotient| >= 448 (infinities included); a NaN
 * quotient stores 0x7F|sign. BF16: the bit patterns are copied.
 * num_tokens == 0 is a no-op. Errors: FKV_EINVAL (null/misaligned pointers,
 * num_tokens < 0), FKV_EHIP.
 */
int fkv_insert(const fkv_cache* cache, const uint16_t* k, const uint16_t* v, const int32_t* slot_mapping,
               int32_t num_tokens, const float* k_scale, const float* v_scale, void* stream);

/*
 * Decode attention shape ([P1] "Initial optimization order": exact q1 and M12
 * paged attention; [P1] Contract: width 12; [P2] "Page-32 attention experiment":
 * q=18, kv=2, head 128, global (-1,-1) and sliding windows; [P4]: 36 layers with a
 * 512-token window and 12 global layers).
 */
typedef struct fkv_decode_desc {
  int32_t num_seqs;            /* >= 0 (0 = no-op)                                          */
  int32_t q_len;               /* M query tokens per sequence (q1 = 1, M12 = 12): 1..16 with
                                  at most 112 packed rows (Hq/Hkv) * M per KV head; longer
                                  windows (chunked prefill: the causal attention of up to
                                  FKV_MAX_PREFILL_Q_LEN new tokens to the cached prefix and
                                  to each other, [P1] "Initial optimization order" leaves the
                                  prefill lane for later) with an FP8 cache, layout 0 or 5,
                                  row_groups 0 and row_exact 0 only (else FKV_EUNSUPPORTED);
                                  fkv_insert_decode takes at most 16                      */
  int32_t num_q_heads;         /* multiple of num_kv_heads; (Hq/Hkv)*M <= 112               */
  int32_t max_blocks_per_seq;  /* row stride of block_table, >= 1                           */
  int32_t max_seq_len;         /* host upper bound on seq_lens[], sizes the split grid      */
  int32_t window_left;         /* -1 = global; w >= 0: keys p-w..p visible to position p    */
  float softmax_scale;         /* > 0, finite; 1/sqrt(128) for these models                 */
  int32_t out_dtype;           /* FKV_OUT_F32 (out is float) or FKV_OUT_BF16 (out is BF16,
                                  each fp32 result rounded to nearest even; the activations
                                  of the models are BF16: [P1] Contract)                   */
  int32_t split_tiles;         /* 0 = automatic; else 32-key tiles per split-KV work group
                                  (at most 128)                                            */
  int32_t layout;              /* work-group layout: 0 = automatic (layout 5 for an FP8 cache,
                                  except layout 3 for fkv_decode_attn when the packed rows
                                  of a KV head fit one 16-row tile and row_exact is 0;
                                  layout 3 for a BF16 cache);
                                  3 = row groups of at most 32 rows in separate work groups
                                  that share K/V tiles through the L2 of one XCD (16-row
                                  tiles, MFMA 16x16x32);
                                  5 = 32-row tiles (MFMA 32x32x16), eight waves per work
                                  group, the split's rows in row_groups work groups on one
                                  XCD; splits merged inside the kernel when the grid fits on
                                  the chip (FP8 cache only, else FKV_EUNSUPPORTED);
                                  6 = layout 5 with two row tiles per work group, both held
                                  by each of its four waves (one per SIMD); results bitwise
                                  equal to layout 5 with the same row tiles per work group
                                  (FP8 cache and at least 33 packed rows, else
                                  FKV_EUNSUPPORTED); any other value: FKV_EINVAL          */
  int32_t row_groups;          /* layout 5: work groups sharing one split's query rows (1, 2
                                  or 4, at most the number of 32-row tiles; 0 = automatic);
                                  layout 6: 0 or the number of 32-row tiles / 2 (else
                                  FKV_EUNSUPPORTED); ignored by the other layouts           */
  int32_t row_exact;           /* nonzero: row-exact mode (layout 0 or 5, FP8 cache, else
                                  FKV_EUNSUPPORTED; split_tiles > 0 and a multiple of 4,
                                  else FKV_EINVAL). A query row's output then depends only on
                                  its own query, its position and the cache: calls with equal
                                  split_tiles give bitwise-equal rows, e.g. row i of a q_len =
                                  12 call equals a q_len = 1 call at seq_len L - 12 + i + 1
                                  ([P3] "Result progression and what actually worked": a
                                  verifier with M=1 numerical lanes; "Numerical width is a
                                  contract, not just a tensor shape": row-wise lanes)     */
} fkv_decode_desc;

/*
 * Bytes of device workspace fkv_decode_attn needs for (cache, desc): split-KV
 * partial results (the long-context decode of [P4] "BF16 versus FP8 in concrete
 * terms" is split along the keys to fill the chip) and, for layout 5, 256 bytes
 * of merge counters per (sequence, KV head) at its end. With the automatic layout and one 16-row tile of an FP8
 * cache the size covers both kernels that fkv_decode_attn and fkv_insert_decode
 * then run, so one workspace serves both calls. Pure host arithmetic; may be 0. The workspace must be
 * zero-filled once before its first use (the counters must start at zero); every
 * call returns the counters to zero, so it can then be reused without clearing.
 * One call at a time may use a workspace. Errors as fkv_decode_attn's validation.
 */
int fkv_decode_workspace_bytes(const fkv_cache* cache, const fkv_decode_desc* desc, size_t* bytes);

/*
 * Paged GQA decode attention over the cache.
 *
 *  q            device BF16 [num_seqs][q_len][num_q_heads][128]
 *  block_table  device int32 [num_seqs][max_blocks_per_seq], physical block ids
 *  seq_lens     device int32 [num_seqs]: L = tokens in the cache for the sequence,
 *               INCLUDING the q_len new tokens (already inserted on this stream);
 *               q_len <= L <= min(max_seq_len, max_blocks_per_seq*block_size)
 *  k_scale, v_scale  device fp32 scalars (FP8 cache; ignored for BF16)
 *  out          device fp32 (out_dtype FKV_OUT_F32) or BF16 (FKV_OUT_BF16)
 *               [num_seqs][q_len][num_q_heads][128], 16-byte aligned
 *
 * Query row i sits at position p = L - q_len + i. Key j is visible to it iff
 * lo <= j <= p with lo = 0 (window_left = -1) or max(0, p - window_left). Query
 * head h reads KV head h / (num_q_heads / num_kv_heads). With
 * k = decode(byte) * k_scale and v = decode(byte) * v_scale (FP8), or the BF16
 * values:
 *    out[i][h] = sum_j softmax_j(softmax_scale * <q[i][h], k_j>) * v_j.
 * The result is attention over the dequantised FP8 cache, never over the
 * BF16 originals ([P1] Contract: exactness against an FP8 teacher).
 * Rows with no visible key (L < q_len) are written as zeros. Values of
 * seq_lens above the documented bound are clamped to it; block ids outside
 * [0, num_blocks) make their 32-key tile invisible (no out-of-pool read).
 * Reads only the cache, q, the metadata and the scales; writes only out and
 * the workspace. The result is bitwise reproducible for a given input, layout,
 * row_groups and split_tiles. Layout 5 merges the split partials inside its own
 * kernel when every work group of the grid fits on the chip at once (one per CU):
 * a work group waits for the other splits of its (sequence, KV head) only when all
 * of them have started, and the last one to finish completes the merge, so no call
 * depends on co-residency. Errors: FKV_EINVAL (also: row_groups not in {0, 1, 2,
 * 4}), FKV_EUNSUPPORTED (shape not compiled), FKV_EWORKSPACE, FKV_EHIP.
 */
int fkv_decode_attn(const fkv_cache* cache, const fkv_decode_desc* desc, const uint16_t* q,
                    const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                    const float* v_scale, void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fkv_decode_attn without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation). The
 * split-KV scratch (merge counters, then partials) is a static array of the library, one
 * FKV_NOALLOC_SCRATCH_BYTES copy per GPU it runs on, held until the process ends; the call
 * itself allocates nothing. Its first call on a device takes the array's device address and,
 * unless the stream is being captured, clears the counter area on the stream.
 *
 *  arguments as fkv_decode_attn, without workspace and workspace_bytes.
 *
 * Limits: at most FKV_NOALLOC_MAX_PAIRS (sequence, KV head) pairs, and the plan's partials
 * (fkv_decode_workspace_bytes less its counters) must fit the array after the counter area
 * (FKV_NOALLOC_MAX_PAIRS * 256 bytes); beyond either, FKV_EWORKSPACE and nothing is launched.
 * Every call on one GPU shares that GPU's array: calls that may overlap on one GPU (other
 * streams, concurrent graph replays) race and must be serialised by the caller. Outputs are
 * bitwise those of fkv_decode_attn. Errors: as fkv_decode_attn; FKV_EHIP when the array's
 * address cannot be obtained.
 */
#define FKV_NOALLOC_SCRATCH_BYTES (32u << 20)
#define FKV_NOALLOC_MAX_PAIRS 4096
int fkv_decode_attn_noalloc(const fkv_cache* cache, const fkv_decode_desc* desc, const uint16_t* q,
                            const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                            const float* v_scale, void* out, void* stream);

/*
 * Cache insertion of the q_len new tokens fused into decode attention: one launch
 * with the effect of fkv_insert of the new tokens followed by fkv_decode_attn
 * ([P1] "Initial optimization order": scaled E4M3 insertion, with fusing it into
 * the neighbouring step named as the next optimization).
 *
 *  k_new, v_new  device BF16 [num_seqs][q_len][num_kv_heads][128]: token i of
 *                sequence b goes to position p = L - q_len + i (L = seq_lens[b],
 *                which counts the new tokens), i.e. to block block_table[b][p /
 *                block_size], offset p % block_size. Positions p < 0 and block ids
 *                outside [0, num_blocks) are skipped, as fkv_insert skips such slots.
 *  other arguments as fkv_decode_attn (same descriptor, workspace and rules).
 *
 * The pool bytes written are those fkv_insert writes for the same tokens, and out is
 * bitwise equal to fkv_decode_attn's after that insert. Each work group encodes the new
 * tokens of its own key range, stores the codes into the pool and waits for those stores
 * to complete before it reads those keys back (work groups that share a key range store
 * the same bytes). Other work must not read or write the receiving pool blocks during
 * the call. FP8 cache and layout 0, 5 or 6 only (else FKV_EUNSUPPORTED).
 * Errors: as fkv_decode_attn, plus FKV_EINVAL for a null or misaligned k_new/v_new.
 */
int fkv_insert_decode(const fkv_cache* cache, const fkv_decode_desc* desc, const uint16_t* q,
                      const uint16_t* k_new, const uint16_t* v_new, const int32_t* block_table,
                      const int32_t* seq_lens, const float* k_scale, const float* v_scale, void* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-head Q/K RMSNorm and rotary position embedding of num_tokens new tokens, with the
 * normalised, rotated K and the raw V inserted into the cache, in one launch ([P1] "Initial
 * optimization order": the scaled E4M3 insert at the Q/K norm + RoPE step; [P3] "Result
 * progression and what actually worked": an exact fused Q/K RMSNorm/RoPE stack).
 *
 *  q            device BF16 [num_tokens][num_q_heads][128], raw (num_q_heads a multiple
 *               of the cache's num_kv_heads)
 *  k, v         device BF16 [num_tokens][num_kv_heads][128], raw
 *  q_weight, k_weight  device BF16 [128]: the RMSNorm weights of Q and of K
 *  eps          RMSNorm epsilon (finite, >= 0)
 *  cos_sin      device fp32 [rope_rows][128]: row p holds cos(p f_i) for i < 64, then
 *               sin(p f_i); the caller's frequencies f_i (its rotary base)
 *  positions    device int32 [num_tokens]: the token's position (a row of cos_sin)
 *  slot_mapping device int32 [num_tokens]: as fkv_insert
 *  k_scale, v_scale  as fkv_insert
 *  q_out        device BF16 [num_tokens][num_q_heads][128]; may be q itself (in place)
 *  all device buffers 16-byte aligned (positions, slot_mapping and the scales 4-byte)
 *
 * For every head vector x of Q and K, in float32 with every product, sum and quotient
 * rounded on its own (no fused multiply-add): s = the sum of x_d^2, each lane of 8
 * consecutive dims in dim order and then the 16 partial sums combined pairwise at
 * distances 1, 2, 4 and 8; r = 1 / sqrt(s / 128 + eps); y_d = bf16(x_d r w_d) (round to
 * nearest even); z_d = bf16(y_d c_d - y_(d+64) s_d) and z_(d+64) = bf16(y_(d+64) c_d +
 * y_d s_d) for d < 64, with c, s the row of the token's position. q_out receives z of Q;
 * z of K is inserted as fkv_insert inserts a key (the same bytes for an FP8 or BF16
 * cache), V as fkv_insert inserts a value. A token whose position is outside [0,
 * rope_rows) gets a zero q_out row and inserts nothing; a slot outside the pool skips the
 * insert only. Errors: FKV_EINVAL (bad pointers, sizes, eps), FKV_EHIP.
 */
int fkv_qk_norm_rope_insert(const fkv_cache* cache, int32_t num_tokens, int32_t num_q_heads, const uint16_t* q,
                            const uint16_t* k, const uint16_t* v, const uint16_t* q_weight, const uint16_t* k_weight,
                            float eps, const float* cos_sin, int32_t rope_rows, const int32_t* positions,
                            const int32_t* slot_mapping, const float* k_scale, const float* v_scale, uint16_t* q_out,
                            void* stream);

/*
 * fkv_insert_decode with the Q/K RMSNorm + RoPE of fkv_qk_norm_rope_insert in front, all in one
 * launch ([P1] "Initial optimization order": the scaled insert at the Q/K norm + RoPE step,
 * optionally inside the attention call): q holds the raw query rows and k_new the raw new keys
 * (as in fkv_insert_decode); each is normalised and rotated in the attention kernel's prologue
 * with the arithmetic fkv_qk_norm_rope_insert documents, at the row's position L - q_len + i.
 * The pool bytes and out are bitwise those of fkv_qk_norm_rope_insert (positions L - q_len + i,
 * the block table's slots) followed by fkv_decode_attn with the rotated Q on layout 5.
 *
 *  q_weight, k_weight, eps, cos_sin as fkv_qk_norm_rope_insert; rope_rows >= desc->max_seq_len
 *  (every position has a table row)
 *  other arguments as fkv_insert_decode (same rules: FP8 cache, layout 0, 5 or 6, q_len <= 16)
 * Errors: as fkv_insert_decode, plus FKV_EINVAL for a null or misaligned weight or table, a
 * negative or non-finite eps, or too few table rows.
 */
int fkv_norm_rope_insert_decode(const fkv_cache* cache, const fkv_decode_desc* desc, const uint16_t* q,
                                const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q_weight,
                                const uint16_t* k_weight, float eps, const float* cos_sin, int32_t rope_rows,
                                const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                                const float* v_scale, void* out, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Human-readable text of a status code (static storage). Bookkeeping: no passage of
 * the pages defines it; it names the FKV_E* refusals, which replace any fallback
 * ([P2] "Transferable learnings"). */
const char* fkv_status_string(int status);

/*
 * Runtime execution proof ([P3] "Harness, recovery, and evidence lessons": a runtime entry
 * marker or counter per experimental feature): host-side counts of kernel launches per
 * variant since load or the last reset. Index 0 is an FP8 cache, 1 a BF16 cache. Every
 * decode launch (fkv_decode_attn, fkv_insert_decode, fkv_norm_rope_insert_decode) counts once
 * in decode_launches and once in exactly one of decode_row_tiles (the decode shapes, by
 * nt = ceil((Hq/Hkv) * q_len / 16) query row tiles, nt <= 7 and q_len <= 16, at index nt - 1)
 * and decode_long_windows (longer query windows). Counters are updated with relaxed atomics;
 * only the launching thread's own calls are ordered.
 */
typedef struct fkv_counters {
  uint64_t insert_launches[2];      /* fkv_insert                                               */
  uint64_t decode_launches[2];      /* decode launches by cache type                            */
  uint64_t decode_row_tiles[2][7];  /* decode shapes: [cache][nt - 1]                           */
  uint64_t decode_long_windows[2];  /* query windows beyond 16 tokens or 112 packed rows        */
  uint64_t decode_combine_launches; /* separate split-combine kernels                           */
  uint64_t rejected_calls;          /* calls that returned an error                             */
  uint64_t insert_decode_launches;  /* fkv_insert_decode and fkv_norm_rope_insert_decode calls  */
  uint64_t norm_rope_insert_launches[2];      /* fkv_qk_norm_rope_insert                        */
  uint64_t norm_rope_insert_decode_launches;  /* fkv_norm_rope_insert_decode calls              */
} fkv_counters;

/* Copies the counters into *out. Errors: FKV_EINVAL for a null out. */
int fkv_get_counters(fkv_counters* out);
/* Sets every counter to zero. Always FKV_OK. */
int fkv_reset_counters(void);

#ifdef __cplusplus
}
#endif

#endif /* FKV_H */
