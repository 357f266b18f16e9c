// Paged GQA decode attention over an FP8 (E4M3FN) or BF16 paged cache.
//
// Operation: exact q1 / M12 paged attention over the calibrated FP8 cache ("Laguna S 2.1
// INT4 -- calibrated FP8 KV on Intel B70", sections Contract and "Initial optimization
// order"; q=18 / kv=2, head 128, global and sliding windows in "Laguna FP8 KV --
// replicated embedding win, page-32 build, and host boundary", section "Page-32
// attention experiment").
//
// Work decomposition (one sequence b, one KV head g per work group column):
//   * the G*M query rows of a KV head (G = Hq/Hkv query heads x M tokens) are packed into
//     NT tiles of 16 rows; every wave holds all of them, so each K/V byte is fetched and
//     converted exactly once per KV head;
//   * the visible keys are cut into 32-key tiles; a work group of 4 waves takes
//     `tiles_per_split` consecutive tiles (one split-KV split) and its waves take every
//     4th tile;
//   * S^T = K * Q^T on MFMA 16x16x32 bf16 (fp8 -> bf16 is exact), online softmax in the
//     log2 domain, O^T += V^T * P^T on MFMA 16x16x32 f16 (fp8 -> f16 exact, P in f16);
//   * the 4 waves merge in LDS in a fixed order, then the group either writes the final
//     rows (single split) or an fp32 partial (m, l, O) that decode_combine merges over
//     splits in split order.
//
// Key permutation that makes both MFMAs read their operands straight from global
// memory: in a 32-key tile, lane (n = l%16, q = l/16) feeds K rows 8*(n/4) + 4*tt + n%4
// (tt = 0, 1) to the two QK^T products, so the score lanes of the output hold keys
// 8*q .. 8*q+7, which is exactly the B-operand slice the PV product wants; the V slab
// stores each 8-key group dimension-major, so lane (n, q) reads the 64 contiguous
// bytes of dimensions 8n .. 8n+7 for keys 8q .. 8q+7 (d = 8m + dt for MFMA row m and
// d-tile dt). The head dimension is permuted the same way on Q and K (lane group q
// owns d = 32q .. 32q+31), which also leaves each lane owning 32 contiguous output
// dimensions of its query row.
#include "fkv_device.h"
#include "fkv_internal.h"

namespace fkv {

// A row's reference maximum is raised only when a tile's maximum exceeds it by more
// than this many log2 units; probabilities then stay below 2^kLazyTau (exact in f16).
constexpr float kLazyTau = 8.0f;
constexpr float kLog2e = 1.4426950408889634f;

template <bool kFp8>
struct CacheTraits;
template <>
struct CacheTraits<true> {
  typedef uint8_t elem_t;
  static constexpr int kKVec = 2;  // u32x4 per lane per 16-key half: 32 bytes of a K row
  static constexpr int kVVec = 4;  // 64 bytes of V
};
template <>
struct CacheTraits<false> {
  typedef uint16_t elem_t;
  static constexpr int kKVec = 4;  // 64 bytes = 32 bf16 of a K row
  static constexpr int kVVec = 8;  // 128 bytes = 64 bf16 of V
};

template <bool kFp8>
struct TileRegs {
  u32x4_t k[2][CacheTraits<kFp8>::kKVec];
  u32x4_t v[CacheTraits<kFp8>::kVVec];
};

// Per-wave state of the split kernel.
template <int NT>
struct WaveState {
  f32x4_t o[NT][8];  // O^T accumulators: row tile t, d-tile dt
  float m[NT];       // reference maximum per row (log2 units), -inf before any key
  float lsum[NT];    // this lane's share of the row sum
  int rpos[NT];      // absolute position of the lane's row in tile t (-1: padding row)
};

// Uniform facts about one work group's share of the keys.
struct SplitCtx {
  int b, g, s;
  int L, lo_u, lo_max, p_min;
  int tb, te, nsplit;
  int lane, n, q;
  float C;  // softmax_scale * k_scale * log2(e)
};

template <bool kFp8>
__device__ __forceinline__ int tile_block(const DecodeArgs& a, int b, int tile) {
  return a.block_table[(int64_t)b * a.max_blocks + (tile * kTile) / a.block_size];
}

template <bool kFp8>
__device__ __forceinline__ const typename CacheTraits<kFp8>::elem_t* slab_base(const DecodeArgs& a, const void* pool,
                                                                                int blk, int g, int tile) {
  typedef typename CacheTraits<kFp8>::elem_t elem_t;
  const int o0 = (tile * kTile) % a.block_size;
  const int64_t slab = ((int64_t)blk * a.num_kv_heads + g) * (int64_t)a.block_size * kHeadDim;
  return reinterpret_cast<const elem_t*>(pool) + slab + (int64_t)o0 * kHeadDim;
}

// K rows 8*(n/4) + 4*tt + n%4 of the tile, dimensions 32q .. 32q+31.
template <bool kFp8>
__device__ __forceinline__ void load_k(const DecodeArgs& a, int blk, int g, int tile, int n, int q, TileRegs<kFp8>& r) {
  const auto* kb = slab_base<kFp8>(a, a.k_pool, blk, g, tile) + 32 * q;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(kb + (8 * (n >> 2) + 4 * tt + (n & 3)) * kHeadDim);
#pragma unroll
    for (int j = 0; j < CacheTraits<kFp8>::kKVec; ++j) r.k[tt][j] = p[j];
  }
}

// V group q (keys 8q .. 8q+7 of the tile), dimensions 8n .. 8n+7.
template <bool kFp8>
__device__ __forceinline__ void load_v(const DecodeArgs& a, int blk, int g, int tile, int n, int q, TileRegs<kFp8>& r) {
  const auto* base = slab_base<kFp8>(a, a.v_pool, blk, g, tile);
  // slab_base points at key o0's K row offset; for V the group of key o0 starts at o0*128 too
  const u32x4_t* p = reinterpret_cast<const u32x4_t*>(base + q * (8 * kHeadDim) + 64 * n);
#pragma unroll
  for (int j = 0; j < CacheTraits<kFp8>::kVVec; ++j) r.v[j] = p[j];
}

// S^T = K Q^T for both 16-key halves of the tile; Q fragments come from LDS.
template <int NT, bool kFp8>
__device__ __forceinline__ void qk_tile(const TileRegs<kFp8>& cur, const u32x4_t* q_lds, int lane,
                                        f32x4_t (&sacc)[2][NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t) sacc[0][t] = sacc[1][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    bf16x8_t kf0, kf1;
    if constexpr (kFp8) {
      const u32x4_t& v0 = cur.k[0][c >> 1];
      const u32x4_t& v1 = cur.k[1][c >> 1];
      kf0 = fp8x8_to_bf16x8(v0[(c & 1) * 2], v0[(c & 1) * 2 + 1]);
      kf1 = fp8x8_to_bf16x8(v1[(c & 1) * 2], v1[(c & 1) * 2 + 1]);
    } else {
      kf0 = __builtin_bit_cast(bf16x8_t, cur.k[0][c]);
      kf1 = __builtin_bit_cast(bf16x8_t, cur.k[1][c]);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bf16x8_t qf = __builtin_bit_cast(bf16x8_t, q_lds[(t * 4 + c) * 64 + lane]);
      sacc[0][t] = mfma_bf16(kf0, qf, sacc[0][t]);
      sacc[1][t] = mfma_bf16(kf1, qf, sacc[1][t]);
    }
  }
}

// Masking, online softmax and O^T += V^T P^T for one tile.
template <int NT, bool kFp8>
__device__ __forceinline__ void softmax_pv_tile(const DecodeArgs& a, const SplitCtx& cx, WaveState<NT>& st,
                                                TileRegs<kFp8>& cur, f32x4_t (&sacc)[2][NT], int tile) {
  const int kt = tile * kTile;
  const int q = cx.q;
  const bool interior = (kt >= cx.lo_max) && (kt + kTile - 1 <= cx.p_min);
  const int wl = a.window_left;
  if (!interior) {
    // Invisible keys get -inf. The test is sign arithmetic, (j - lo) | (hi - j) < 0,
    // turned into a bit mask, so no per-element compare masks occupy scalar registers.
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int hi = st.rpos[t];
      const int lo = (wl < 0) ? 0 : max(0, hi - wl);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = kt + 8 * q + 4 * tt + i;
          const uint32_t bad = (uint32_t)(((j - lo) | (hi - j)) >> 31);
          sacc[tt][t][i] = __uint_as_float((bad & 0xFF800000u) | (~bad & __float_as_uint(sacc[tt][t][i])));
        }
    }
    // keys outside [lo_u, L) may hold stale bytes: zero their V so 0 * NaN cannot occur
    const int e0 = min(8, max(0, cx.lo_u - (kt + 8 * q)));
    const int e1 = min(8, max(0, cx.L - (kt + 8 * q)));
    if (e0 > 0 || e1 < 8) {
      if constexpr (kFp8) {
        const uint64_t keep = (e1 >= 8 ? ~0ull : ((1ull << (8 * e1)) - 1)) &
                              (e0 >= 8 ? 0ull : ~((1ull << (8 * e0)) - 1));
        const uint32_t klo = (uint32_t)keep, khi = (uint32_t)(keep >> 32);
#pragma unroll
        for (int j = 0; j < CacheTraits<kFp8>::kVVec; ++j) {
          cur.v[j][0] &= klo;
          cur.v[j][1] &= khi;
          cur.v[j][2] &= klo;
          cur.v[j][3] &= khi;
        }
      } else {
#pragma unroll
        for (int j = 0; j < CacheTraits<kFp8>::kVVec; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e < e0 || e >= e1) cur.v[j][e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
      }
    }
  }

  // ---- online softmax with a lazily raised reference maximum. The rescale is a cold,
  // wave-uniform branch per row tile, so it touches 32 accumulators at a time.
  const float C = cx.C;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float mx = fmaxf(fmaxf(fmaxf(sacc[0][t][0], sacc[0][t][1]), fmaxf(sacc[0][t][2], sacc[0][t][3])),
                           fmaxf(fmaxf(sacc[1][t][0], sacc[1][t][1]), fmaxf(sacc[1][t][2], sacc[1][t][3])));
    const float cand = group_max(mx) * C;
    const bool up = cand > st.m[t] + kLazyTau;
    // A row's first visible keys set its reference: its accumulators are still zero,
    // so only a raise of an existing finite reference needs the rescale.
    const bool rescale = up && st.m[t] != -INFINITY;
    if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
      const float alpha = rescale ? __builtin_amdgcn_exp2f(st.m[t] - cand) : 1.0f;
      st.lsum[t] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) st.o[t][dt] *= alpha;
    }
    st.m[t] = up ? cand : st.m[t];
  }

  if constexpr (kFp8) {
    f16x8_t P[NT];
    const uint32_t ones = 0x3C003C00u;  // (1.0h, 1.0h)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float ms = (st.m[t] == -INFINITY) ? 0.f : st.m[t];
      float p[2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[tt][i] = __builtin_amdgcn_exp2f(fmaf(sacc[tt][t][i], C, -ms));
      // Four separate packed words: with the words read back out of one vector the
      // dot products were emitted on the first word four times.
      const uint32_t h0 = pack_f16(p[0][0], p[0][1]), h1 = pack_f16(p[0][2], p[0][3]);
      const uint32_t h2 = pack_f16(p[1][0], p[1][1]), h3 = pack_f16(p[1][2], p[1][3]);
      P[t] = __builtin_bit_cast(f16x8_t, u32x4_t{h0, h1, h2, h3});
      // the row sum uses the same rounded probabilities the PV product sees
      const f16x2_t one2 = __builtin_bit_cast(f16x2_t, ones);
      float l = st.lsum[t];
      l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, h0), one2, l, false);
      l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, h1), one2, l, false);
      l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, h2), one2, l, false);
      l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, h3), one2, l, false);
      st.lsum[t] = l;
    }
    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const u32x4_t& v = cur.v[dt >> 1];
      const f16x8_t vf = fp8x8_to_f16x8(v[(dt & 1) * 2], v[(dt & 1) * 2 + 1]);
#pragma unroll
      for (int t = 0; t < NT; ++t) st.o[t][dt] = mfma_f16(vf, P[t], st.o[t][dt]);
    }
  } else {
    // BF16 cache: V stays BF16, so P is split into a BF16 head and a BF16 tail
    bf16x8_t Ph[NT], Pl[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float ms = (st.m[t] == -INFINITY) ? 0.f : st.m[t];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[tt][t][i], C, -ms));
          const __bf16 hi = (__bf16)p;
          Ph[t][4 * tt + i] = hi;
          Pl[t][4 * tt + i] = (__bf16)(p - (float)hi);
          st.lsum[t] += p;
        }
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, cur.v[dt]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        st.o[t][dt] = mfma_bf16(vf, Ph[t], st.o[t][dt]);
        st.o[t][dt] = mfma_bf16(vf, Pl[t], st.o[t][dt]);
      }
    }
  }
}

// Everything one wave does for its row group: rows of row tiles [T0, T0+NT), keys of
// tiles tb+kl, tb+kl+K, ... of the split, then the fixed-order merge with the other K-1
// key lanes of its group and the write of the final rows or of the split partial.
// Every wave of the work group executes the same barrier sequence.
// sm_m / sm_l: [K][NT*16] floats of this group; sm_o: [K/2][NT*8*64] f32x4 of this group.
template <int NT, int K, bool kFp8>
__device__ __forceinline__ void group_body(const DecodeArgs& a, const SplitCtx& cx, int T0, int kl,
                                           const u32x4_t* q_lds, float* sm_m, float* sm_l, f32x4_t* sm_o) {
  const int G = a.group, M = a.q_len, GM = G * M;
  const int n = cx.n, q = cx.q, lane = cx.lane;
  WaveState<NT> st;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int r = 16 * (T0 + t) + n;
    st.rpos[t] = (r < GM) ? cx.L - M + r / G : -1;
    st.m[t] = -INFINITY;
    st.lsum[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[t][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const u32x4_t* qg = q_lds + T0 * 4 * 64;

  // ---- this wave's tiles. One register set: the next tile's K is requested as soon as
  // the QK^T products have consumed the current K, its V once the PV products are done.
  // Loads are unconditional (past the end the last tile is fetched again, an invalid
  // page-table entry fetches block 0) so no stale copy stays live across a branch;
  // validity only decides whether a tile is computed.
  int tile = cx.tb + kl;
  if (tile < cx.te) {
    TileRegs<kFp8> cur;
    int blk = tile_block<kFp8>(a, cx.b, tile);
    bool ok = (unsigned)blk < (unsigned)a.num_blocks;
    blk = ok ? blk : 0;
    load_k<kFp8>(a, blk, cx.g, tile, n, q, cur);
    load_v<kFp8>(a, blk, cx.g, tile, n, q, cur);
    for (;;) {
      const int nxt = tile + K;
      const int nld = min(nxt, cx.te - 1);
      int nblk = tile_block<kFp8>(a, cx.b, nld);
      const bool nok = (unsigned)nblk < (unsigned)a.num_blocks;
      nblk = nok ? nblk : 0;
      f32x4_t sacc[2][NT];
      if (ok) qk_tile<NT, kFp8>(cur, qg, lane, sacc);
      load_k<kFp8>(a, nblk, cx.g, nld, n, q, cur);
      if (ok) softmax_pv_tile<NT, kFp8>(a, cx, st, cur, sacc, tile);
      load_v<kFp8>(a, nblk, cx.g, nld, n, q, cur);
      if (nxt >= cx.te) break;
      tile = nxt;
      ok = nok;
    }
  }

  // ---- merge the K key lanes of the group: common maximum, then a fixed-order tree sum
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float lt = group_sum(st.lsum[t]);
    if (q == 0) {
      sm_m[kl * NT * 16 + 16 * t + n] = st.m[t];
      sm_l[kl * NT * 16 + 16 * t + n] = lt;
    }
  }
  __syncthreads();  // every loop is done: the Q area may now be reused
  float Mw[NT], Lw[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float mm = -INFINITY;
#pragma unroll
    for (int u = 0; u < K; ++u) mm = fmaxf(mm, sm_m[u * NT * 16 + 16 * t + n]);
    float ll = 0.f;
#pragma unroll
    for (int u = 0; u < K; ++u) {
      const float mu = sm_m[u * NT * 16 + 16 * t + n];
      ll += (mu == -INFINITY) ? 0.f : sm_l[u * NT * 16 + 16 * t + n] * __builtin_amdgcn_exp2f(mu - mm);
    }
    Mw[t] = mm;
    Lw[t] = ll;
    const float alpha = (st.m[t] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.m[t] - mm);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[t][dt] *= alpha;
  }
  // tree: lanes [K/2, K) hand their sums to lanes [0, K/2), halving until lane 0 holds all
#pragma unroll
  for (int half = K / 2; half >= 1; half /= 2) {
    if (kl >= half && kl < 2 * half) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) sm_o[(kl - half) * NT * 8 * 64 + (t * 8 + dt) * 64 + lane] = st.o[t][dt];
    }
    __syncthreads();
    if (kl < half) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) st.o[t][dt] += sm_o[kl * NT * 8 * 64 + (t * 8 + dt) * 64 + lane];
    }
    if (half > 1) __syncthreads();
  }
  if (kl != 0) return;

  // ---- write: lane (n, q) owns row 16t+n, dimensions 32q .. 32q+31 (d = 32q + 8i + dt)
  const bool direct = (cx.nsplit == 1);
  const float vsc = kFp8 ? *a.v_scale : 1.0f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int r = 16 * (T0 + t) + n;
    if (r >= GM) continue;
    float* dst;
    float mul;
    if (direct) {
      const int i = r / G, h = cx.g * G + (r - i * G);
      dst = a.out + (((int64_t)cx.b * M + i) * a.num_q_heads + h) * kHeadDim + 32 * q;
      mul = Lw[t] > 0.f ? vsc / Lw[t] : 0.f;
    } else {
      const int64_t part = ((int64_t)cx.b * a.num_kv_heads + cx.g) * a.max_splits + cx.s;
      dst = a.ws_o + (part * a.rows_pad + r) * kHeadDim + 32 * q;
      mul = 1.0f;
      if (q == 0) {
        a.ws_ml[part * 2 * a.rows_pad + r] = Mw[t];
        a.ws_ml[part * 2 * a.rows_pad + a.rows_pad + r] = Lw[t];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<f32x4_t*>(dst + 8 * i) =
          f32x4_t{st.o[t][0][i], st.o[t][1][i], st.o[t][2][i], st.o[t][3][i]} * mul;
      *reinterpret_cast<f32x4_t*>(dst + 8 * i + 4) =
          f32x4_t{st.o[t][4][i], st.o[t][5][i], st.o[t][6][i], st.o[t][7][i]} * mul;
    }
  }
}

// Split kernel: R row groups x K key lanes = R*K waves. Group rg owns row tiles
// [rg*NTW, rg*NTW + NTW); lane kl of a group takes tiles tb+kl, tb+kl+K, ... The groups
// of one key lane read the same tiles, so with two waves per SIMD one wave's MFMA work
// overlaps another's softmax work; a single group of wide row tiles keeps every byte's
// conversion unique at one wave per SIMD.
template <int NTW, int R, int K>
struct SplitShape {
  static constexpr int kWavesPerGroup = K;
  static constexpr int kThreads = 64 * R * K;
  static constexpr int kRowTiles = NTW * R;
  static constexpr int kQBytes = kRowTiles * 4 * 64 * 16;
  static constexpr int kMergeBytes = R * (K / 2) * NTW * 8 * 64 * 16;
  static constexpr int kBigBytes = kQBytes > kMergeBytes ? kQBytes : kMergeBytes;
  static constexpr int kMinWavesPerEU = (R * K > 4 || NTW <= 2) ? 2 : 1;
};

template <int NTW, int R, int K, bool kFp8>
__global__ __launch_bounds__((SplitShape<NTW, R, K>::kThreads), (SplitShape<NTW, R, K>::kMinWavesPerEU))
void decode_split_kernel(DecodeArgs a) {
  typedef SplitShape<NTW, R, K> S;
  __shared__ __align__(16) unsigned char big[S::kBigBytes];  // Q staging, then merge buffers
  __shared__ float sm_ml[R * 2 * K * NTW * 16];
  u32x4_t* q_lds = reinterpret_cast<u32x4_t*>(big);

  SplitCtx cx;
  cx.s = blockIdx.x;
  cx.g = blockIdx.y;
  cx.b = blockIdx.z;
  cx.lane = threadIdx.x & 63;
  cx.n = cx.lane & 15;
  cx.q = cx.lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, uniform
  const int G = a.group, M = a.q_len, GM = G * M;
  const int wl = a.window_left;
  int L = a.seq_lens[cx.b];
  L = min(L, min(a.max_seq_len, a.max_blocks * a.block_size));
  cx.L = L;
  cx.lo_u = (wl < 0) ? 0 : max(0, L - M - wl);
  const int t_first = cx.lo_u / kTile;
  const int t_end = L > 0 ? (L + kTile - 1) / kTile : 0;
  const int ntiles = max(0, t_end - t_first);
  const int tps = a.tiles_per_split;
  cx.nsplit = (ntiles + tps - 1) / tps;

  if (ntiles == 0) {  // no visible key for any row: the rows are zeros
    if (cx.s == 0) {
      for (int idx = threadIdx.x; idx < GM * (kHeadDim / 4); idx += S::kThreads) {
        const int r = idx / (kHeadDim / 4), d4 = idx - r * (kHeadDim / 4);
        const int i = r / G, h = cx.g * G + (r - i * G);
        *reinterpret_cast<f32x4_t*>(a.out + (((int64_t)cx.b * M + i) * a.num_q_heads + h) * kHeadDim + 4 * d4) =
            f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    return;
  }
  if (cx.s >= cx.nsplit) return;
  cx.tb = t_first + cx.s * tps;
  cx.te = min(cx.tb + tps, t_end);
  cx.lo_max = (wl < 0) ? 0 : max(0, L - 1 - wl);  // largest row lower bound
  cx.p_min = L - M;                                // smallest row position
  cx.C = a.softmax_scale * (kFp8 ? *a.k_scale : 1.0f) * kLog2e;  // score -> log2 units

  // ---- Q fragments to LDS: fragment (t, c) of lane (n, q) is Q[row 16t+n][32q + 8c .. +7],
  // row r -> token r / G, head g*G + r % G
  for (int idx = threadIdx.x; idx < S::kRowTiles * 4 * 64; idx += S::kThreads) {
    const int t = idx >> 8, c = (idx >> 6) & 3, ln = idx & 63;
    const int r = 16 * t + (ln & 15);
    u32x4_t val{0u, 0u, 0u, 0u};
    if (r < GM) {
      const int i = r / G, h = cx.g * G + (r - i * G);
      val = *reinterpret_cast<const u32x4_t*>(a.q + (((int64_t)cx.b * M + i) * a.num_q_heads + h) * kHeadDim +
                                              32 * (ln >> 4) + 8 * c);
    }
    q_lds[idx] = val;
  }
  __syncthreads();

  const int rg = w / K, kl = w % K;
  group_body<NTW, K, kFp8>(a, cx, rg * NTW, kl, q_lds, sm_ml + rg * 2 * K * NTW * 16,
                           sm_ml + rg * 2 * K * NTW * 16 + K * NTW * 16,
                           reinterpret_cast<f32x4_t*>(big) + rg * (K / 2) * NTW * 8 * 64);
}

// ---------------------------------------------------------------------------------------
// LDS-pipelined split kernel (layout 1): R row groups of NTW <= 2 row tiles x K key lanes.
// Each step the group consumes K tiles (key lane kl takes tile tb + step*K + kl). Their
// K/V bytes arrive by global->LDS DMA into an S-stage ring, issued S-1 steps ahead and
// shared by the R row-group waves of each key lane; the bytes never occupy registers in
// flight. Every wave issues D = K*kChunks/(R*K) of the step's 16-byte-per-lane DMA
// chunks. Step protocol: wait for the wave's own chunks of this step (vmcnt), barrier
// (everyone's chunks landed, everyone finished the previous stage), refill the stage read
// in the previous step, read this step's fragments, compute.
// ---------------------------------------------------------------------------------------
template <bool kFp8>
struct DmaTraits {
  static constexpr int kChunks = kFp8 ? 8 : 16;           // 1 KB DMA chunks per 32-key tile
  static constexpr int kTileBytes = kChunks * 1024;
};

template <int NTW, int R, int K, bool kFp8>
struct DmaShape {
  static constexpr int kWaves = R * K;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kD = K * DmaTraits<kFp8>::kChunks / kWaves;     // chunks per wave per step
  static constexpr int kStageBytes = K * DmaTraits<kFp8>::kTileBytes;
  // ring depth: as deep as ~64-96 KB of LDS allows
  static constexpr int kStages = kStageBytes <= 16384 ? 4 : (kStageBytes <= 32768 ? (R * K > 4 ? 3 : 2) : 2);
  static constexpr int kRingBytes = kStages * kStageBytes;
  static constexpr int kMergeBytes = R * (K / 2) * NTW * 8 * 64 * 16;
  static constexpr int kMlFloats = R * 2 * K * NTW * 16;
  static constexpr int kHead = ((kMlFloats * 4 + 255) / 256) * 256;   // (m, l) first: no DMA targets address 0
  static constexpr int kBody = kRingBytes > kMergeBytes ? kRingBytes : kMergeBytes;
  static constexpr int kLdsBytes = kHead + kBody;
  // two waves per SIMD where two work groups' LDS fits in a CU, else one
  static constexpr int kMinWavesPerEU = (163840 / kLdsBytes) * kWaves >= 8 ? 2 : 1;
  static_assert(kD * kWaves == K * DmaTraits<kFp8>::kChunks, "chunks must split evenly over the waves");
};

// Per-lane byte offset of chunk j of a tile, relative to the tile's K slab (j < kChunks/2)
// or V group base (j >= kChunks/2): the same 16 bytes lane (n, q) loads in the register path.
template <bool kFp8>
__device__ __forceinline__ uint32_t chunk_lane_offset(int j, int n, int q) {
  constexpr int kHalf = DmaTraits<kFp8>::kChunks / 2;     // K chunks = V chunks
  constexpr int kEs = kFp8 ? 1 : 2;
  if (j < kHalf) {
    const int per_tt = kHalf / 2;                          // 2 (FP8) or 4 (BF16) 16-byte pieces
    const int tt = j / per_tt, piece = j % per_tt;
    const int key = 8 * (n >> 2) + 4 * tt + (n & 3);
    return (uint32_t)((key * kHeadDim + 32 * q) * kEs + 16 * piece);
  }
  const int jj = j - kHalf;
  return (uint32_t)((q * 8 * kHeadDim + 64 * n) * kEs + 16 * jj);
}

template <int NTW, int R, int K, bool kFp8>
__global__ __launch_bounds__((DmaShape<NTW, R, K, kFp8>::kThreads), (DmaShape<NTW, R, K, kFp8>::kMinWavesPerEU))
void decode_split_dma_kernel(DecodeArgs a) {
  typedef DmaShape<NTW, R, K, kFp8> S;
  typedef typename CacheTraits<kFp8>::elem_t elem_t;
  constexpr int kChunks = DmaTraits<kFp8>::kChunks;
  constexpr int kTileBytes = DmaTraits<kFp8>::kTileBytes;
  __shared__ __align__(256) unsigned char lds[S::kLdsBytes];
  float* sm_ml = reinterpret_cast<float*>(lds);
  unsigned char* body = lds + S::kHead;

  SplitCtx cx;
  cx.s = blockIdx.x;
  cx.g = blockIdx.y;
  cx.b = blockIdx.z;
  cx.lane = threadIdx.x & 63;
  cx.n = cx.lane & 15;
  cx.q = cx.lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.group, M = a.q_len, GM = G * M;
  const int wl = a.window_left;
  int L = a.seq_lens[cx.b];
  L = min(L, min(a.max_seq_len, a.max_blocks * a.block_size));
  cx.L = L;
  cx.lo_u = (wl < 0) ? 0 : max(0, L - M - wl);
  const int t_first = cx.lo_u / kTile;
  const int t_end = L > 0 ? (L + kTile - 1) / kTile : 0;
  const int ntiles = max(0, t_end - t_first);
  const int tps = a.tiles_per_split;
  cx.nsplit = (ntiles + tps - 1) / tps;
  if (ntiles == 0) {
    if (cx.s == 0) {
      for (int idx = threadIdx.x; idx < GM * (kHeadDim / 4); idx += S::kThreads) {
        const int r = idx / (kHeadDim / 4), d4 = idx - r * (kHeadDim / 4);
        const int i = r / G, h = cx.g * G + (r - i * G);
        *reinterpret_cast<f32x4_t*>(a.out + (((int64_t)cx.b * M + i) * a.num_q_heads + h) * kHeadDim + 4 * d4) =
            f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    return;
  }
  if (cx.s >= cx.nsplit) return;
  cx.tb = t_first + cx.s * tps;
  cx.te = min(cx.tb + tps, t_end);
  cx.lo_max = (wl < 0) ? 0 : max(0, L - 1 - wl);
  cx.p_min = L - M;
  cx.C = a.softmax_scale * (kFp8 ? *a.k_scale : 1.0f) * kLog2e;

  const int rg = w / K, kl = w % K;
  const int T0 = rg * NTW;
  const int n = cx.n, q = cx.q, lane = cx.lane;

  // ---- this wave's query rows, Q fragments in registers
  WaveState<NTW> st;
  bf16x8_t qreg[NTW][4];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int r = 16 * (T0 + t) + n;
    st.rpos[t] = (r < GM) ? L - M + r / G : -1;
    st.m[t] = -INFINITY;
    st.lsum[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[t][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (r < GM) {
      const int i = r / G, h = cx.g * G + (r - i * G);
      const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(
          a.q + (((int64_t)cx.b * M + i) * a.num_q_heads + h) * kHeadDim + 32 * q);
#pragma unroll
      for (int c = 0; c < 4; ++c) qreg[t][c] = __builtin_bit_cast(bf16x8_t, qp[c]);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) qreg[t][c] = __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
    }
  }

  // ---- the group's page-table window in two registers (entry e in lane e % 64), read with
  // readlane: the loop then issues no vector loads but the DMAs, whose counts the waits
  // below rely on. tiles_per_split <= 128 keeps the window within 128 entries.
  const int lb0 = (cx.tb * kTile) / a.block_size;
  const int nbw = ((cx.te - 1) * kTile) / a.block_size - lb0 + 1;
  const int32_t* btrow = a.block_table + (int64_t)cx.b * a.max_blocks + lb0;
  int bt_lo = lane < nbw ? btrow[lane] : 0;
  int bt_hi = lane + 64 < nbw ? btrow[lane + 64] : 0;
  // complete the two loads here, through an asm that redefines the registers: later reads
  // then carry no pending-load dependence that would make the compiler wait on the DMAs
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(bt_lo), "+v"(bt_hi)::"memory");
  auto block_of = [&](int tile) -> int {
    const int e = (tile * kTile) / a.block_size - lb0;
    return __builtin_amdgcn_readlane(e < 64 ? bt_lo : bt_hi, e & 63);
  };

  // ---- DMA plan of this wave: chunks c = w*D + d -> tile lane c / kChunks, chunk c % kChunks
  uint32_t dma_off[S::kD];
#pragma unroll
  for (int d = 0; d < S::kD; ++d) dma_off[d] = chunk_lane_offset<kFp8>((w * S::kD + d) % kChunks, n, q);
  const int nsteps = (cx.te - cx.tb + K - 1) / K;
  const int64_t slab_elems = (int64_t)a.block_size * kHeadDim;

  auto issue = [&](int step) {
    const int stage = step % S::kStages;
#pragma unroll
    for (int d = 0; d < S::kD; ++d) {
      const int c = w * S::kD + d;
      const int tl = c / kChunks, j = c % kChunks;
      const int tile = min(cx.tb + step * K + tl, cx.te - 1);
      int blk = block_of(tile);
      blk = ((unsigned)blk < (unsigned)a.num_blocks) ? blk : 0;
      const int o0 = (tile * kTile) % a.block_size;
      const int64_t slab = ((int64_t)blk * a.num_kv_heads + cx.g) * slab_elems + (int64_t)o0 * kHeadDim;
      const elem_t* base = reinterpret_cast<const elem_t*>(j < kChunks / 2 ? a.k_pool : a.v_pool) + slab;
      const unsigned char* src = reinterpret_cast<const unsigned char*>(base) + dma_off[d];
      unsigned char* dst = body + stage * S::kStageBytes + tl * kTileBytes + j * 1024;
      __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    }
  };

#pragma unroll
  for (int p = 0; p < S::kStages - 1; ++p)
    if (p < nsteps) issue(p);

  const uint32_t lds_lane = (uint32_t)(uintptr_t)(body + kl * kTileBytes) + 16u * (uint32_t)lane;
  for (int step = 0; step < nsteps; ++step) {
    // own chunks of this step done: later steps' chunks (up to S-2 steps) may stay in flight
    if (step + S::kStages - 2 < nsteps) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(S::kD * (S::kStages - 2)) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __builtin_amdgcn_s_barrier();
    if (step + S::kStages - 1 < nsteps) issue(step + S::kStages - 1);

    const int tile = cx.tb + step * K + kl;
    const uint32_t addr = lds_lane + (uint32_t)((step % S::kStages) * S::kStageBytes);
    TileRegs<kFp8> cur;
    if constexpr (kFp8) {
      asm volatile(
          "ds_read_b128 %0, %8 offset:0\n\t"
          "ds_read_b128 %1, %8 offset:1024\n\t"
          "ds_read_b128 %2, %8 offset:2048\n\t"
          "ds_read_b128 %3, %8 offset:3072\n\t"
          "ds_read_b128 %4, %8 offset:4096\n\t"
          "ds_read_b128 %5, %8 offset:5120\n\t"
          "ds_read_b128 %6, %8 offset:6144\n\t"
          "ds_read_b128 %7, %8 offset:7168\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(cur.k[0][0]), "=&v"(cur.k[0][1]), "=&v"(cur.k[1][0]), "=&v"(cur.k[1][1]), "=&v"(cur.v[0]),
            "=&v"(cur.v[1]), "=&v"(cur.v[2]), "=&v"(cur.v[3])
          : "v"(addr)
          : "memory");
    } else {
      asm volatile(
          "ds_read_b128 %0, %8 offset:0\n\t"
          "ds_read_b128 %1, %8 offset:1024\n\t"
          "ds_read_b128 %2, %8 offset:2048\n\t"
          "ds_read_b128 %3, %8 offset:3072\n\t"
          "ds_read_b128 %4, %8 offset:4096\n\t"
          "ds_read_b128 %5, %8 offset:5120\n\t"
          "ds_read_b128 %6, %8 offset:6144\n\t"
          "ds_read_b128 %7, %8 offset:7168\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(cur.k[0][0]), "=&v"(cur.k[0][1]), "=&v"(cur.k[0][2]), "=&v"(cur.k[0][3]), "=&v"(cur.k[1][0]),
            "=&v"(cur.k[1][1]), "=&v"(cur.k[1][2]), "=&v"(cur.k[1][3])
          : "v"(addr)
          : "memory");
      asm volatile(
          "ds_read_b128 %0, %8 offset:8192\n\t"
          "ds_read_b128 %1, %8 offset:9216\n\t"
          "ds_read_b128 %2, %8 offset:10240\n\t"
          "ds_read_b128 %3, %8 offset:11264\n\t"
          "ds_read_b128 %4, %8 offset:12288\n\t"
          "ds_read_b128 %5, %8 offset:13312\n\t"
          "ds_read_b128 %6, %8 offset:14336\n\t"
          "ds_read_b128 %7, %8 offset:15360\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(cur.v[0]), "=&v"(cur.v[1]), "=&v"(cur.v[2]), "=&v"(cur.v[3]), "=&v"(cur.v[4]), "=&v"(cur.v[5]),
            "=&v"(cur.v[6]), "=&v"(cur.v[7])
          : "v"(addr)
          : "memory");
    }
    if (tile < cx.te) {
      const int blk = block_of(tile);
      if ((unsigned)blk < (unsigned)a.num_blocks) {
        f32x4_t sacc[2][NTW];
#pragma unroll
        for (int t = 0; t < NTW; ++t) sacc[0][t] = sacc[1][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          bf16x8_t kf0, kf1;
          if constexpr (kFp8) {
            const u32x4_t& v0 = cur.k[0][c >> 1];
            const u32x4_t& v1 = cur.k[1][c >> 1];
            kf0 = fp8x8_to_bf16x8(v0[(c & 1) * 2], v0[(c & 1) * 2 + 1]);
            kf1 = fp8x8_to_bf16x8(v1[(c & 1) * 2], v1[(c & 1) * 2 + 1]);
          } else {
            kf0 = __builtin_bit_cast(bf16x8_t, cur.k[0][c]);
            kf1 = __builtin_bit_cast(bf16x8_t, cur.k[1][c]);
          }
#pragma unroll
          for (int t = 0; t < NTW; ++t) {
            sacc[0][t] = mfma_bf16(kf0, qreg[t][c], sacc[0][t]);
            sacc[1][t] = mfma_bf16(kf1, qreg[t][c], sacc[1][t]);
          }
        }
        softmax_pv_tile<NTW, kFp8>(a, cx, st, cur, sacc, tile);
      }
    }
  }
  // every chunk (including clamped tail refills) has landed before LDS is reused
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // ---- merge the K key lanes of the row group (fixed-order tree), then write
  float* sm_m = sm_ml + rg * 2 * K * NTW * 16;
  float* sm_l = sm_m + K * NTW * 16;
  f32x4_t* sm_o = reinterpret_cast<f32x4_t*>(body) + rg * (K / 2) * NTW * 8 * 64;
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const float lt = group_sum(st.lsum[t]);
    if (q == 0) {
      sm_m[kl * NTW * 16 + 16 * t + n] = st.m[t];
      sm_l[kl * NTW * 16 + 16 * t + n] = lt;
    }
  }
  __syncthreads();
  float Mw[NTW], Lw[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    float mm = -INFINITY;
#pragma unroll
    for (int u = 0; u < K; ++u) mm = fmaxf(mm, sm_m[u * NTW * 16 + 16 * t + n]);
    float ll = 0.f;
#pragma unroll
    for (int u = 0; u < K; ++u) {
      const float mu = sm_m[u * NTW * 16 + 16 * t + n];
      ll += (mu == -INFINITY) ? 0.f : sm_l[u * NTW * 16 + 16 * t + n] * __builtin_amdgcn_exp2f(mu - mm);
    }
    Mw[t] = mm;
    Lw[t] = ll;
    const float alpha = (st.m[t] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.m[t] - mm);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[t][dt] *= alpha;
  }
#pragma unroll
  for (int half = K / 2; half >= 1; half /= 2) {
    if (kl >= half && kl < 2 * half) {
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) sm_o[(kl - half) * NTW * 8 * 64 + (t * 8 + dt) * 64 + lane] = st.o[t][dt];
    }
    __syncthreads();
    if (kl < half) {
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) st.o[t][dt] += sm_o[kl * NTW * 8 * 64 + (t * 8 + dt) * 64 + lane];
    }
    if (half > 1) __syncthreads();
  }
  if (kl != 0) return;
  const bool direct = (cx.nsplit == 1);
  const float vsc = kFp8 ? *a.v_scale : 1.0f;
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int r = 16 * (T0 + t) + n;
    if (r >= GM) continue;
    float* dst;
    float mul;
    if (direct) {
      const int i = r / G, h = cx.g * G + (r - i * G);
      dst = a.out + (((int64_t)cx.b * M + i) * a.num_q_heads + h) * kHeadDim + 32 * q;
      mul = Lw[t] > 0.f ? vsc / Lw[t] : 0.f;
    } else {
      const int64_t part = ((int64_t)cx.b * a.num_kv_heads + cx.g) * a.max_splits + cx.s;
      dst = a.ws_o + (part * a.rows_pad + r) * kHeadDim + 32 * q;
      mul = 1.0f;
      if (q == 0) {
        a.ws_ml[part * 2 * a.rows_pad + r] = Mw[t];
        a.ws_ml[part * 2 * a.rows_pad + a.rows_pad + r] = Lw[t];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<f32x4_t*>(dst + 8 * i) =
          f32x4_t{st.o[t][0][i], st.o[t][1][i], st.o[t][2][i], st.o[t][3][i]} * mul;
      *reinterpret_cast<f32x4_t*>(dst + 8 * i + 4) =
          f32x4_t{st.o[t][4][i], st.o[t][5][i], st.o[t][6][i], st.o[t][7][i]} * mul;
    }
  }
}

// Merges the split partials of each (sequence, KV head) row in split order:
// out = v_scale * sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// A thread owns 4 dimensions of one row; a group of 128 threads holds 4 rows. Splits are
// taken 8 at a time: the 8 partials' (m, l) and output pieces are all requested before
// any is used (one memory round trip per 8 splits), then folded in split order into a
// running maximum, row sum and output (the same order for every call).
constexpr int kCombineRows = 4;
constexpr int kCombineChunk = 8;

__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a, int kfp8) {
  const int b = blockIdx.z, g = blockIdx.y;
  const int G = a.group, M = a.q_len, GM = G * M;
  const int wl = a.window_left;
  int L = a.seq_lens[b];
  L = min(L, min(a.max_seq_len, a.max_blocks * a.block_size));
  const int lo_u = (wl < 0) ? 0 : max(0, L - M - wl);
  const int t_first = lo_u / kTile;
  const int t_end = L > 0 ? (L + kTile - 1) / kTile : 0;
  const int ntiles = max(0, t_end - t_first);
  const int nsplit = (ntiles + a.tiles_per_split - 1) / a.tiles_per_split;
  if (nsplit <= 1) return;
  const int r = blockIdx.x * kCombineRows + (threadIdx.x >> 5);
  const int d4 = threadIdx.x & 31;
  if (r >= GM) return;
  const int64_t base = ((int64_t)b * a.num_kv_heads + g) * a.max_splits;
  const int64_t ml_stride = 2 * (int64_t)a.rows_pad;
  const int64_t o_stride = (int64_t)a.rows_pad * kHeadDim;
  const float* mlp = a.ws_ml + base * ml_stride + r;
  const float* op = a.ws_o + (base * a.rows_pad + r) * kHeadDim + 4 * d4;

  float mrun = -INFINITY, lrun = 0.f;
  f32x4_t acc{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += kCombineChunk) {
    float ms[kCombineChunk], ls[kCombineChunk];
    f32x4_t os[kCombineChunk];
#pragma unroll
    for (int j = 0; j < kCombineChunk; ++j) {
      const int sj = min(s0 + j, nsplit - 1);  // clamped: in-range loads, unused past the end
      ms[j] = mlp[sj * ml_stride];
      ls[j] = mlp[sj * ml_stride + a.rows_pad];
      os[j] = *reinterpret_cast<const f32x4_t*>(op + sj * o_stride);
    }
    float mc = mrun;
#pragma unroll
    for (int j = 0; j < kCombineChunk; ++j)
      if (s0 + j < nsplit) mc = fmaxf(mc, ms[j]);
    // rescale what has been folded so far to the new maximum, then fold this chunk in order
    const float keep = (mrun == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mrun - mc);
    lrun *= keep;
    acc *= keep;
#pragma unroll
    for (int j = 0; j < kCombineChunk; ++j) {
      if (s0 + j < nsplit) {
        const float wgt = (ms[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms[j] - mc);
        lrun += wgt * ls[j];
        acc += os[j] * wgt;
      }
    }
    mrun = mc;
  }
  const float vsc = kfp8 ? *a.v_scale : 1.0f;
  const float mul = lrun > 0.f ? vsc / lrun : 0.f;
  const int i = r / G, h = g * G + (r - i * G);
  store_out4(a.out, a.out_bf16, (((int64_t)b * M + i) * a.num_q_heads + h) * kHeadDim + 4 * d4, acc * mul);
}

template <int NTW, int R, int K, bool kFp8>
static hipError_t launch_split(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<NTW, R, K, kFp8>), dim3(a.max_splits, a.num_kv_heads, a.num_seqs),
                     dim3(SplitShape<NTW, R, K>::kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int NTW, int R, int K, bool kFp8>
static hipError_t launch_split_dma(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_dma_kernel<NTW, R, K, kFp8>), dim3(a.max_splits, a.num_kv_heads, a.num_seqs),
                     dim3(DmaShape<NTW, R, K, kFp8>::kThreads), 0, stream, a);
  return hipGetLastError();
}

template <bool kFp8>
static hipError_t dispatch_split(const DecodeArgs& a, const SplitShapeInfo& sh, hipStream_t stream) {
  const int key = sh.ntw * 100 + sh.r * 10 + sh.k;
  switch (key) {
    case 114: return launch_split_dma<1, 1, 4, kFp8>(a, stream);
    case 214: return launch_split_dma<2, 1, 4, kFp8>(a, stream);
    case 224: return launch_split_dma<2, 2, 4, kFp8>(a, stream);
    case 242: return launch_split_dma<2, 4, 2, kFp8>(a, stream);
    case 314: return launch_split<3, 1, 4, kFp8>(a, stream);
    case 414: return launch_split<4, 1, 4, kFp8>(a, stream);
    case 514: return launch_split<5, 1, 4, kFp8>(a, stream);
    case 614: return launch_split<6, 1, 4, kFp8>(a, stream);
    case 714: return launch_split<7, 1, 4, kFp8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine(const DecodeArgs& a, bool fp8, hipStream_t stream) {
  const int rows = a.group * a.q_len;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((rows + kCombineRows - 1) / kCombineRows, a.num_kv_heads, a.num_seqs),
                     dim3(32 * kCombineRows), 0, stream, a, fp8 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, const SplitShapeInfo& shape, bool fp8, hipStream_t stream,
                         bool* launched_combine) {
  *launched_combine = false;
  if (a.num_seqs == 0) return hipSuccess;
  hipError_t e;
  if (shape.groups_per_cu == 0) {
    e = launch_rows(a, shape.ntw, fp8, stream);
  } else if (shape.groups_per_cu == -2 || shape.groups_per_cu == -3) {
    // row tiles per work group (rows_pad / 32 row tiles in row_groups groups); layout 6 holds
    // two row tiles per wave
    e = launch_m32(a, a.rows_pad / 32 / a.row_groups, shape.groups_per_cu == -3 ? 2 : 1, a.key_lanes, fp8, stream);
  } else if (shape.groups_per_cu < 0) {
    e = launch_wide(a, shape.ntw, fp8, stream);
  } else {
    e = fp8 ? dispatch_split<true>(a, shape, stream) : dispatch_split<false>(a, shape, stream);
  }
  if (e != hipSuccess) return e;
  if (a.max_splits > 1 && !a.fused_combine) {
    e = shape.groups_per_cu == -1 ? launch_combine_lanes(a, fp8, stream) : launch_combine(a, fp8, stream);
    *launched_combine = true;
  }
  return e;
}

}  // namespace fkv
