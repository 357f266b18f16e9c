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

// Loads one 32-key tile's K and V fragments for this lane. Returns false (and loads
// nothing) when the page table entry is outside the pool.
template <bool kFp8>
__device__ __forceinline__ bool load_tile(const DecodeArgs& a, int b, int g, int tile, int n, int q,
                                          TileRegs<kFp8>& r) {
  typedef typename CacheTraits<kFp8>::elem_t elem_t;
  const int kt = tile * kTile;
  const int lb = kt / a.block_size;
  const int o0 = kt - lb * a.block_size;
  const int blk = a.block_table[(int64_t)b * a.max_blocks + lb];
  if ((unsigned)blk >= (unsigned)a.num_blocks) return false;
  const int64_t slab = ((int64_t)blk * a.num_kv_heads + g) * (int64_t)a.block_size * kHeadDim;
  const elem_t* kb = reinterpret_cast<const elem_t*>(a.k_pool) + slab + (int64_t)o0 * kHeadDim + 32 * q;
  const elem_t* vb = reinterpret_cast<const elem_t*>(a.v_pool) + slab + (o0 >> 3) * (8 * kHeadDim) +
                     q * (8 * kHeadDim) + 64 * n;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int kk = 8 * (n >> 2) + 4 * tt + (n & 3);
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(kb + kk * kHeadDim);
#pragma unroll
    for (int j = 0; j < CacheTraits<kFp8>::kKVec; ++j) r.k[tt][j] = p[j];
  }
  const u32x4_t* pv = reinterpret_cast<const u32x4_t*>(vb);
#pragma unroll
  for (int j = 0; j < CacheTraits<kFp8>::kVVec; ++j) r.v[j] = pv[j];
  return true;
}

// Per-wave state of the split kernel.
template <int NT>
struct WaveState {
  f32x4_t o[NT][8];  // O^T accumulators: row tile t, d-tile dt
  float m[NT];       // reference maximum per row (log2 units), -inf before any key
  float lsum[NT];    // this lane's share of the row sum
  int rpos[NT];      // absolute position of the lane's row in tile t (-1: padding row)
};

template <int NT, bool kFp8, bool kQInLds>
__device__ __forceinline__ void attend_tile(const DecodeArgs& a, WaveState<NT>& st, TileRegs<kFp8>& cur,
                                            const bf16x8_t (&qreg)[kQInLds ? 1 : NT][4], const u32x4_t* q_lds,
                                            int tile, int lane, int q, int lo_u, int lo_max, int p_min, int L,
                                            float C) {
  const int kt = tile * kTile;
  const bool interior = (kt >= lo_max) && (kt + kTile - 1 <= p_min);
  const int wl = a.window_left;

  // ---- S^T = K Q^T for both 16-key halves; each Q fragment feeds two products
  f32x4_t sacc[2][NT];
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
      bf16x8_t qf;
      if constexpr (kQInLds)
        qf = __builtin_bit_cast(bf16x8_t, q_lds[(t * 4 + c) * 64 + lane]);
      else
        qf = qreg[t][c];
      sacc[0][t] = mfma_bf16(kf0, qf, sacc[0][t]);
      sacc[1][t] = mfma_bf16(kf1, qf, sacc[1][t]);
    }
  }

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
    const int e0 = min(8, max(0, lo_u - (kt + 8 * q)));
    const int e1 = min(8, max(0, L - (kt + 8 * q)));
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
      const uint32_t h0 = pack_f16_rtz(p[0][0], p[0][1]), h1 = pack_f16_rtz(p[0][2], p[0][3]);
      const uint32_t h2 = pack_f16_rtz(p[1][0], p[1][1]), h3 = pack_f16_rtz(p[1][2], p[1][3]);
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

template <int NT, bool kFp8>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr bool kQInLds = NT > 2;  // wide row packings keep Q in LDS to free registers
  __shared__ float sm_m[kWaves][NT * 16];
  __shared__ float sm_l[kWaves][NT * 16];
  __shared__ f32x4_t sm_o[2][NT * 8 * 64];
  __shared__ u32x4_t q_lds[kQInLds ? NT * 4 * 64 : 1];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, uniform
  const int n = lane & 15, q = lane >> 4;
  const int G = a.group, M = a.q_len, GM = G * M;
  const int wl = a.window_left;
  int L = a.seq_lens[b];
  L = min(L, min(a.max_seq_len, a.max_blocks * a.block_size));
  const int lo_u = (wl < 0) ? 0 : max(0, L - M - wl);
  const int t_first = lo_u / kTile;
  const int t_end = L > 0 ? (L + kTile - 1) / kTile : 0;
  const int ntiles = max(0, t_end - t_first);
  const int tps = a.tiles_per_split;
  const int nsplit = (ntiles + tps - 1) / tps;

  if (ntiles == 0) {  // no visible key for any row: the rows are zeros
    if (s == 0) {
      for (int idx = threadIdx.x; idx < GM * (kHeadDim / 4); idx += 256) {
        const int r = idx / (kHeadDim / 4), d4 = idx - r * (kHeadDim / 4);
        const int i = r / G, h = g * G + (r - i * G);
        *reinterpret_cast<f32x4_t*>(a.out + (((int64_t)b * M + i) * a.num_q_heads + h) * kHeadDim + 4 * d4) =
            f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    return;
  }
  if (s >= nsplit) return;
  const int tb = t_first + s * tps;
  const int te = min(tb + tps, t_end);
  const int lo_max = (wl < 0) ? 0 : max(0, L - 1 - wl);  // largest row lower bound
  const int p_min = L - M;                                // smallest row position

  // ---- query rows: row r = 16*t + n -> token i = r / G, head g*G + r % G.
  // Fragment (t, c) of lane (n, q) is Q[row 16t+n][32q + 8c .. +7].
  WaveState<NT> st;
  bf16x8_t qreg[kQInLds ? 1 : NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int r = 16 * t + n;
    st.rpos[t] = (r < GM) ? L - M + r / G : -1;
    st.m[t] = -INFINITY;
    st.lsum[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[t][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (kQInLds) {
    for (int idx = threadIdx.x; idx < NT * 4 * 64; idx += 256) {
      const int t = idx >> 8, c = (idx >> 6) & 3, ln = idx & 63;
      const int r = 16 * t + (ln & 15);
      u32x4_t val{0u, 0u, 0u, 0u};
      if (r < GM) {
        const int i = r / G, h = g * G + (r - i * G);
        val = *reinterpret_cast<const u32x4_t*>(a.q + (((int64_t)b * M + i) * a.num_q_heads + h) * kHeadDim +
                                                32 * (ln >> 4) + 8 * c);
      }
      q_lds[idx] = val;
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int r = 16 * t + n;
      if (r < GM) {
        const int i = r / G, h = g * G + (r - i * G);
        const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(
            a.q + (((int64_t)b * M + i) * a.num_q_heads + h) * kHeadDim + 32 * q);
#pragma unroll
        for (int c = 0; c < 4; ++c) qreg[t][c] = __builtin_bit_cast(bf16x8_t, qp[c]);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) qreg[t][c] = __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
      }
    }
  }

  const float C = a.softmax_scale * (kFp8 ? *a.k_scale : 1.0f) * kLog2e;  // score -> log2 units

  // ---- tiles of this wave, double-buffered: the next tile's loads fly during the current one
  TileRegs<kFp8> ra = {}, rb = {};
  int tile = tb + w;
  bool ok_a = tile < te ? load_tile<kFp8>(a, b, g, tile, n, q, ra) : false;
  bool ok_b = false;
  while (tile < te) {
    if (tile + kWaves < te) ok_b = load_tile<kFp8>(a, b, g, tile + kWaves, n, q, rb);
    if (ok_a) attend_tile<NT, kFp8, kQInLds>(a, st, ra, qreg, q_lds, tile, lane, q, lo_u, lo_max, p_min, L, C);
    tile += kWaves;
    if (tile >= te) break;
    if (tile + kWaves < te) ok_a = load_tile<kFp8>(a, b, g, tile + kWaves, n, q, ra);
    if (ok_b) attend_tile<NT, kFp8, kQInLds>(a, st, rb, qreg, q_lds, tile, lane, q, lo_u, lo_max, p_min, L, C);
    tile += kWaves;
  }

  // ---- merge the 4 waves of the group: common maximum, then a fixed-order tree sum
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float lt = group_sum(st.lsum[t]);
    if (q == 0) {
      sm_m[w][16 * t + n] = st.m[t];
      sm_l[w][16 * t + n] = lt;
    }
  }
  __syncthreads();
  float Mw[NT], Lw[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float mm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) mm = fmaxf(mm, sm_m[u][16 * t + n]);
    float ll = 0.f;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) {
      const float mu = sm_m[u][16 * t + n];
      ll += (mu == -INFINITY) ? 0.f : sm_l[u][16 * t + n] * __builtin_amdgcn_exp2f(mu - mm);
    }
    Mw[t] = mm;
    Lw[t] = ll;
    const float alpha = (st.m[t] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.m[t] - mm);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[t][dt] *= alpha;
  }
  if (w >= 2) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) sm_o[w - 2][(t * 8 + dt) * 64 + lane] = st.o[t][dt];
  }
  __syncthreads();
  if (w < 2) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) st.o[t][dt] += sm_o[w][(t * 8 + dt) * 64 + lane];
  }
  __syncthreads();
  if (w == 1) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) sm_o[0][(t * 8 + dt) * 64 + lane] = st.o[t][dt];
  }
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[t][dt] += sm_o[0][(t * 8 + dt) * 64 + lane];

  // ---- write: lane (n, q) owns row 16t+n, dimensions 32q .. 32q+31 (d = 32q + 8i + dt)
  const bool direct = (nsplit == 1);
  const float vsc = kFp8 ? *a.v_scale : 1.0f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int r = 16 * t + n;
    if (r >= GM) continue;
    float* dst;
    float mul;
    if (direct) {
      const int i = r / G, h = g * G + (r - i * G);
      dst = a.out + (((int64_t)b * M + i) * a.num_q_heads + h) * kHeadDim + 32 * q;
      mul = Lw[t] > 0.f ? vsc / Lw[t] : 0.f;
    } else {
      const int64_t part = ((int64_t)b * a.num_kv_heads + g) * a.max_splits + s;
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
// A group handles 8 rows; the (m, l) of all splits are staged in LDS first, so the
// partial-output loads of the accumulation loop are independent of each other.
constexpr int kCombineRows = 8;

__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a, int kfp8) {
  __shared__ float w_s[kCombineRows][kMaxSplits];
  __shared__ float l_tot[kCombineRows];
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
  const int64_t base = ((int64_t)b * a.num_kv_heads + g) * a.max_splits;
  const int r0 = blockIdx.x * kCombineRows;
  const int lane = threadIdx.x & 31, rr = threadIdx.x >> 5;  // 8 rows x 32 lanes

  // pass 1: row r0+rr's maximum over splits, then its weights 2^(m_s - M) and total l
  if (r0 + rr < GM) {
    float mx = -INFINITY;
    for (int s2 = lane; s2 < nsplit; s2 += 32) mx = fmaxf(mx, a.ws_ml[(base + s2) * 2 * a.rows_pad + r0 + rr]);
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 32));
    float lsum = 0.f;
    for (int s2 = lane; s2 < nsplit; s2 += 32) {
      const float* ml = a.ws_ml + (base + s2) * 2 * a.rows_pad;
      const float ms = ml[r0 + rr];
      const float wgt = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - mx);
      w_s[rr][s2] = wgt;
      lsum += wgt * ml[a.rows_pad + r0 + rr];
    }
    // fixed-shape butterfly: the same order for every call
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off, 32);
    if (lane == 0) l_tot[rr] = lsum;
  }
  __syncthreads();
  const int r = r0 + rr;
  if (r >= GM) return;
  // pass 2: lane owns 4 dimensions; split loads are independent and unrolled
  const float* src = a.ws_o + (base * a.rows_pad + r) * kHeadDim + 4 * lane;
  const int64_t stride = (int64_t)a.rows_pad * kHeadDim;
  f32x4_t acc{0.f, 0.f, 0.f, 0.f};
  int s2 = 0;
  for (; s2 + 4 <= nsplit; s2 += 4) {
    const f32x4_t o0 = *reinterpret_cast<const f32x4_t*>(src + (s2 + 0) * stride);
    const f32x4_t o1 = *reinterpret_cast<const f32x4_t*>(src + (s2 + 1) * stride);
    const f32x4_t o2 = *reinterpret_cast<const f32x4_t*>(src + (s2 + 2) * stride);
    const f32x4_t o3 = *reinterpret_cast<const f32x4_t*>(src + (s2 + 3) * stride);
    acc += o0 * w_s[rr][s2] + o1 * w_s[rr][s2 + 1] + o2 * w_s[rr][s2 + 2] + o3 * w_s[rr][s2 + 3];
  }
  for (; s2 < nsplit; ++s2) acc += *reinterpret_cast<const f32x4_t*>(src + s2 * stride) * w_s[rr][s2];
  const float vsc = kfp8 ? *a.v_scale : 1.0f;
  const float lt = l_tot[rr];
  const float mul = lt > 0.f ? vsc / lt : 0.f;
  const int i = r / G, h = g * G + (r - i * G);
  *reinterpret_cast<f32x4_t*>(a.out + (((int64_t)b * M + i) * a.num_q_heads + h) * kHeadDim + 4 * lane) = acc * mul;
}

template <int NT, bool kFp8>
static hipError_t launch_split(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<NT, kFp8>), dim3(a.max_splits, a.num_kv_heads, a.num_seqs), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

template <bool kFp8>
static hipError_t dispatch_split(const DecodeArgs& a, int nt, hipStream_t stream) {
  switch (nt) {
    case 1: return launch_split<1, kFp8>(a, stream);
    case 2: return launch_split<2, kFp8>(a, stream);
    case 3: return launch_split<3, kFp8>(a, stream);
    case 4: return launch_split<4, kFp8>(a, stream);
    case 5: return launch_split<5, kFp8>(a, stream);
    case 6: return launch_split<6, kFp8>(a, stream);
    case 7: return launch_split<7, kFp8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs& a, int nt, bool fp8, hipStream_t stream, bool* launched_combine) {
  *launched_combine = false;
  if (a.num_seqs == 0) return hipSuccess;
  hipError_t e = fp8 ? dispatch_split<true>(a, nt, stream) : dispatch_split<false>(a, nt, stream);
  if (e != hipSuccess) return e;
  if (a.max_splits > 1) {
    const int rows = a.group * a.q_len;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((rows + kCombineRows - 1) / kCombineRows, a.num_kv_heads, a.num_seqs),
                       dim3(256), 0, stream, a, fp8 ? 1 : 0);
    e = hipGetLastError();
    *launched_combine = true;
  }
  return e;
}

}  // namespace fkv
