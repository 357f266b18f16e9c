// Paged GQA decode attention, row-group split kernel.
//
// Operation: exact q1 / M12 paged attention over the calibrated FP8 cache ("Laguna S 2.1
// INT4 -- calibrated FP8 KV on Intel B70", sections Contract and "Initial optimization
// order"; q=18 / kv=2, head 128, global and sliding windows in "Laguna FP8 KV --
// replicated embedding win, page-32 build, and host boundary", section "Page-32
// attention experiment").
//
// Work decomposition. The G*M query rows of a KV head (G = Hq/Hkv heads x M tokens) are
// packed into 16-row tiles and cut into row groups of NTW tiles. One work group takes one
// (sequence, KV head, split, row group): the split's 32-key tiles, for the group's rows.
//   * The row groups of one (sequence, KV head, split) are launched on the same XCD
//     (work group ids congruent mod 8), so the second and later readers of a K/V tile
//     hit that XCD's L2 instead of HBM.
//   * Each of the K waves streams its own tiles (tb + kl, tb + kl + K, ...) through a
//     private two-slot LDS ring filled by global_load_lds: a tile is requested two tiles
//     ahead of its use, the registers only hold the tile being computed, and no wave
//     waits for another inside the loop.
//   * S^T = K Q^T on MFMA 16x16x32 bf16 (fp8 -> bf16 exact), online softmax in the log2
//     domain with a lazily raised reference maximum, O^T += V^T P^T on MFMA 16x16x32 f16
//     (fp8 -> f16 exact, P in f16).
//   * After the loop the K waves merge in LDS in a fixed order and the group writes its
//     rows: final rows when the sequence has one split, else an fp32 partial (m, l, O)
//     that decode_combine_kernel merges over splits in split order.
//
// Lane layout (lane l = 16*q + n): the K rows fed to the two 16-key halves of a tile are
// permuted (lane (n, q) feeds key 8*(n/4) + 4*tt + n%4) so that score lane (n, q) holds
// keys 8q .. 8q+7 of query row n, which is the P^T operand slice of the PV product; V is
// stored with each 8-key group dimension-major, so lane (n, q) reads dimensions 8n .. 8n+7
// of keys 8q .. 8q+7 as 64 contiguous bytes. Head dimensions are permuted the same way in
// Q and K (lane group q owns d = 32q .. 32q+31); an output lane holds row n, dimensions
// 32q + 8i + dt for accumulator element i of d-tile dt.
#include "fkv_device.h"
#include "fkv_internal.h"
#include "fkv_tile.h"

namespace fkv {

namespace {

template <int NTW, int K, bool kFp8>
struct RowsShape {
  static constexpr int kThreads = 64 * K;
  static constexpr int kRows = 16 * NTW;                       // rows of one group
  static constexpr int kMl = (2 * K + 2) * kRows * 4;          // (m, l) of every wave's rows; merged (M, L)
  static constexpr int kHead = ((kMl + 255) / 256) * 256;      // first: no DMA targets address 0
  static constexpr int kStride = kHeadDim + 4;                 // padded row: no LDS bank conflicts
  static constexpr int kStage = kRows * kStride * 4;           // merged rows, row-major fp32
  static constexpr int kRing = K * 2 * TileGeom<kFp8>::kBytes; // per-wave two-slot rings
  static constexpr int kMerge = K * NTW * 8 * 64 * 16;         // every wave's scaled O (lane layout)
  static constexpr int kBody = kRing > kMerge ? kRing : kMerge;
  static constexpr int kLds = kHead + kStage + kBody;
  static_assert(kLds <= 160 * 1024, "LDS budget of one CU");
  static_assert(8 % K == 0 || K % 8 == 0, "d-tiles split evenly over the waves");
};

}  // namespace

template <int NTW, int K, bool kFp8, bool kEarly>
__global__ __launch_bounds__((RowsShape<NTW, K, kFp8>::kThreads), (K >= 8 ? 2 : 1))
void decode_rows_kernel(DecodeArgs a) {
  typedef RowsShape<NTW, K, kFp8> S;
  typedef TileGeom<kFp8> T;
  __shared__ __align__(256) unsigned char lds[S::kLds];
  float* sm_m = reinterpret_cast<float*>(lds);        // [K][kRows]
  float* sm_l = sm_m + K * S::kRows;                  // [K][kRows]
  float* sm_row = sm_l + K * S::kRows;                // [2][kRows]: merged maximum and row sum
  float* stage = reinterpret_cast<float*>(lds + S::kHead);
  unsigned char* body = lds + S::kHead + S::kStage;

  // ---- which (sequence, KV head, split, row group): row groups of a unit share an XCD
  const int RG = a.row_groups;
  const int wg = blockIdx.x;
  int rg, s, bg;
  if (a.xcd_pairs) {
    // every work group of a (sequence, KV head) pair on one XCD (ids congruent mod 8): its
    // row groups share the K/V tiles through that XCD's L2
    const int per = a.max_splits * RG, slot = wg / 8;
    bg = (slot / per) * 8 + (wg % 8);
    s = (slot % per) / RG;
    rg = (slot % per) % RG;
  } else {
    // the row groups of a (sequence, KV head, split) on one XCD
    rg = (wg % (8 * RG)) / 8;
    const int unit = (wg / (8 * RG)) * 8 + (wg % 8);
    s = unit % a.max_splits;
    bg = unit / a.max_splits;
  }
  if (bg >= a.num_seqs * a.num_kv_heads) return;
  const int g = bg % a.num_kv_heads, b = bg / a.num_kv_heads;

  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const int kl = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.group, M = a.q_len, GM = G * M;
  const int wl = a.window_left;
  const int R0 = rg * S::kRows;  // first packed row of the group
  const int bshift = a.block_size == 64 ? 1 : 0;  // tiles per page: 1 (page 32) or 2 (page 64)

  // Page-table window of the split, requested together with the sequence length for
  // global attention (the split's first tile does not depend on it).
  const int tps = a.tiles_per_split;
  const int32_t* btrow = a.block_table + (int64_t)b * a.max_blocks;
  int bt_lo = 0, bt_hi = 0;
  int lb0 = 0;
  if (wl < 0) {
    lb0 = (s * tps) >> bshift;
    if (lb0 + lane < a.max_blocks) bt_lo = btrow[lb0 + lane];
    if (lb0 + lane + 64 < a.max_blocks) bt_hi = btrow[lb0 + lane + 64];
  }
  // Q does not depend on the sequence length. With kEarly (the grid is about one wave of work
  // groups) it is requested with the length and the page table, in one round trip; else after
  // them, so that work groups whose split lies past a short sequence's end request nothing.
  bf16x8_t qf[NTW][4];
  auto load_q = [&]() {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int r = R0 + 16 * t + n;
      if (r < GM) {
        const int i = r / G, h = g * G + (r - i * G);
        const u32x4_t* qp =
            reinterpret_cast<const u32x4_t*>(a.q + (((int64_t)b * M + i) * a.num_q_heads + h) * kHeadDim + 32 * q);
#pragma unroll
        for (int c = 0; c < 4; ++c) qf[t][c] = __builtin_bit_cast(bf16x8_t, qp[c]);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) qf[t][c] = __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
      }
    }
  };
  if constexpr (kEarly) load_q();
  int L = a.seq_lens[b];
  L = min(L, min(a.max_seq_len, a.max_blocks * a.block_size));
  const int lo_u = (wl < 0) ? 0 : max(0, L - M - wl);
  const int t_first = lo_u / kTile;
  const int t_end = L > 0 ? (L + kTile - 1) / kTile : 0;
  const int ntiles = max(0, t_end - t_first);
  const int nsplit = (ntiles + tps - 1) / tps;
  if (ntiles == 0) {
    // no visible key for any row: split 0 writes the group's rows as zeros
    if (s == 0) {
      for (int idx = threadIdx.x; idx < S::kRows * (kHeadDim / 4); idx += S::kThreads) {
        const int r = R0 + idx / (kHeadDim / 4), d4 = idx % (kHeadDim / 4);
        if (r >= GM) continue;
        const int i = r / G, h = g * G + (r - i * G);
        store_out4(a.out, a.out_bf16, (((int64_t)b * M + i) * a.num_q_heads + h) * kHeadDim + 4 * d4,
            f32x4_t{0.f, 0.f, 0.f, 0.f});
      }
    }
    return;
  }
  if (s >= nsplit) return;
  const int tb = t_first + s * tps;
  const int te = min(tb + tps, t_end);
  if (wl >= 0) {
    lb0 = tb >> bshift;
    if (lb0 + lane < a.max_blocks) bt_lo = btrow[lb0 + lane];
    if (lb0 + lane + 64 < a.max_blocks) bt_hi = btrow[lb0 + lane + 64];
  }
  const int lo_max = (wl < 0) ? 0 : max(0, L - 1 - wl);  // largest row window start
  const int p_min = L - M;                               // smallest row position
  const float C = a.softmax_scale * (kFp8 ? *a.k_scale : 1.0f) * kLog2e;

  // ---- this wave's query rows: positions and Q fragments (dims 32q + 8c .. +7)
  float m_ref[NTW], lsum[NTW];
  int rpos[NTW];
  f32x4_t o[NTW][8];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int r = R0 + 16 * t + n;
    rpos[t] = (r < GM) ? L - M + r / G : -1;
    m_ref[t] = -INFINITY;
    lsum[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[t][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (!kEarly) load_q();
  // Complete every pending load (page table, Q) here, through an asm that redefines the
  // page-table registers: later reads carry no load dependence, so the compiler adds no
  // wait on the DMAs below, whose counts the loop relies on.
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(bt_lo), "+v"(bt_hi)::"memory");
  auto block_of = [&](int tile) -> int {
    const int e = (tile >> bshift) - lb0;
    return __builtin_amdgcn_readlane(e < 64 ? bt_lo : bt_hi, e & 63);
  };

  // ---- this wave's tiles and its ring
  const int nt_w = (te - tb - kl + K - 1) / K;  // tiles tb + kl + K*i, i < nt_w (may be <= 0)
  const uint32_t koff = tile_chunk_offset<kFp8>(0, n, q);
  const uint32_t voff = tile_chunk_offset<kFp8>(T::kChunks / 2, n, q);
  unsigned char* ring = body + kl * 2 * T::kBytes;
  const uint32_t ring_lane = (uint32_t)(uintptr_t)ring + 16u * (uint32_t)lane;
  const int64_t slab_bytes = (int64_t)a.block_size * kHeadDim * (kFp8 ? 1 : 2);

  auto issue = [&](int i) {
    const int tile = tb + kl + K * i;
    int blk = block_of(tile);
    blk = ((unsigned)blk < (unsigned)a.num_blocks) ? blk : 0;
    const int o0 = (tile & bshift) * kTile;
    const int64_t off = ((int64_t)blk * a.num_kv_heads + g) * slab_bytes + (int64_t)o0 * kHeadDim * (kFp8 ? 1 : 2);
    const unsigned char* kb = a.k_pool + off + koff;
    const unsigned char* vb = a.v_pool + off + voff;
    dma_tile<kFp8>(kb, vb, ring + (i & 1) * T::kBytes);
  };

  // Software pipeline over the wave's tiles: the front half of a tile (wait for its DMA,
  // LDS read, refill of the slot, K conversion, S^T = K Q^T, masking) is issued before the
  // back half of the previous tile (online softmax, V conversion, O^T += V^T P^T), so one
  // tile's MFMAs overlap the other's VALU and transcendental work. Two register sets (A, B)
  // alternate, so no tile's registers are copied.
  struct Tile {
    TileRegs32<kFp8> r;
    f32x4_t s[2][NTW];
    int kt;
    bool valid, interior;
  };
  auto front = [&](int i, Tile& x) {
    if (i + 1 < nt_w) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(T::kChunks) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    if constexpr (kFp8) {
      // inline-asm reads (the compiler would otherwise wait for every DMA in flight); the
      // registers only feed the fp8 conversions
      read_slot<kFp8>(ring_lane + (uint32_t)((i & 1) * T::kBytes), x.r);
    } else {
      // BF16 registers feed the MFMAs directly: compiler-visible loads, which also wait for
      // the DMAs still in flight
      const u32x4_t* slot = reinterpret_cast<const u32x4_t*>(ring + (i & 1) * T::kBytes) + lane;
#pragma unroll
      for (int j = 0; j < 4; ++j) x.r.k[0][j] = slot[j * 64];
#pragma unroll
      for (int j = 0; j < 4; ++j) x.r.k[1][j] = slot[(4 + j) * 64];
#pragma unroll
      for (int j = 0; j < 8; ++j) x.r.v[j] = slot[(8 + j) * 64];
    }
    if (i + 2 < nt_w) issue(i + 2);
    const int tile = tb + kl + K * i;
    x.kt = tile * kTile;
    x.valid = (unsigned)block_of(tile) < (unsigned)a.num_blocks;
    x.interior = x.valid && (x.kt >= lo_max) && (x.kt + kTile - 1 <= p_min);
    // ---- S^T = K Q^T
#pragma unroll
    for (int t = 0; t < NTW; ++t) x.s[0][t] = x.s[1][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8_t kf0, kf1;
      if constexpr (kFp8) {
        const u32x4_t& v0 = x.r.k[0][c >> 1];
        const u32x4_t& v1 = x.r.k[1][c >> 1];
        kf0 = fp8x8_to_bf16x8(v0[(c & 1) * 2], v0[(c & 1) * 2 + 1]);
        kf1 = fp8x8_to_bf16x8(v1[(c & 1) * 2], v1[(c & 1) * 2 + 1]);
      } else {
        kf0 = __builtin_bit_cast(bf16x8_t, x.r.k[0][c]);
        kf1 = __builtin_bit_cast(bf16x8_t, x.r.k[1][c]);
      }
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        x.s[0][t] = mfma_bf16(kf0, qf[t][c], x.s[0][t]);
        x.s[1][t] = mfma_bf16(kf1, qf[t][c], x.s[1][t]);
      }
    }
    // ---- masking, only on tiles that are not visible to every row of the KV head
    if (!x.interior) {
      const int kt = x.kt;
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int hi = x.valid ? rpos[t] : -1;
        const int lo = (wl < 0) ? 0 : max(0, rpos[t] - wl);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = kt + 8 * q + 4 * tt + e;
            const uint32_t bad = (uint32_t)(((j - lo) | (hi - j)) >> 31);
            x.s[tt][t][e] = __uint_as_float((bad & 0xFF800000u) | (~bad & __float_as_uint(x.s[tt][t][e])));
          }
      }
      // keys outside [lo_u, L), and every key of an invalid block, may hold stale bytes:
      // zero their V so that 0 * NaN cannot occur
      const int e0 = x.valid ? min(8, max(0, lo_u - (kt + 8 * q))) : 8;
      const int e1 = min(8, max(0, L - (kt + 8 * q)));
      if (e0 > 0 || e1 < 8) {
        if constexpr (kFp8) {
          const uint64_t keep =
              (e1 >= 8 ? ~0ull : ((1ull << (8 * e1)) - 1)) & (e0 >= 8 ? 0ull : ~((1ull << (8 * e0)) - 1));
          const uint32_t klo = (uint32_t)keep, khi = (uint32_t)(keep >> 32);
#pragma unroll
          for (int j = 0; j < T::kVVec; ++j) {
            x.r.v[j][0] &= klo;
            x.r.v[j][1] &= khi;
            x.r.v[j][2] &= klo;
            x.r.v[j][3] &= khi;
          }
        } else {
#pragma unroll
          for (int j = 0; j < T::kVVec; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e < e0 || e >= e1) x.r.v[j][e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        }
      }
    }
  };

  auto back = [&](Tile& x) {
    // ---- online softmax: a row's reference maximum rises only when a tile exceeds it by
    // more than kLazyTau, so probabilities stay below 2^kLazyTau (exact range in f16)
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const float mx = fmaxf(fmaxf(fmaxf(x.s[0][t][0], x.s[0][t][1]), fmaxf(x.s[0][t][2], x.s[0][t][3])),
                             fmaxf(fmaxf(x.s[1][t][0], x.s[1][t][1]), fmaxf(x.s[1][t][2], x.s[1][t][3])));
      const float cand = group_max(mx) * C;
      const bool up = cand > m_ref[t] + kLazyTau;
      // the first visible keys of a row set its reference; its accumulators are still 0
      const bool rescale = up && m_ref[t] != -INFINITY;
      if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
        const float alpha = rescale ? __builtin_amdgcn_exp2f(m_ref[t] - cand) : 1.0f;
        lsum[t] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[t][dt] *= alpha;
      }
      m_ref[t] = up ? cand : m_ref[t];
    }

    if constexpr (kFp8) {
      f16x8_t P[NTW];
      const f16x2_t one2 = __builtin_bit_cast(f16x2_t, 0x3C003C00u);
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const float ms = (m_ref[t] == -INFINITY) ? 0.f : m_ref[t];
        float p[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e) p[tt][e] = __builtin_amdgcn_exp2f(fmaf(x.s[tt][t][e], C, -ms));
        // four separate words: read back out of one vector, the dot products were once
        // emitted on the first word four times
        const uint32_t h0 = pack_f16(p[0][0], p[0][1]), h1 = pack_f16(p[0][2], p[0][3]);
        const uint32_t h2 = pack_f16(p[1][0], p[1][1]), h3 = pack_f16(p[1][2], p[1][3]);
        P[t] = __builtin_bit_cast(f16x8_t, u32x4_t{h0, h1, h2, h3});
        // the row sum uses the same rounded probabilities the PV product sees
        float l = lsum[t];
        l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, h0), one2, l, false);
        l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, h1), one2, l, false);
        l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, h2), one2, l, false);
        l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, h3), one2, l, false);
        lsum[t] = l;
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const u32x4_t& v = x.r.v[dt >> 1];
        const f16x8_t vf = fp8x8_to_f16x8(v[(dt & 1) * 2], v[(dt & 1) * 2 + 1]);
#pragma unroll
        for (int t = 0; t < NTW; ++t) o[t][dt] = mfma_f16(vf, P[t], o[t][dt]);
      }
    } else {
      // BF16 cache: V stays BF16, so P is split into a BF16 head and a BF16 tail
      bf16x8_t Ph[NTW], Pl[NTW];
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const float ms = (m_ref[t] == -INFINITY) ? 0.f : m_ref[t];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(x.s[tt][t][e], C, -ms));
            const __bf16 hi = (__bf16)p;
            Ph[t][4 * tt + e] = hi;
            Pl[t][4 * tt + e] = (__bf16)(p - (float)hi);
            lsum[t] += p;
          }
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, x.r.v[dt]);
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          o[t][dt] = mfma_bf16(vf, Ph[t], o[t][dt]);
          o[t][dt] = mfma_bf16(vf, Pl[t], o[t][dt]);
        }
      }
    }
  };

  if (nt_w > 0) issue(0);
  if (nt_w > 1) issue(1);
  Tile ta, tb2;
  if (nt_w > 0) front(0, ta);
  for (int i = 0; i < nt_w; i += 2) {
    if (i + 1 < nt_w) front(i + 1, tb2);
    back(ta);
    if (i + 1 >= nt_w) break;
    if (i + 2 < nt_w) front(i + 2, ta);
    back(tb2);
  }

  // ---- merge the K waves: common maximum per row, then a fixed-order sum in LDS
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const float lt = group_sum(lsum[t]);
    if (q == 0) {
      sm_m[kl * S::kRows + 16 * t + n] = m_ref[t];
      sm_l[kl * S::kRows + 16 * t + n] = lt;
    }
  }
  __syncthreads();  // also: every wave's ring reads are done, the ring area is free
  f32x4_t* sm_o = reinterpret_cast<f32x4_t*>(body);  // [K][NTW*8][64]
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    float mm = -INFINITY;
#pragma unroll
    for (int u = 0; u < K; ++u) mm = fmaxf(mm, sm_m[u * S::kRows + 16 * t + n]);
    const float alpha = (m_ref[t] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref[t] - mm);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) sm_o[(kl * NTW * 8 + t * 8 + dt) * 64 + lane] = o[t][dt] * alpha;
    if (kl == 0 && q == 0) {
      // merged row sum, in wave order
      float lw = 0.f;
#pragma unroll
      for (int u = 0; u < K; ++u) {
        const float mu = sm_m[u * S::kRows + 16 * t + n];
        lw += (mu == -INFINITY) ? 0.f : sm_l[u * S::kRows + 16 * t + n] * __builtin_amdgcn_exp2f(mu - mm);
      }
      sm_row[16 * t + n] = mm;
      sm_row[S::kRows + 16 * t + n] = lw;
    }
  }
  __syncthreads();
  // wave kl sums d-tiles dt = kl*DPW .. over the K waves in wave order and stores them
  // row-major (padded rows) into the staging area
  constexpr int kDpw = (8 + K - 1) / K;
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int dd = 0; dd < kDpw; ++dd) {
      const int dt = kl * kDpw + dd;
      if (dt < 8) {
        f32x4_t acc = sm_o[(t * 8 + dt) * 64 + lane];
#pragma unroll
        for (int u = 1; u < K; ++u) acc += sm_o[(u * NTW * 8 + t * 8 + dt) * 64 + lane];
        float* row = stage + (16 * t + n) * S::kStride + 32 * q + dt;
#pragma unroll
        for (int e = 0; e < 4; ++e) row[8 * e] = acc[e];
      }
    }
  __syncthreads();

  // ---- write the group's rows: final (one split) or the split partial
  const bool direct = (nsplit == 1);
  const float vsc = kFp8 ? *a.v_scale : 1.0f;
  const int64_t part = ((int64_t)b * a.num_kv_heads + g) * a.max_splits + s;
  for (int idx = threadIdx.x; idx < S::kRows * (kHeadDim / 4); idx += S::kThreads) {
    const int rl = idx / (kHeadDim / 4), d4 = idx % (kHeadDim / 4);
    const int r = R0 + rl;
    if (r >= GM) continue;
    const f32x4_t val = *reinterpret_cast<const f32x4_t*>(stage + rl * S::kStride + 4 * d4);
    const float lw = sm_row[S::kRows + rl];
    if (direct) {
      const int i = r / G, h = g * G + (r - i * G);
      const float mul = lw > 0.f ? vsc / lw : 0.f;
      store_out4(a.out, a.out_bf16, (((int64_t)b * M + i) * a.num_q_heads + h) * kHeadDim + 4 * d4,
          val * mul);
    } else {
      *reinterpret_cast<f32x4_t*>(a.ws_o + (part * a.rows_pad + r) * kHeadDim + 4 * d4) = val;
      if (d4 == 0) {
        a.ws_ml[part * 2 * a.rows_pad + r] = sm_row[rl];
        a.ws_ml[part * 2 * a.rows_pad + a.rows_pad + r] = lw;
      }
    }
  }
}

template <int NTW, int K, bool kFp8>
static hipError_t launch_rows_t(const DecodeArgs& a, hipStream_t stream) {
  const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * a.max_splits;
  // per-XCD pairs: (pairs rounded up to 8) x splits x row groups; else (units rounded up to 8) x row groups
  const int64_t grid = a.xcd_pairs ? ((int64_t)a.num_seqs * a.num_kv_heads + 7) / 8 * 8 * a.max_splits * a.row_groups
                               : (units + 7) / 8 * 8 * a.row_groups;
  // early Q loads pay for a grid of about one wave of work groups (a layer of one sequence),
  // not for a large batch grid whose work groups mostly leave at once
  if (grid <= 2 * 256)
    hipLaunchKernelGGL((decode_rows_kernel<NTW, K, kFp8, true>), dim3((unsigned)grid),
                       dim3(RowsShape<NTW, K, kFp8>::kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_rows_kernel<NTW, K, kFp8, false>), dim3((unsigned)grid),
                       dim3(RowsShape<NTW, K, kFp8>::kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_rows(const DecodeArgs& a, int ntw, bool fp8, hipStream_t stream) {
  if (fp8) {
    if (ntw == 1) return launch_rows_t<1, 8, true>(a, stream);
    if (ntw == 2) return launch_rows_t<2, 8, true>(a, stream);
  } else {
    if (ntw == 1) return launch_rows_t<1, 4, false>(a, stream);
    if (ntw == 2) return launch_rows_t<2, 4, false>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fkv
