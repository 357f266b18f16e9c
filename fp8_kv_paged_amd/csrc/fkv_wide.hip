// Paged GQA decode attention, wide split kernel: row halves x key lanes in one work group.
//
// Operation: exact q1 / M12 paged attention over the calibrated FP8 cache ("Laguna S 2.1
// INT4 -- calibrated FP8 KV on Intel B70", sections Contract and "Initial optimization
// order"; 9 query heads per KV head, head 128, global and sliding windows in "Laguna FP8
// KV -- replicated embedding win, page-32 build, and host boundary", section "Page-32
// attention experiment").
//
// Work decomposition. A work group of four waves (one per SIMD, so each wave has the
// whole register file of its SIMD) takes one (sequence, KV head, split). The KV head's
// packed query rows (16-row tiles) are cut into two halves of NTW tiles and the split's
// 32-key tiles into pairs; wave (h, k) holds the rows of half h and computes key tile k
// of every pair.
//   * A pair is fetched into an LDS ring slot by all four waves together (global_load_lds,
//     each wave a quarter of the 1 KB chunks), kDepth - 1 pairs ahead of its use. One
//     barrier per pair publishes it and frees the slot read in the previous step. Each
//     K/V byte is read from HBM once and converted twice (once per row half).
//   * Per tile a wave converts K (fp8 -> bf16, exact), forms S^T = K Q^T (8 MFMAs 16x16x32
//     per row tile, Q held in registers), exponentiates in the log2 domain against a per-row
//     reference, converts V (fp8 -> f16, exact) and accumulates O^T += V^T P^T (8 MFMAs per
//     row tile) into accumulators that stay in AGPRs.
//   * The hot path has no cross-lane step. A row tile's probabilities are accepted when
//     the eight a lane holds sum to at most 2^15, so each one fits f16. Otherwise, and on
//     a wave's first visible tile, a cold path takes the row maxima across lanes, raises
//     the reference of every row whose maximum exceeds it by more than kLazyTau, rescales
//     those rows' accumulators and recomputes the probabilities.
//   * After the loop the two key lanes of a row half merge in LDS (each wave finishes four
//     of the eight d-tiles) and the group writes final rows (one split) or an fp32 partial
//     in lane layout, which decode_combine_lanes_kernel merges over splits in split order.
//
// Lane layout (lane l = 16*q + n) as in the row-group kernel: score lane (n, q) holds keys
// 8q .. 8q+7 of row n (K rows permuted within each 16-key half), V is stored with each
// 8-key group dimension-major, and accumulator element e of d-tile dt at lane (n, q) is row
// n, dimension 32q + 8e + dt.
#include "fkv_device.h"
#include "fkv_internal.h"
#include "fkv_tile.h"

#include <type_traits>

namespace fkv {

namespace {

constexpr int kWideThreads = 256;      // four waves: (row half h, key lane k), wave = 2k + h

template <int NTW, bool kFp8>
struct WideShape {
  static constexpr int kDepth = kFp8 ? 6 : 3;                   // tile pairs in the LDS ring
  static constexpr int kPair = 2 * TileGeom<kFp8>::kBytes;
  static constexpr int kRing = kDepth * kPair;
  static constexpr int kMerge = 4 * NTW * 4 * 64 * 16;          // each wave: NTW row tiles x 4 d-tiles
  static constexpr int kBody = kRing > kMerge ? kRing : kMerge;
  static constexpr int kRowsW = 16 * NTW;                       // rows of one wave
  static_assert(2 * 4 * kRowsW * 4 + 256 + kBody <= 160 * 1024, "LDS budget of one CU");
};

// Waits until at most `pending` pairs of this wave's DMAs (kPer instructions each) are
// outstanding. global_load_lds completes in issue order, so the oldest pair has landed.
template <int kPer, int kMaxPending>
__device__ __forceinline__ void wait_pairs(int pending) {
  static_assert(kPer * kMaxPending <= 63, "vmcnt range");
  if (pending <= 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else if (pending == 1 || kMaxPending < 2) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPer) : "memory");
  } else if (pending == 2 || kMaxPending < 3) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kPer) : "memory");
  } else if (pending == 3 || kMaxPending < 4) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * kPer) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * kPer) : "memory");
  }
}

}  // namespace

template <int NTW, bool kFp8>
__global__ __launch_bounds__(kWideThreads, 1) void decode_wide_kernel(DecodeArgs a) {
  typedef WideShape<NTW, kFp8> S;
  typedef TileGeom<kFp8> T;
  constexpr int kHalf = T::kChunks / 2;  // DMA instructions per wave per pair
  constexpr int kNTT = 2 * NTW;          // row tiles of both halves (partial layout)
  // (m, l) of every wave's rows, apart from the ring so that its reads never wait for DMAs
  __shared__ float sm_ml[2 * 4 * S::kRowsW];
  // ring, then the merge exchange; 256 bytes first so that no DMA targets LDS address 0
  __shared__ __align__(256) unsigned char lds_body[256 + S::kBody];
  unsigned char* body = lds_body + 256;
  float* sm_m = sm_ml;                   // [wave][kRowsW]
  float* sm_l = sm_ml + 4 * S::kRowsW;   // [wave][kRowsW]

  const int unit = blockIdx.x;
  const int s = unit % a.max_splits;
  const int bg = unit / a.max_splits;
  if (bg >= a.num_seqs * a.num_kv_heads) return;
  const int g = bg % a.num_kv_heads, b = bg / a.num_kv_heads;

  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const int kl = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = kl & 1, k = kl >> 1;   // row half, key lane
  const int G = a.group, M = a.q_len, GM = G * M;
  const int wl = a.window_left;
  const int R0 = h * S::kRowsW;        // first packed row of the half
  const int bshift = a.block_size == 64 ? 1 : 0;

  // Page-table window of the split, requested with the sequence length for global
  // attention (the split's first tile does not depend on it).
  const int tps = a.tiles_per_split;
  const int32_t* btrow = a.block_table + (int64_t)b * a.max_blocks;
  int bt_lo = 0, bt_hi = 0;
  int lb0 = 0;
  if (wl < 0) {
    lb0 = (s * tps) >> bshift;
    if (lb0 + lane < a.max_blocks) bt_lo = btrow[lb0 + lane];
    if (lb0 + lane + 64 < a.max_blocks) bt_hi = btrow[lb0 + lane + 64];
  }
  int L = a.seq_lens[b];
  L = min(L, min(a.max_seq_len, a.max_blocks * a.block_size));
  const int lo_u = (wl < 0) ? 0 : max(0, L - M - wl);
  const int t_first = lo_u / kTile;
  const int t_end = L > 0 ? (L + kTile - 1) / kTile : 0;
  const int ntiles = max(0, t_end - t_first);
  const int nsplit = (ntiles + tps - 1) / tps;
  if (ntiles == 0) {
    // no visible key for any row: split 0 writes the rows as zeros
    if (s == 0) {
      for (int idx = threadIdx.x; idx < GM * (kHeadDim / 4); idx += kWideThreads) {
        const int r = idx / (kHeadDim / 4), d4 = idx % (kHeadDim / 4);
        const int i = r / G, hh = g * G + (r - i * G);
        *reinterpret_cast<f32x4_t*>(a.out + (((int64_t)b * M + i) * a.num_q_heads + hh) * kHeadDim + 4 * d4) =
            f32x4_t{0.f, 0.f, 0.f, 0.f};
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
  bf16x8_t qf[NTW][4];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int r = R0 + 16 * t + n;
    rpos[t] = (r < GM) ? L - M + r / G : -1;
    m_ref[t] = kRefInit;
    lsum[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[t][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc_fence(o[t]);
    if (r < GM) {
      const int i = r / G, hh = g * G + (r - i * G);
      const u32x4_t* qp =
          reinterpret_cast<const u32x4_t*>(a.q + (((int64_t)b * M + i) * a.num_q_heads + hh) * kHeadDim + 32 * q);
#pragma unroll
      for (int c = 0; c < 4; ++c) qf[t][c] = __builtin_bit_cast(bf16x8_t, qp[c]);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) qf[t][c] = __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
    }
  }
  // Complete the page-table and Q loads through an asm that redefines the page-table
  // registers: later reads carry no load dependence, so the compiler adds no wait on the
  // DMAs below, whose counts the loop relies on.
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(bt_lo), "+v"(bt_hi)::"memory");
  auto block_of = [&](int tile) -> int {
    const int e = (tile >> bshift) - lb0;
    return __builtin_amdgcn_readlane(e < 64 ? bt_lo : bt_hi, e & 63);
  };

  // ---- the ring: pair p (tiles tb + 2p, tb + 2p + 1) in slot p % kDepth; wave (h, k)
  // fetches the K half (h = 0) or the V half (h = 1) of the pair's tile k
  const int npairs = (te - tb + 1) / 2;
  const uint32_t koff = tile_chunk_offset<kFp8>(0, n, q);
  const uint32_t voff = tile_chunk_offset<kFp8>(kHalf, n, q);
  const int64_t slab_bytes = (int64_t)a.block_size * kHeadDim * (kFp8 ? 1 : 2);
  constexpr int kEs = kFp8 ? 1 : 2;
  auto issue = [&](int p) {
    // a tile past the split's end re-fetches its last tile (same instruction count per pair)
    const int tile = min(tb + 2 * p + k, te - 1);
    int blk = block_of(tile);
    blk = ((unsigned)blk < (unsigned)a.num_blocks) ? blk : 0;
    const int o0 = (tile & bshift) * kTile;
    const int64_t off = ((int64_t)blk * a.num_kv_heads + g) * slab_bytes + (int64_t)o0 * kHeadDim * kEs;
    unsigned char* dst = body + (p % S::kDepth) * S::kPair + k * T::kBytes;
    if (h == 0) {
      const unsigned char* kb = a.k_pool + off + koff;
#pragma unroll
      for (int j = 0; j < kHalf; ++j) {
        const int per_tt = kHalf / 2, tt = j / per_tt, piece = j % per_tt;
        __builtin_amdgcn_global_load_lds(kb + tt * 4 * kHeadDim * kEs + 16 * piece, dst + j * 1024, 16, 0, 0);
      }
    } else {
      const unsigned char* vb = a.v_pool + off + voff;
#pragma unroll
      for (int j = 0; j < kHalf; ++j)
        __builtin_amdgcn_global_load_lds(vb + 16 * j, dst + (kHalf + j) * 1024, 16, 0, 0);
    }
  };
  const uint32_t ring_lane = (uint32_t)(uintptr_t)body + (uint32_t)(k * T::kBytes) + 16u * (uint32_t)lane;

  // ---- one tile: S^T = K Q^T, masking, probabilities, O^T += V^T P^T
  auto tile_step = [&](int tile, TileRegs32<kFp8>& x) {
    const int kt = tile * kTile;
    const bool valid = (unsigned)block_of(tile) < (unsigned)a.num_blocks;
    const bool interior = valid && (kt >= lo_max) && (kt + kTile - 1 <= p_min);
    f32x4_t sc[2][NTW];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8_t kf0, kf1;
      if constexpr (kFp8) {
        const u32x4_t& v0 = x.k[0][c >> 1];
        const u32x4_t& v1 = x.k[1][c >> 1];
        kf0 = fp8x8_to_bf16x8(v0[(c & 1) * 2], v0[(c & 1) * 2 + 1]);
        kf1 = fp8x8_to_bf16x8(v1[(c & 1) * 2], v1[(c & 1) * 2 + 1]);
      } else {
        kf0 = __builtin_bit_cast(bf16x8_t, x.k[0][c]);
        kf1 = __builtin_bit_cast(bf16x8_t, x.k[1][c]);
      }
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const f32x4_t z = f32x4_t{0.f, 0.f, 0.f, 0.f};
        sc[0][t] = mfma_bf16(kf0, qf[t][c], c == 0 ? z : sc[0][t]);
        sc[1][t] = mfma_bf16(kf1, qf[t][c], c == 0 ? z : sc[1][t]);
      }
    }
    // ---- masking, only on tiles that are not visible to every row of the KV head
    if (!interior) {
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int hi = valid ? rpos[t] : -1;
        const int lo = (wl < 0) ? 0 : max(0, rpos[t] - wl);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = kt + 8 * q + 4 * tt + e;
            const uint32_t bad = (uint32_t)(((j - lo) | (hi - j)) >> 31);
            sc[tt][t][e] = __uint_as_float((bad & 0xFF800000u) | (~bad & __float_as_uint(sc[tt][t][e])));
          }
      }
      // keys outside [lo_u, L), and every key of an invalid block, may hold stale bytes:
      // zero their V so that 0 * NaN cannot occur
      const int e0 = valid ? min(8, max(0, lo_u - (kt + 8 * q))) : 8;
      const int e1 = min(8, max(0, L - (kt + 8 * q)));
      if (e0 > 0 || e1 < 8) {
        if constexpr (kFp8) {
          const uint64_t keep =
              (e1 >= 8 ? ~0ull : ((1ull << (8 * e1)) - 1)) & (e0 >= 8 ? 0ull : ~((1ull << (8 * e0)) - 1));
          const uint32_t klo = (uint32_t)keep, khi = (uint32_t)(keep >> 32);
#pragma unroll
          for (int j = 0; j < T::kVVec; ++j) {
            x.v[j][0] &= klo;
            x.v[j][1] &= khi;
            x.v[j][2] &= klo;
            x.v[j][3] &= khi;
          }
        } else {
#pragma unroll
          for (int j = 0; j < T::kVVec; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e < e0 || e >= e1) x.v[j][e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        }
      }
    }

    // ---- probabilities against the current references; the lane's sum is the range check
    float lt[NTW];
    f16x8_t P[NTW];            // FP8 cache: P in f16
    bf16x8_t Ph[NTW], Pl[NTW];  // BF16 cache: P as a bf16 head and tail
    auto probs = [&](int t) {
      if constexpr (kFp8) {
        float p[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e) p[tt][e] = __builtin_amdgcn_exp2f(fmaf(sc[tt][t][e], C, -m_ref[t]));
        const uint32_t h0 = pack_f16(p[0][0], p[0][1]), h1 = pack_f16(p[0][2], p[0][3]);
        const uint32_t h2 = pack_f16(p[1][0], p[1][1]), h3 = pack_f16(p[1][2], p[1][3]);
        P[t] = __builtin_bit_cast(f16x8_t, u32x4_t{h0, h1, h2, h3});
        // the row sum uses the same rounded probabilities the PV product sees
        const f16x2_t one2 = __builtin_bit_cast(f16x2_t, 0x3C003C00u);
        float l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, h0), one2, 0.f, false);
        l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, h1), one2, l, false);
        l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, h2), one2, l, false);
        lt[t] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, h3), one2, l, false);
      } else {
        float l = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sc[tt][t][e], C, -m_ref[t]));
            const __bf16 hi = (__bf16)p;
            Ph[t][4 * tt + e] = hi;
            Pl[t][4 * tt + e] = (__bf16)(p - (float)hi);
            l += p;
          }
        lt[t] = l;
      }
    };
    float chk = 0.f;
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      probs(t);
      chk = fmaxf(chk, lt[t]);
    }
    if (__builtin_amdgcn_ballot_w64(!(chk <= kAcceptSum)) != 0) {
      // cold path: exact row maxima; raise the references that are exceeded by more than
      // kLazyTau, rescale those rows, recompute the probabilities
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const float mx = fmaxf(fmaxf(fmaxf(sc[0][t][0], sc[0][t][1]), fmaxf(sc[0][t][2], sc[0][t][3])),
                               fmaxf(fmaxf(sc[1][t][0], sc[1][t][1]), fmaxf(sc[1][t][2], sc[1][t][3])));
        const float cand = group_max(mx) * C;  // -inf when the row sees no key of this tile
        const bool up = cand > m_ref[t] + kLazyTau;
        if (__builtin_amdgcn_ballot_w64(up) != 0) {
          const float alpha = up ? __builtin_amdgcn_exp2f(m_ref[t] - cand) : 1.0f;
          lsum[t] *= alpha;
          acc_fence(o[t]);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[t][dt] *= alpha;
          acc_fence(o[t]);
          m_ref[t] = up ? cand : m_ref[t];
          probs(t);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NTW; ++t) lsum[t] += lt[t];

    // ---- O^T += V^T P^T
    if constexpr (kFp8) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const u32x4_t& v = x.v[dt >> 1];
        const f16x8_t vf = fp8x8_to_f16x8(v[(dt & 1) * 2], v[(dt & 1) * 2 + 1]);
#pragma unroll
        for (int t = 0; t < NTW; ++t) pv_f16(o[t][dt], vf, P[t]);
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, x.v[dt]);
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          pv_bf16(o[t][dt], vf, Ph[t]);
          pv_bf16(o[t][dt], vf, Pl[t]);
        }
      }
    }
  };

  // ---- the pipeline: kDepth - 1 pairs in flight; one barrier per pair
#pragma unroll
  for (int p = 0; p < S::kDepth - 1; ++p)
    if (p < npairs) issue(p);
  for (int i = 0; i < npairs; ++i) {
    wait_pairs<kHalf, S::kDepth - 2>(min(npairs - 1 - i, S::kDepth - 2));
    // every wave's share of pair i has landed, and every wave has read pair i - 1
    asm volatile("s_barrier" ::: "memory");
    if (i + S::kDepth - 1 < npairs) issue(i + S::kDepth - 1);
    const int tile = tb + 2 * i + k;
    if (tile < te) {
      TileRegs32<kFp8> x;
      read_slot<kFp8>(ring_lane + (uint32_t)((i % S::kDepth) * S::kPair), x);
      tile_step(tile, x);
    }
  }

  // ---- merge the two key lanes of each row half
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    acc_fence(o[t]);
    const float lt = group_sum(lsum[t]);
    if (q == 0) {
      sm_m[kl * S::kRowsW + 16 * t + n] = m_ref[t];
      sm_l[kl * S::kRowsW + 16 * t + n] = lt;
    }
  }
  __syncthreads();  // also: every ring read is done, the ring area is free
  const int kp = kl ^ 2;  // the other key lane of the same row half
  f32x4_t* xch = reinterpret_cast<f32x4_t*>(body);  // [wave][t][4][64]
  float asf[NTW], Mrow[NTW], Lrow[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const float m0 = sm_m[(h + 0) * S::kRowsW + 16 * t + n], m1 = sm_m[(h + 2) * S::kRowsW + 16 * t + n];
    const float l0 = sm_l[(h + 0) * S::kRowsW + 16 * t + n], l1 = sm_l[(h + 2) * S::kRowsW + 16 * t + n];
    const float mm = fmaxf(m0, m1);
    const float a0 = __builtin_amdgcn_exp2f(m0 - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
    Mrow[t] = mm;
    Lrow[t] = l0 * a0 + l1 * a1;
    asf[t] = k == 0 ? a0 : a1;
  }
  const bool direct = (nsplit == 1);
  const float vsc = kFp8 ? *a.v_scale : 1.0f;
  const int64_t part = ((int64_t)b * a.num_kv_heads + g) * a.max_splits + s;
  // Key lane KL (a compile-time value, so the accumulators are only indexed by constants)
  // hands the other lane d-tiles 4 (1 - KL) .. +3, then finishes d-tiles 4 KL .. +3.
  auto merge = [&](auto kl_const) {
    constexpr int KL = decltype(kl_const)::value;
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) xch[((kl * NTW + t) * 4 + dd) * 64 + lane] = o[t][4 * (1 - KL) + dd] * asf[t];
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int r = R0 + 16 * t + n;
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        const int dt = 4 * KL + dd;
        const f32x4_t v = o[t][dt] * asf[t] + xch[((kp * NTW + t) * 4 + dd) * 64 + lane];
        if (direct) {
          if (r < GM) {
            const int i = r / G, hh = g * G + (r - i * G);
            const float mul = Lrow[t] > 0.f ? vsc / Lrow[t] : 0.f;
            float* op = a.out + (((int64_t)b * M + i) * a.num_q_heads + hh) * kHeadDim + 32 * q + dt;
#pragma unroll
            for (int e = 0; e < 4; ++e) op[8 * e] = v[e] * mul;
          }
        } else {
          *reinterpret_cast<f32x4_t*>(a.ws_o + (((part * kNTT + h * NTW + t) * 8 + dt) * 64 + lane) * 4) = v;
        }
      }
      if (!direct && KL == 0 && q == 0) {
        a.ws_ml[part * 2 * a.rows_pad + r] = Mrow[t];
        a.ws_ml[part * 2 * a.rows_pad + a.rows_pad + r] = Lrow[t];
      }
    }
  };
  if (k == 0) {
    merge(std::integral_constant<int, 0>());
  } else {
    merge(std::integral_constant<int, 1>());
  }
}

// Merges the lane-layout split partials of the wide kernel over splits, in split order:
// O = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s. One wave per (row tile, d-tile) slot
// of a (sequence, KV head), so the partials' reads spread over every CU; a thread holds
// four output values, dimensions 32q + 8e + dt of row 16 * tile + n.
__global__ __launch_bounds__(64) void decode_combine_lanes_kernel(DecodeArgs a, int kfp8) {
  constexpr int kChunk = 32;  // splits whose loads are in flight together (one round trip at 32 splits)
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
  const int ntt = a.rows_pad / 16;
  const int slot = blockIdx.x;
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  if (slot >= ntt * 8) return;
  const int tt = slot >> 3, dt = slot & 7;
  const int r = 16 * tt + n;
  if (r >= GM) return;
  const int64_t base = ((int64_t)b * a.num_kv_heads + g) * a.max_splits;
  const int64_t ml_stride = 2 * (int64_t)a.rows_pad;
  const int64_t o_stride = (int64_t)a.rows_pad * kHeadDim;  // floats per partial
  const float* mlp = a.ws_ml + base * ml_stride + r;
  const float* op = a.ws_o + base * o_stride + ((int64_t)slot * 64 + lane) * 4;

  float mrun = -INFINITY, lrun = 0.f;
  f32x4_t acc{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += kChunk) {
    float ms[kChunk], ls[kChunk];
    f32x4_t os[kChunk];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const int sj = min(s0 + j, nsplit - 1);  // clamped: in-range loads, unused past the end
      ms[j] = mlp[sj * ml_stride];
      ls[j] = mlp[sj * ml_stride + a.rows_pad];
      os[j] = *reinterpret_cast<const f32x4_t*>(op + sj * o_stride);
    }
    float mc = mrun;
#pragma unroll
    for (int j = 0; j < kChunk; ++j)
      if (s0 + j < nsplit) mc = fmaxf(mc, ms[j]);
    const float keep = (mrun == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mrun - mc);
    lrun *= keep;
    acc *= keep;
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      if (s0 + j < nsplit) {
        const float wgt = __builtin_amdgcn_exp2f(ms[j] - mc);
        lrun += wgt * ls[j];
        acc += os[j] * wgt;
      }
    }
    mrun = mc;
  }
  const float vsc = kfp8 ? *a.v_scale : 1.0f;
  const float mul = lrun > 0.f ? vsc / lrun : 0.f;
  const int i = r / G, hh = g * G + (r - i * G);
  float* out = a.out + (((int64_t)b * M + i) * a.num_q_heads + hh) * kHeadDim + 32 * q + dt;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[8 * e] = acc[e] * mul;
}

template <int NTW, bool kFp8>
static hipError_t launch_wide_t(const DecodeArgs& a, hipStream_t stream) {
  const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * a.max_splits;
  hipLaunchKernelGGL((decode_wide_kernel<NTW, kFp8>), dim3((unsigned)units), dim3(kWideThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_wide(const DecodeArgs& a, int ntw, bool fp8, hipStream_t stream) {
  switch (ntw * 2 + (fp8 ? 1 : 0)) {
    case 2 * 2 + 1: return launch_wide_t<2, true>(a, stream);
    case 3 * 2 + 1: return launch_wide_t<3, true>(a, stream);
    case 4 * 2 + 1: return launch_wide_t<4, true>(a, stream);
    case 2 * 2: return launch_wide_t<2, false>(a, stream);
    case 3 * 2: return launch_wide_t<3, false>(a, stream);
    case 4 * 2: return launch_wide_t<4, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine_lanes(const DecodeArgs& a, bool fp8, hipStream_t stream) {
  const int slots = (a.rows_pad / 16) * 8;
  hipLaunchKernelGGL(decode_combine_lanes_kernel, dim3(slots, a.num_kv_heads, a.num_seqs), dim3(64), 0, stream, a,
                     fp8 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace fkv
