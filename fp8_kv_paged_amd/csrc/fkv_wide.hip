// Paged GQA decode attention, wide split kernel: every packed query row of a KV head in
// every wave.
//
// Operation: exact q1 / M12 paged attention over the calibrated FP8 cache ("Laguna S 2.1
// INT4 -- calibrated FP8 KV on Intel B70", sections Contract and "Initial optimization
// order"; 9 query heads per KV head, head 128, global and sliding windows in "Laguna FP8
// KV -- replicated embedding win, page-32 build, and host boundary", section "Page-32
// attention experiment").
//
// A work group of four waves (one per SIMD) takes one (sequence, KV head, split); each
// wave holds all NT 16-row query tiles of the KV head (NT = 7 at nine heads x M=12) and
// streams its own tiles (tb + kl, tb + kl + 4, ...) through a private two-slot LDS ring
// filled by global_load_lds. A K/V byte is therefore fetched and converted once. The
// NT*8 output accumulators live in AGPRs; Q sits in LDS (one 16-byte fragment per lane
// per row tile and 32-dimension chunk), so the VGPRs hold the converted tile (K as bf16,
// V as f16), one row tile's scores and probabilities, and the softmax state. Per tile
// the row tiles are processed in order: S^T = K Q^T (8 MFMAs), online softmax with a
// lazily raised reference maximum, O^T += V^T P^T (8 MFMAs). After the loop the four
// waves merge in LDS in a fixed order and the group writes final rows (one split) or an
// fp32 partial (m, l, O) for decode_combine_kernel. Lane and dimension layout as in the
// row-group kernel (fkv_rows.hip).
#include "fkv_device.h"
#include "fkv_internal.h"
#include "fkv_tile.h"

namespace fkv {

namespace {

constexpr int kWideWaves = 4;

template <int NT, bool kFp8>
struct WideShape {
  static constexpr int kThreads = 64 * kWideWaves;
  static constexpr int kRows = 16 * NT;
  static constexpr int kQ = NT * 4 * 64;                           // Q fragments (u32x4), lane layout
  static constexpr int kRing = kWideWaves * 2 * TileGeom<kFp8>::kBytes;
  static constexpr int kAcc = NT * 8 * 64 * 16;                    // one wave's O (lane layout)
  static constexpr int kMerge = 2 * kAcc;                          // two waves' O at once
  static constexpr int kStage = kRows * kHeadDim * 4;              // merged rows, row-major fp32
  static constexpr int kTail = (kMerge > kStage ? kMerge : kStage);
  static constexpr int kBody = kRing > kTail ? kRing : kTail;      // DMA rings, then merge / staging
  static_assert(2 * kWideWaves * kRows * 4 + kQ * 16 + 256 + kBody <= 160 * 1024, "LDS budget of one CU");
};

}  // namespace

template <int NT, bool kFp8>
__global__ __launch_bounds__((WideShape<NT, kFp8>::kThreads), 1) void decode_wide_kernel(DecodeArgs a) {
  typedef WideShape<NT, kFp8> S;
  typedef TileGeom<kFp8> T;
  constexpr int K = kWideWaves;
  // Three separate LDS objects: the compiler can then tell that reads of Q and of (m, l)
  // never touch what the DMAs write, and adds no wait on the DMAs before them.
  __shared__ float sm_ml[2 * K * S::kRows];                  // (m, l) of every wave's rows
  __shared__ u32x4_t q_lds[S::kQ];                          // [(t*4 + c)*64 + lane]
  // DMA rings, then merge / staging; 256 bytes of padding first so that no DMA can target
  // LDS address 0 (a null LDS pointer to the compiler) whatever order the objects take
  __shared__ __align__(256) unsigned char lds_body[256 + S::kBody];
  unsigned char* body = lds_body + 256;
  float* sm_m = sm_ml;                                      // [K][kRows]
  float* sm_l = sm_ml + K * S::kRows;                       // [K][kRows]
  unsigned char* rings = body;

  const int unit = blockIdx.x;
  const int s = unit % a.max_splits;
  const int bg = unit / a.max_splits;
  if (bg >= a.num_seqs * a.num_kv_heads) return;
  const int g = bg % a.num_kv_heads, b = bg / a.num_kv_heads;

  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const int kl = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.group, M = a.q_len, GM = G * M;
  const int wl = a.window_left;
  const int bshift = a.block_size == 64 ? 1 : 0;

  const int tps = a.tiles_per_split;
  const int32_t* btrow = a.block_table + (int64_t)b * a.max_blocks;
  int bt_lo = 0, bt_hi = 0;
  int lb0 = 0;
  if (wl < 0) {  // global attention: the split's first tile does not depend on the length
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
    if (s == 0) {
      for (int idx = threadIdx.x; idx < GM * (kHeadDim / 4); idx += S::kThreads) {
        const int r = idx / (kHeadDim / 4), d4 = idx % (kHeadDim / 4);
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
  if (wl >= 0) {
    lb0 = tb >> bshift;
    if (lb0 + lane < a.max_blocks) bt_lo = btrow[lb0 + lane];
    if (lb0 + lane + 64 < a.max_blocks) bt_hi = btrow[lb0 + lane + 64];
  }
  const int lo_max = (wl < 0) ? 0 : max(0, L - 1 - wl);
  const int p_min = L - M;
  const float C = a.softmax_scale * (kFp8 ? *a.k_scale : 1.0f) * kLog2e;

  // ---- Q of the KV head into LDS: entry (t, c, lane) = row 16t+n, dims 32q + 8c .. +7
  for (int e = threadIdx.x; e < NT * 4 * 64; e += S::kThreads) {
    const int t = e / 256, c = (e / 64) % 4, ln = e % 64;
    const int r = 16 * t + (ln & 15);
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (r < GM) {
      const int i = r / G, h = g * G + (r - i * G);
      v = *reinterpret_cast<const u32x4_t*>(a.q + (((int64_t)b * M + i) * a.num_q_heads + h) * kHeadDim +
                                            32 * (ln >> 4) + 8 * c);
    }
    q_lds[e] = v;
  }
  // finish every pending load (page table, Q) through an asm that redefines the page-table
  // registers, so no later instruction carries a load dependence that would make the
  // compiler wait on the DMAs below
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(bt_lo), "+v"(bt_hi)::"memory");
  __syncthreads();
  auto block_of = [&](int tile) -> int {
    const int e = (tile >> bshift) - lb0;
    return __builtin_amdgcn_readlane(e < 64 ? bt_lo : bt_hi, e & 63);
  };

  float m_ref[NT], lsum[NT];
  f32x4_t o[NT][8];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_ref[t] = -INFINITY;
    lsum[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[t][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int nt_w = (te - tb - kl + K - 1) / K;
  const uint32_t koff = tile_chunk_offset<kFp8>(0, n, q);
  const uint32_t voff = tile_chunk_offset<kFp8>(T::kChunks / 2, n, q);
  unsigned char* ring = rings + kl * 2 * T::kBytes;
  const uint32_t ring_lane = (uint32_t)(uintptr_t)ring + 16u * (uint32_t)lane;
  const int64_t slab_bytes = (int64_t)a.block_size * kHeadDim * (kFp8 ? 1 : 2);
  auto issue = [&](int i) {
    const int tile = tb + kl + K * i;
    int blk = block_of(tile);
    blk = ((unsigned)blk < (unsigned)a.num_blocks) ? blk : 0;
    const int o0 = (tile & bshift) * kTile;
    const int64_t off = ((int64_t)blk * a.num_kv_heads + g) * slab_bytes + (int64_t)o0 * kHeadDim * (kFp8 ? 1 : 2);
    dma_tile<kFp8>(a.k_pool + off + koff, a.v_pool + off + voff, ring + (i & 1) * T::kBytes);
  };

  // S^T = K Q^T for one row tile (8 MFMAs); Q fragments come from LDS, masked keys -> -inf
  bf16x8_t kf[2][4];
  TileRegs32<kFp8> cur;
  int kt = 0;
  bool valid = true, interior = true;
  auto qk = [&](int t, f32x4_t& s0, f32x4_t& s1) {
    // plain LDS loads: Q feeds the MFMAs directly, and only compiler-visible loads get the
    // wait states the MFMA operand hazards need
    u32x4_t qv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) qv[c] = q_lds[(t * 4 + c) * 64 + lane];
    s0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    s1 = s0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8_t qf = __builtin_bit_cast(bf16x8_t, qv[c]);
      s0 = mfma_bf16(kf[0][c], qf, s0);
      s1 = mfma_bf16(kf[1][c], qf, s1);
    }
    if (!interior) {
      // opaque copies: keep the compiler from hoisting this cold code's per-lane values
      // out of the loop, where they would hold registers for every tile
      // the row's position (-1 for padding rows), recomputed here rather than kept in a
      // register for every row tile
      int qq = q, nn = n;
      asm volatile("" : "+v"(qq), "+v"(nn));
      const int r = 16 * t + nn;
      const int rp = (r < GM) ? L - M + r / G : -1;
      const int hi = valid ? rp : -1;
      const int lo = (wl < 0) ? 0 : max(0, rp - wl);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j0 = kt + 8 * qq + e, j1 = j0 + 4;
        const uint32_t bad0 = (uint32_t)(((j0 - lo) | (hi - j0)) >> 31);
        const uint32_t bad1 = (uint32_t)(((j1 - lo) | (hi - j1)) >> 31);
        s0[e] = __uint_as_float((bad0 & 0xFF800000u) | (~bad0 & __float_as_uint(s0[e])));
        s1[e] = __uint_as_float((bad1 & 0xFF800000u) | (~bad1 & __float_as_uint(s1[e])));
      }
    }
  };

  // Probabilities of the tile, per row tile: the P^T fragment of the PV product (FP8 cache:
  // one f16x8; BF16 cache: a BF16 head and tail pair).
  constexpr int kPW = kFp8 ? 1 : 2;
  u32x4_t pfrag[NT][kPW];
  float alpha[NT];  // accumulator factor of each row for this tile (1 unless its reference rose)

  // Phase 1 of a tile: S^T = K Q^T, online softmax with a lazily raised reference maximum
  // (a row's reference rises only when a tile exceeds it by more than kLazyTau, so
  // probabilities stay below 2^kLazyTau, an exact range in f16), P and the row sums. The
  // row sums take the raise factor at once; the accumulators, which only MFMAs touch in the
  // hot loop, take it in the cold path. Returns true if some accumulator needs it.
  auto phase1 = [&]() -> bool {
    bool need = false;
    // up to six row tiles the next row tile's QK^T MFMAs are issued before this one's VALU
    // work, so the two overlap; at seven the registers do not allow it
    constexpr bool kPipe = NT <= 6;
    f32x4_t sn0, sn1;
    if (kPipe) qk(0, sn0, sn1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x4_t s0, s1;
      if (kPipe) {
        s0 = sn0;
        s1 = sn1;
        if (t + 1 < NT) qk(t + 1, sn0, sn1);
      } else {
        qk(t, s0, s1);
      }
      const float mx =
          fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])), fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
      const float cand = group_max(mx) * C;
      const bool up = cand > m_ref[t] + kLazyTau;
      const bool rescale = up && m_ref[t] != -INFINITY;  // first keys of a row: nothing to rescale
      alpha[t] = rescale ? __builtin_amdgcn_exp2f(m_ref[t] - cand) : 1.0f;
      need |= __builtin_amdgcn_ballot_w64(rescale) != 0;
      m_ref[t] = up ? cand : m_ref[t];
      const float ms = (m_ref[t] == -INFINITY) ? 0.f : m_ref[t];
      if constexpr (kFp8) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = __builtin_amdgcn_exp2f(fmaf(s0[e], C, -ms));
          p[4 + e] = __builtin_amdgcn_exp2f(fmaf(s1[e], C, -ms));
        }
        const uint32_t h0 = pack_f16_rtz(p[0], p[1]), h1 = pack_f16_rtz(p[2], p[3]);
        const uint32_t h2 = pack_f16_rtz(p[4], p[5]), h3 = pack_f16_rtz(p[6], p[7]);
        pfrag[t][0] = u32x4_t{h0, h1, h2, h3};
        // the row sum uses the same rounded probabilities the PV product sees
        const f16x2_t one2 = __builtin_bit_cast(f16x2_t, 0x3C003C00u);
        float l = lsum[t] * alpha[t];
        l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, h0), one2, l, false);
        l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, h1), one2, l, false);
        l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, h2), one2, l, false);
        l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, h3), one2, l, false);
        lsum[t] = l;
      } else {
        bf16x8_t Ph, Pl;
        float l = lsum[t] * alpha[t];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = __builtin_amdgcn_exp2f(fmaf(e < 4 ? s0[e] : s1[e - 4], C, -ms));
          const __bf16 hi = (__bf16)pe;
          Ph[e] = hi;
          Pl[e] = (__bf16)(pe - (float)hi);
          l += pe;
        }
        lsum[t] = l;
        pfrag[t][0] = __builtin_bit_cast(u32x4_t, Ph);
        pfrag[t][kPW - 1] = __builtin_bit_cast(u32x4_t, Pl);
      }
    }
    return need;
  };

  // Phase 2 of a tile: O^T += V^T P^T, one d-tile of V converted at a time
  auto phase2 = [&]() {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      if constexpr (kFp8) {
        const u32x4_t& v = cur.v[dt >> 1];
        const f16x8_t vf = fp8x8_to_f16x8(v[(dt & 1) * 2], v[(dt & 1) * 2 + 1]);
#pragma unroll
        for (int t = 0; t < NT; ++t) o[t][dt] = mfma_f16(vf, __builtin_bit_cast(f16x8_t, pfrag[t][0]), o[t][dt]);
      } else {
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, cur.v[dt]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          o[t][dt] = mfma_bf16(vf, __builtin_bit_cast(bf16x8_t, pfrag[t][0]), o[t][dt]);
          o[t][dt] = mfma_bf16(vf, __builtin_bit_cast(bf16x8_t, pfrag[t][kPW - 1]), o[t][dt]);
        }
      }
    }
  };

  if (nt_w > 0) issue(0);
  if (nt_w > 1) issue(1);
  int i = 0;
  for (;;) {
    bool cold = false;
    for (; i < nt_w; ++i) {
      if (i + 1 < nt_w) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(T::kChunks) : "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      if constexpr (kFp8) {
        // inline-asm reads: the compiler would otherwise wait for every DMA in flight; the
        // registers only feed the fp8 conversions
        read_slot<kFp8>(ring_lane + (uint32_t)((i & 1) * T::kBytes), cur);
      } else {
        // BF16 registers feed the MFMAs directly: compiler-visible loads (they wait for all
        // DMAs in flight, which costs the BF16 path some overlap)
        const u32x4_t* slot = reinterpret_cast<const u32x4_t*>(ring + (i & 1) * T::kBytes) + lane;
#pragma unroll
        for (int j = 0; j < 4; ++j) cur.k[0][j] = slot[j * 64];
#pragma unroll
        for (int j = 0; j < 4; ++j) cur.k[1][j] = slot[(4 + j) * 64];
#pragma unroll
        for (int j = 0; j < 8; ++j) cur.v[j] = slot[(8 + j) * 64];
      }
      if (i + 2 < nt_w) issue(i + 2);

      const int tile = tb + kl + K * i;
      kt = tile * kTile;
      valid = (unsigned)block_of(tile) < (unsigned)a.num_blocks;
      interior = valid && (kt >= lo_max) && (kt + kTile - 1 <= p_min);
      if (!interior) {
        // keys outside [lo_u, L), and every key of an invalid block, may hold stale bytes:
        // zero their V so that 0 * NaN cannot occur
        int qq = q;
        asm volatile("" : "+v"(qq));
        const int e0 = valid ? min(8, max(0, lo_u - (kt + 8 * qq))) : 8;
        const int e1 = min(8, max(0, L - (kt + 8 * qq)));
        if (e0 > 0 || e1 < 8) {
          if constexpr (kFp8) {
            const uint64_t keep =
                (e1 >= 8 ? ~0ull : ((1ull << (8 * e1)) - 1)) & (e0 >= 8 ? 0ull : ~((1ull << (8 * e0)) - 1));
            const uint32_t klo = (uint32_t)keep, khi = (uint32_t)(keep >> 32);
#pragma unroll
            for (int j = 0; j < T::kVVec; ++j) {
              cur.v[j][0] &= klo;
              cur.v[j][1] &= khi;
              cur.v[j][2] &= klo;
              cur.v[j][3] &= khi;
            }
          } else {
#pragma unroll
            for (int j = 0; j < T::kVVec; ++j)
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (e < e0 || e >= e1) cur.v[j][e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
          }
        }
      }
      // K converted once per tile: bf16 for the FP8 cache, as stored for the BF16 cache
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (kFp8) {
          const u32x4_t& v0 = cur.k[0][c >> 1];
          const u32x4_t& v1 = cur.k[1][c >> 1];
          kf[0][c] = fp8x8_to_bf16x8(v0[(c & 1) * 2], v0[(c & 1) * 2 + 1]);
          kf[1][c] = fp8x8_to_bf16x8(v1[(c & 1) * 2], v1[(c & 1) * 2 + 1]);
        } else {
          kf[0][c] = __builtin_bit_cast(bf16x8_t, cur.k[0][c]);
          kf[1][c] = __builtin_bit_cast(bf16x8_t, cur.k[1][c]);
        }
      }
      if (phase1()) {
        cold = true;
        break;
      }
      phase2();
    }
    if (!cold) break;
    // ---- cold path: a row's reference rose; rescale its accumulators, finish the tile, resume
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (__builtin_amdgcn_ballot_w64(alpha[t] != 1.0f) != 0) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[t][dt] *= alpha[t];
      }
    }
    phase2();
    ++i;
  }

  // ---- merge the four waves: common maximum per row, then a fixed-order sum in LDS
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float lt = group_sum(lsum[t]);
    if (q == 0) {
      sm_m[kl * S::kRows + 16 * t + n] = m_ref[t];
      sm_l[kl * S::kRows + 16 * t + n] = lt;
    }
  }
  __syncthreads();  // also: the loop's LDS (Q, rings) is free from here on
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float mm = -INFINITY;
#pragma unroll
    for (int u = 0; u < K; ++u) mm = fmaxf(mm, sm_m[u * S::kRows + 16 * t + n]);
    const float alpha = (m_ref[t] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref[t] - mm);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[t][dt] *= alpha;
  }
  f32x4_t* acc = reinterpret_cast<f32x4_t*>(body);  // two slots of [NT*8][64]
  // round 1: waves 1 and 3 hand their sums to waves 0 and 2; round 2: wave 2 to wave 0
  if (kl & 1) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[((kl >> 1) * NT * 8 + t * 8 + dt) * 64 + lane] = o[t][dt];
  }
  __syncthreads();
  if (!(kl & 1)) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[t][dt] += acc[((kl >> 1) * NT * 8 + t * 8 + dt) * 64 + lane];
  }
  __syncthreads();
  if (kl == 2) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[(t * 8 + dt) * 64 + lane] = o[t][dt];
  }
  __syncthreads();
  if (kl == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[t][dt] += acc[(t * 8 + dt) * 64 + lane];
  }
  __syncthreads();
  // wave 0 stores the merged rows row-major into the staging area
  float* stage = reinterpret_cast<float*>(body);
  if (kl == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        float* row = stage + (16 * t + n) * kHeadDim + 32 * q + dt;
#pragma unroll
        for (int e = 0; e < 4; ++e) row[8 * e] = o[t][dt][e];
      }
  }
  __syncthreads();

  // ---- write: final rows (one split) or the split partial
  const bool direct = (nsplit == 1);
  const float vsc = kFp8 ? *a.v_scale : 1.0f;
  const int64_t part = ((int64_t)b * a.num_kv_heads + g) * a.max_splits + s;
  for (int idx = threadIdx.x; idx < GM * (kHeadDim / 4); idx += S::kThreads) {
    const int r = idx / (kHeadDim / 4), d4 = idx % (kHeadDim / 4);
    float mm = -INFINITY;
#pragma unroll
    for (int u = 0; u < K; ++u) mm = fmaxf(mm, sm_m[u * S::kRows + r]);
    float lw = 0.f;
#pragma unroll
    for (int u = 0; u < K; ++u) {
      const float mu = sm_m[u * S::kRows + r];
      lw += (mu == -INFINITY) ? 0.f : sm_l[u * S::kRows + r] * __builtin_amdgcn_exp2f(mu - mm);
    }
    const f32x4_t val = *reinterpret_cast<const f32x4_t*>(stage + r * kHeadDim + 4 * d4);
    if (direct) {
      const int i = r / G, h = g * G + (r - i * G);
      const float mul = lw > 0.f ? vsc / lw : 0.f;
      *reinterpret_cast<f32x4_t*>(a.out + (((int64_t)b * M + i) * a.num_q_heads + h) * kHeadDim + 4 * d4) = val * mul;
    } else {
      *reinterpret_cast<f32x4_t*>(a.ws_o + (part * a.rows_pad + r) * kHeadDim + 4 * d4) = val;
      if (d4 == 0) {
        a.ws_ml[part * 2 * a.rows_pad + r] = mm;
        a.ws_ml[part * 2 * a.rows_pad + a.rows_pad + r] = lw;
      }
    }
  }
}

template <int NT, bool kFp8>
static hipError_t launch_wide_t(const DecodeArgs& a, hipStream_t stream) {
  const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * a.max_splits;
  hipLaunchKernelGGL((decode_wide_kernel<NT, kFp8>), dim3((unsigned)units), dim3(WideShape<NT, kFp8>::kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_wide(const DecodeArgs& a, int nt, bool fp8, hipStream_t stream) {
  switch (nt * 2 + (fp8 ? 1 : 0)) {
    case 3 * 2 + 1: return launch_wide_t<3, true>(a, stream);
    case 4 * 2 + 1: return launch_wide_t<4, true>(a, stream);
    case 5 * 2 + 1: return launch_wide_t<5, true>(a, stream);
    case 6 * 2 + 1: return launch_wide_t<6, true>(a, stream);
    case 7 * 2 + 1: return launch_wide_t<7, true>(a, stream);
    case 3 * 2: return launch_wide_t<3, false>(a, stream);
    case 4 * 2: return launch_wide_t<4, false>(a, stream);
    case 5 * 2: return launch_wide_t<5, false>(a, stream);
    case 6 * 2: return launch_wide_t<6, false>(a, stream);
    case 7 * 2: return launch_wide_t<7, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fkv
