// Paged GQA decode attention, 32-row tile kernel (layouts 5 and 6), with the new tokens'
// cache insertion optionally fused into its prologue.
//
// Operation: exact q1 / M12 paged attention over the calibrated FP8 cache ("Laguna S 2.1
// INT4 -- calibrated FP8 KV on Intel B70", sections Contract and "Initial optimization
// order"; 9 query heads per KV head, head 128, global and sliding windows in "Laguna FP8
// KV -- replicated embedding win, page-32 build, and host boundary", section "Page-32
// attention experiment").
//
// Work decomposition. One work group per (sequence, KV head, split, row group): RT row
// tiles of 32 packed query rows (G*M rows of the KV head, at most 128, over the row groups)
// and the split's 32-key tiles in KL key lanes; each wave holds RW row tiles of one key
// lane. Layout 5 (RW = 1): eight waves, waves w and w + 4 on one SIMD, so each SIMD runs two
// waves whose MFMA and softmax phases overlap. Layout 6 (RW = 2): four waves, one per SIMD,
// every converted K/V operand feeding two MFMAs.
//   * All waves fill an LDS ring of kDepth steps (a step = the KL tiles computed
//     together) with global_load_lds, kDepth - 1 steps ahead; one barrier per step
//     publishes a step and frees the slot read in the previous one. Each chunk is fetched
//     in the order the MFMA operands want it, so the LDS reads are lane-contiguous.
//   * S^T = K Q^T on MFMA 32x32x16 bf16 (fp8 -> bf16 exact), online softmax in the log2
//     domain against a lazily raised per-row reference, O^T += V^T P^T on MFMA 32x32x16
//     f16 (fp8 -> f16 exact, P rounded to the nearest f16). The S^T products of tile i+1
//     are issued in the same block as the probabilities of tile i, so MFMA and VALU work
//     interleave.
//   * After the loop the KL key lanes of a row tile merge through LDS in a fixed order
//     and the group writes final rows (one split) or an fp32 partial (m, l, O). The
//     partials of a (sequence, KV head) are merged in split order inside this kernel when
//     the grid fits on the chip, else by decode_combine_kernel.
//   * Work groups are numbered so that every split of one (sequence, KV head) runs on the
//     same XCD (ids congruent mod 8) when there are at least 8 such pairs.
//
// Lane layout (lane l = 32 h + n). MFMA 32x32x16: A lane l holds row l%32, k = 8(l/32)+e;
// B lane l holds column l%32, k = 8(l/32)+e; D lane l holds column l%32, rows
// 8(v/4) + 4(l/32) + v%4 for accumulator element v.
//   * Head dimensions are permuted the same way in Q and K: k-chunk c of lane half h is
//     d = 32(c/2) + 16h + 8(c%2) + e, so a lane reads 16 contiguous dims per pair of chunks.
//   * K row m of the A operand is key pi(m) (bits 2 and 3 of m swapped). Then score element
//     v of lane (n, h) is key 16(v/8) + 8h + v%8 of query row n: elements 0..7 and 8..15 are
//     exactly the P^T operand slices of the two 16-key halves of the PV product.
//   * V is stored with each 8-key group dimension-major; the A operand of d-tile 2a+b,
//     key half c' at lane (n, h) is dim 64a + 2n + b of keys 16c' + 8h + 0..7 (8 bytes), so
//     one 16-byte read serves d-tiles 2a and 2a+1. Output element v of d-tile 2a+b at lane
//     (n, h) is dim 64a + 16(v/4) + 8h + 2(v%4) + b of row n.
#include "fkv_device.h"
#include "fkv_internal.h"
#include "fkv_tile.h"

namespace fkv {

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// RT row tiles of 32 per work group, KL key lanes, RW row tiles per wave: (RT / RW) * KL
// waves. RW = 1: eight waves, two per SIMD; RW = 2: four waves, one per SIMD, each holding
// two row tiles so that every converted K/V operand feeds two MFMAs.
template <int RT, int KL, int RW, bool kFp8>
struct M32Shape {
  static constexpr int kWaves = RT / RW * KL;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kEs = kFp8 ? 1 : 2;
  static constexpr int kTileBytes = 2 * kTile * kHeadDim * kEs;  // K and V of one 32-key tile
  static constexpr int kChunks = kTileBytes / 1024;              // 1 KB DMA chunks per tile
  static constexpr int kStepBytes = KL * kTileBytes;
  static constexpr int kPerWave = KL * kChunks / kWaves;         // DMA instructions per wave per step
  static constexpr int kDepth = (128 * 1024) / kStepBytes < 8 ? (128 * 1024) / kStepBytes : 8;
  static constexpr int kRing = kDepth * kStepBytes;
  // key-lane merge: each owner receives (KL - 1) sources x (16 / KL) quads x 64 lanes of
  // f32x4 per row tile; the merged rows are staged in an area of their own
  static constexpr int kXch = RT * (KL - 1) * 16 * 64 * 16;
  static constexpr int kStageStride = kHeadDim + 4;                 // floats per staged row (conflict-free)
  static constexpr int kStage = 32 * RT * kStageStride * 4;
  static constexpr int kBody = kRing > kXch + kStage ? kRing : kXch + kStage;
  static_assert(kDepth >= 2, "ring of at least two steps");
  static_assert((kDepth - 2) * kPerWave <= 63, "vmcnt range");
  static_assert(KL * kChunks % kWaves == 0, "DMA chunks split evenly over the waves");
  static_assert(8 % KL == 0, "output groups split evenly over the key lanes");
  static_assert(RT % RW == 0 && (RW == 1 || RW == 2), "whole row tiles per wave");
  static_assert(kWaves == 4 || kWaves == 8, "one or two waves per SIMD");
  static_assert(256 + kBody + 2 * KL * RT * 32 * 4 <= 160 * 1024, "LDS budget of one CU");
};

// O^T += V^T P^T. The accumulators stay in VGPRs (MFMA VGPR form): pinning them to AGPRs
// would split the 256-register budget of a two-wave-per-SIMD kernel in halves.
__device__ __forceinline__ void pv32_f16(f32x16_t& acc, const f16x8_t& a, const f16x8_t& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
}
// With two row tiles per wave the 128 accumulators would not fit beside the operands in
// the 256 VGPRs: they live in AGPRs and only inline asm touches them. The asm carries the
// wait states the hazard recognizer cannot see: two after a VALU write of a source
// register; back-to-back MFMAs on one accumulator need none.
// All 16 P.V MFMAs of one tile for two row tiles in one asm block, accumulators in AGPRs:
// the compiler can put no code between them (a register copy of an accumulator while an MFMA
// writing it is in flight would read a stale value; the hazard recognizer cannot see into
// asm), and the trailing 24 wait states let every later instruction read the results. Per
// accumulator the products come in the order of pv32_f16: key half 0, then key half 1.
__device__ __forceinline__ void pv32_f16_agpr_rw2(f32x16_t (&o0)[4], f32x16_t (&o1)[4], const f16x8_t (&va)[4],
                                                  const f16x8_t (&vb)[4], const f16x8_t& p00, const f16x8_t& p01,
                                                  const f16x8_t& p10, const f16x8_t& p11) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_f16 %0, %8, %16, %0\n\t"
      "v_mfma_f32_32x32x16_f16 %4, %8, %18, %4\n\t"
      "v_mfma_f32_32x32x16_f16 %0, %12, %17, %0\n\t"
      "v_mfma_f32_32x32x16_f16 %4, %12, %19, %4\n\t"
      "v_mfma_f32_32x32x16_f16 %1, %9, %16, %1\n\t"
      "v_mfma_f32_32x32x16_f16 %5, %9, %18, %5\n\t"
      "v_mfma_f32_32x32x16_f16 %1, %13, %17, %1\n\t"
      "v_mfma_f32_32x32x16_f16 %5, %13, %19, %5\n\t"
      "v_mfma_f32_32x32x16_f16 %2, %10, %16, %2\n\t"
      "v_mfma_f32_32x32x16_f16 %6, %10, %18, %6\n\t"
      "v_mfma_f32_32x32x16_f16 %2, %14, %17, %2\n\t"
      "v_mfma_f32_32x32x16_f16 %6, %14, %19, %6\n\t"
      "v_mfma_f32_32x32x16_f16 %3, %11, %16, %3\n\t"
      "v_mfma_f32_32x32x16_f16 %7, %11, %18, %7\n\t"
      "v_mfma_f32_32x32x16_f16 %3, %15, %17, %3\n\t"
      "v_mfma_f32_32x32x16_f16 %7, %15, %19, %7\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7"
      : "+a"(o0[0]), "+a"(o0[1]), "+a"(o0[2]), "+a"(o0[3]), "+a"(o1[0]), "+a"(o1[1]), "+a"(o1[2]), "+a"(o1[3])
      : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(vb[0]), "v"(vb[1]), "v"(vb[2]), "v"(vb[3]), "v"(p00),
        "v"(p01), "v"(p10), "v"(p11));
}
// Orders every later access of a row tile's AGPR accumulators after the MFMAs in flight on
// them (a 32x32 MFMA result may be read by other instructions only some passes after the
// MFMA issues; 24 wait states cover it).
__device__ __forceinline__ void acc_fence32(f32x16_t (&o)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]));
}
// Maximum of the two lanes that hold one query row (l and l ^ 32).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Waits until at most `pending` steps of this wave's DMAs (kPer instructions each) are
// outstanding; global_load_lds completes in issue order.
template <int kPer, int kMaxPending>
__device__ __forceinline__ void wait_steps(int pending) {
  if (pending <= 0 || kMaxPending <= 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else if (pending == 1 || kMaxPending < 2) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPer) : "memory");
  } else if (pending == 2 || kMaxPending < 3) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kPer) : "memory");
  } else if (pending == 3 || kMaxPending < 4) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * kPer) : "memory");
  } else if (pending == 4 || kMaxPending < 5) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * kPer) : "memory");
  } else if (pending == 5 || kMaxPending < 6) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(5 * kPer) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(6 * kPer) : "memory");
  }
}

__device__ __forceinline__ f32x16_t mfma32_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// K row fed by A-operand row m of a 32-key tile: bits 2 and 3 of m swapped.
__device__ __forceinline__ int key_of_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Split partials and merge counters are written and read only with the device-scope cache
// policy (sc1). The LLVM AMDGPU memory model for GFX942/GFX950 (AMDGPUUsage, "Memory Model
// GFX942") lowers agent-scope monotonic atomic loads, stores and RMWs to exactly these sc1
// accesses, i.e. they are coherent across the XCDs' separate L2 caches by themselves; its
// agent-scope release/acquire add an L2 write-back / invalidate only for plain (non-sc1)
// accesses, plus the vmcnt waits. So the publishing order needs only those waits: every
// partial store completes (s_waitcnt vmcnt(0), then a barrier) before the finished counter is
// incremented, and partial loads are issued after the counter load has returned.
constexpr int kCoherent = 16;  // cache-policy bits of the buffer intrinsics: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

constexpr int kSpinLimit = 1 << 15;  // polls (each with a short sleep) before a waiting group gives up
// Per pair, alone in a 256-byte block: counters of started, finished and exited work groups,
// then one claim bit per output slice (at most 256 slices).
constexpr int kCtlStride = 64;
constexpr int kCtlStarted = 0, kCtlFinished = 1, kCtlExited = 2, kCtlClaim = 8;
constexpr int kFastSplits = kFastMergeSplits;  // split counts whose partials one thread requests at once

// Merges the split partials of output quads [q0, q0 + count) of one (sequence, KV head)
// (quad q = packed row q / 32, dims 4(q % 32) .. +3): out = v_scale * sum_s w_s O_s / sum_s
// w_s l_s with w_s = 2^(m_s - max_s m_s), sums in split order. The rows' (m, l) pairs are
// read once into LDS and their weights computed once per (row, split); each thread then
// requests its quad of every split at once.
template <int kThreads>
__device__ __forceinline__ void merge_slice(const DecodeArgs& a, int b, int g, int nsplit, int q0, int count, float vsc,
                                            float* wsm) {
  const int G = a.group, M = a.q_len, GM = G * M;
  const int r0 = q0 >> 5, r1 = min((q0 + count - 1) >> 5, GM - 1);
  const int nr = r1 - r0 + 1;
  const int64_t base = ((int64_t)b * a.num_kv_heads + g) * a.max_splits;
  const uint32_t o_bytes = (uint32_t)((int64_t)nsplit * a.rows_pad * kHeadDim * 4);
  const uint32_t ml_bytes = (uint32_t)((int64_t)nsplit * 2 * a.rows_pad * 4);
  const __amdgpu_buffer_rsrc_t orsrc = coherent_rsrc(a.ws_o + base * a.rows_pad * kHeadDim, o_bytes);
  const __amdgpu_buffer_rsrc_t mlrsrc = coherent_rsrc(a.ws_ml + base * 2 * a.rows_pad, ml_bytes);
  float* wm = wsm;                 // [nr][nsplit]: m, then the weight
  float* wl = wsm + nr * nsplit;   // [nr][nsplit]: l
  float* mul = wl + nr * nsplit;   // [nr]: v_scale / sum_s w_s l_s
  for (int idx = threadIdx.x; idx < nr * nsplit; idx += kThreads) {
    const int rr = idx / nsplit, sj = idx % nsplit;
    const int off = (sj * 2 * a.rows_pad + r0 + rr) * 4;
    wm[idx] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mlrsrc, off, 0, kCoherent));
    wl[idx] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mlrsrc, off + a.rows_pad * 4, 0, kCoherent));
  }
  __syncthreads();
  if ((int)threadIdx.x < nr) {
    float* m = wm + threadIdx.x * nsplit;
    const float* l = wl + threadIdx.x * nsplit;
    float mx = -INFINITY;
    for (int sj = 0; sj < nsplit; ++sj) mx = fmaxf(mx, m[sj]);
    float lsum = 0.f;
    for (int sj = 0; sj < nsplit; ++sj) {
      const float wgt = __builtin_amdgcn_exp2f(m[sj] - mx);
      m[sj] = wgt;
      lsum += wgt * l[sj];
    }
    mul[threadIdx.x] = lsum > 0.f ? vsc / lsum : 0.f;
  }
  __syncthreads();
  constexpr int kChunk = 32;
  for (int t = (int)threadIdx.x; t < count; t += kThreads) {
    const int q = q0 + t, r = q >> 5, d4 = q & 31;
    if (r >= GM) continue;
    const float* wr = wm + (r - r0) * nsplit;
    const int o_off = (r * kHeadDim + 4 * d4) * 4, o_stride = a.rows_pad * kHeadDim * 4;
    f32x4_t acc{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nsplit; s0 += kChunk) {
      f32x4_t os[kChunk];
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        const int sj = min(s0 + j, nsplit - 1);  // clamped: in-range loads, unused past the end
        os[j] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(orsrc, o_off + sj * o_stride, 0, kCoherent));
      }
#pragma unroll
      for (int j = 0; j < kChunk; ++j)
        if (s0 + j < nsplit) acc += os[j] * wr[s0 + j];
    }
    const int i = r / G, hq = g * G + (r - i * G);
    store_out4(a.out, a.out_bf16, (((int64_t)b * M + i) * a.num_q_heads + hq) * kHeadDim + 4 * d4,
        acc * mul[r - r0]);
  }
  __syncthreads();  // the LDS weights are free again
}

// One output quad merged from at most kFastSplits partials by one thread: every load is
// requested at once (quad_issue) and combined later (quad_finish), with the same sums in
// the same order as merge_slice.
struct QuadLoads {
  f32x4_t o[kFastSplits];
  float m[kFastSplits], l[kFastSplits];
};
__device__ __forceinline__ void quad_issue(const DecodeArgs& a, int b, int g, int nsplit, int q, QuadLoads& x) {
  const int r = q >> 5, d4 = q & 31;
  const int64_t base = ((int64_t)b * a.num_kv_heads + g) * a.max_splits;
  const __amdgpu_buffer_rsrc_t orsrc = coherent_rsrc(a.ws_o + base * a.rows_pad * kHeadDim,
                                                     (uint32_t)((int64_t)nsplit * a.rows_pad * kHeadDim * 4));
  const __amdgpu_buffer_rsrc_t mlrsrc =
      coherent_rsrc(a.ws_ml + base * 2 * a.rows_pad, (uint32_t)((int64_t)nsplit * 2 * a.rows_pad * 4));
  const int o_off = (r * kHeadDim + 4 * d4) * 4, o_stride = a.rows_pad * kHeadDim * 4;
#pragma unroll
  for (int j = 0; j < kFastSplits; ++j) {
    const int sj = min(j, nsplit - 1);  // clamped: in-range loads, unused past the end
    x.o[j] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(orsrc, o_off + sj * o_stride, 0, kCoherent));
    x.m[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mlrsrc, (sj * 2 * a.rows_pad + r) * 4, 0, kCoherent));
    x.l[j] = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(mlrsrc, (sj * 2 * a.rows_pad + a.rows_pad + r) * 4, 0, kCoherent));
  }
}
__device__ __forceinline__ void quad_finish(const DecodeArgs& a, int b, int g, int nsplit, int q, const QuadLoads& x,
                                            float vsc) {
  const int r = q >> 5, d4 = q & 31;
  if (r >= a.group * a.q_len) return;
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < kFastSplits; ++j)
    if (j < nsplit) mx = fmaxf(mx, x.m[j]);
  float w[kFastSplits];
  float lsum = 0.f;
#pragma unroll
  for (int j = 0; j < kFastSplits; ++j) {
    w[j] = __builtin_amdgcn_exp2f(x.m[j] - mx);
    if (j < nsplit) lsum += w[j] * x.l[j];
  }
  const float mul = lsum > 0.f ? vsc / lsum : 0.f;
  f32x4_t acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kFastSplits; ++j)
    if (j < nsplit) acc += x.o[j] * w[j];
  const int G = a.group, i = r / G, hq = g * G + (r - i * G);
  store_out4(a.out, a.out_bf16, (((int64_t)b * a.q_len + i) * a.num_q_heads + hq) * kHeadDim + 4 * d4,
      acc * mul);
}

}  // namespace

namespace {

// RMSNorm + RoPE (norm_rope16's order) of one query row held by lanes n and n + 32 in the MFMA
// operand layout: lane half hh holds dims 32j + 16hh .. +15 (j = 0..3) as q[2j] (the first 8)
// and q[2j + 1], i.e. q[c] holds group g = 4(c / 2) + 2hh + c % 2 of 8 dims. Group distances
// 1, 4 and 8 stay inside the lane (c xor 1, 2, 4), distance 2 is the lane pair; the rotate-half
// partner of q[c] (c < 4) is q[c + 4]. Every lane of the wave must call it.
__device__ __forceinline__ void norm_rope_q64(u32x4_t (&q)[8], const uint16_t* w, int hh, float eps,
                                              const float* row) {
#pragma clang fp contract(off)
  float x[8][8], s[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int k = 0; k < 8; ++k) x[c][k] = (k & 1) ? bf16_hi(q[c][k >> 1]) : bf16_lo(q[c][k >> 1]);
    s[c] = x[c][0] * x[c][0];
#pragma unroll
    for (int k = 1; k < 8; ++k) s[c] = s[c] + x[c][k] * x[c][k];
  }
  float t[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) t[c] = s[c] + s[c ^ 1];  // group distance 1
#pragma unroll
  for (int c = 0; c < 8; ++c) s[c] = t[c] + __shfl_xor(t[c], 32);  // distance 2: the lane pair
#pragma unroll
  for (int c = 0; c < 8; ++c) t[c] = s[c] + s[c ^ 2];  // distance 4
#pragma unroll
  for (int c = 0; c < 8; ++c) s[c] = t[c] + t[c ^ 4];  // distance 8
  const float rr = __fdiv_rn(1.0f, sqrtf(__fdiv_rn(s[0], 128.0f) + eps));
  float y[8][8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int g = 4 * (c >> 1) + 2 * hh + (c & 1);
    const u32x4_t wv = *reinterpret_cast<const u32x4_t*>(w + 8 * g);
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
      const float w0 = bf16_lo(wv[k >> 1]), w1 = bf16_hi(wv[k >> 1]);
      const uint32_t yb = bf16x2_rne((x[c][k] * rr) * w0, (x[c][k + 1] * rr) * w1);
      y[c][k] = bf16_lo(yb);
      y[c][k + 1] = bf16_hi(yb);
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int g = 4 * (c >> 1) + 2 * hh + (c & 1);  // dims 8g .. 8g + 7 (< 64), partners in q[c + 4]
    const f32x4_t c0 = *reinterpret_cast<const f32x4_t*>(row + 8 * g);
    const f32x4_t c1 = *reinterpret_cast<const f32x4_t*>(row + 8 * g + 4);
    const f32x4_t s0 = *reinterpret_cast<const f32x4_t*>(row + 64 + 8 * g);
    const f32x4_t s1 = *reinterpret_cast<const f32x4_t*>(row + 64 + 8 * g + 4);
    const float cs[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    const float sn[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    float zl[8], zh[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      zl[k] = y[c][k] * cs[k] - y[c + 4][k] * sn[k];
      zh[k] = y[c + 4][k] * cs[k] + y[c][k] * sn[k];
    }
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
      q[c][k >> 1] = bf16x2_rne(zl[k], zl[k + 1]);
      q[c + 4][k >> 1] = bf16x2_rne(zh[k], zh[k + 1]);
    }
  }
}

template <int RT, int KL, int RW, bool kFp8, bool kIns, bool kEarly>
__global__ __launch_bounds__((M32Shape<RT, KL, RW, kFp8>::kThreads), 1) void decode_m32_kernel(DecodeArgs a) {
  typedef M32Shape<RT, KL, RW, kFp8> S;
  static_assert(kFp8, "the 32-row kernel reads FP8 caches");
  constexpr int kRows = 32 * RT;
  // (m, l) of every wave's rows, apart from the ring so that its reads never wait for DMAs
  __shared__ float sm_ml[2 * KL * kRows];
  // ring, then the merge exchange; 256 bytes first so that no DMA targets LDS address 0
  __shared__ __align__(256) unsigned char lds_body[256 + S::kBody];
  unsigned char* body = lds_body + 256;
  float* sm_m = sm_ml;               // [kl][row]
  float* sm_l = sm_ml + KL * kRows;  // [kl][row]

  // ---- (sequence, KV head, split); with >= 8 pairs every split of a pair on one XCD
  const int x = blockIdx.x;
  const int RG = a.row_groups;   // work groups per (sequence, KV head, split), kRows rows each
  const int per_pair = a.max_splits * RG;
  int bg, rem;
  if (a.xcd_pairs) {
    const int slot = x >> 3;
    bg = (slot / per_pair) * 8 + (x & 7);
    rem = slot % per_pair;
  } else {
    bg = x / per_pair;
    rem = x % per_pair;
  }
  const int s = rem / RG, rg = rem % RG;
  const int row0 = rg * kRows;   // first packed row of this work group
  if (bg >= a.num_seqs * a.num_kv_heads) return;
  const int g = bg % a.num_kv_heads, b = bg / a.num_kv_heads;

  const int lane = threadIdx.x & 63, n = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int kTG = RT / RW;                // row-tile groups of a work group
  const int rtg = w % kTG, kl = w / kTG;      // this wave: row tiles rtg * RW .. +RW-1, key lane kl
  const int G = a.group, M = a.q_len, GM = G * M;
  const int wl = a.window_left;
  const int bshift = a.block_size == 64 ? 1 : 0;  // 32-key tiles per page: 1 or 2

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
  // The scales, Q and the new tokens do not depend on the sequence length. With kEarly (the
  // grid is about one wave of work groups, e.g. a layer of one sequence) they are requested
  // with it and the page table, in one round trip; else (many splits past a short sequence's
  // end, as in a batch of mixed lengths) after it, so that the work groups that leave at once
  // request nothing and free their CU sooner.
  int L = a.seq_lens[b];
  float ks = 1.0f, vs_ins = 1.0f;
  int rl[RW], rpos[RW];
  u32x4_t qraw[RW][8];
  const bool wave_rows = row0 + 32 * rtg * RW < GM;  // wave-uniform: the wave's row tiles hold a real row
  // Fused insert: every group requests the q_len new tokens' K and V of its KV head with Q
  // (thread t < 16 M: K of token t / 16, dims 8 (t % 16) .. +7; the next 16 M threads: V);
  // only the groups whose split holds the new positions use them.
  constexpr bool fuse_ins = kIns;  // the instantiation with the new tokens' insert (k_new, v_new set)
  constexpr int kInsPer = 512 / S::kThreads;  // chunks per thread (32 M <= 512)
  int ci[kInsPer];
  bool ins_v_chunk[kInsPer], ins_chunk[kInsPer];
  u32x4_t nraw[kInsPer];
  auto load_inputs = [&]() {
    ks = *a.k_scale;
    if constexpr (kIns) vs_ins = *a.v_scale;
    // this wave's query rows and Q operands: lane (n, hh) of row tile r holds dims
    // 32j + 16hh .. +15 of row 32 (rtg * RW + r) + n
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      rl[r] = 32 * (rtg * RW + r) + n;  // row within the work group (LDS index)
      const int pr = row0 + rl[r];      // packed row of the KV head
      if (pr < GM) {
        const int i = pr / G, hq = g * G + (pr - i * G);
        const u32x4_t* qp =
            reinterpret_cast<const u32x4_t*>(a.q + (((int64_t)b * M + i) * a.num_q_heads + hq) * kHeadDim);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          qraw[r][2 * j] = qp[4 * j + 2 * hh];
          qraw[r][2 * j + 1] = qp[4 * j + 2 * hh + 1];
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) qraw[r][c] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kInsPer; ++u) {
      const int t = (int)threadIdx.x + u * S::kThreads;
      ci[u] = t < 16 * M ? t : t - 16 * M;  // chunk of K or V
      ins_v_chunk[u] = t >= 16 * M;
      ins_chunk[u] = fuse_ins && t < 32 * M;
      nraw[u] = u32x4_t{0u, 0u, 0u, 0u};
      if (ins_chunk[u]) {
        const uint16_t* src = (ins_v_chunk[u] ? a.v_new : a.k_new) +
                              (((int64_t)b * M + (ci[u] >> 4)) * a.num_kv_heads + g) * kHeadDim + 8 * (ci[u] & 15);
        nraw[u] = *reinterpret_cast<const u32x4_t*>(src);
      }
    }
  };
  if constexpr (kEarly) load_inputs();
  L = min(L, min(a.max_seq_len, a.max_blocks * a.block_size));
  const int lo_u = (wl < 0) ? 0 : max(0, L - M - wl);
  const int t_first = lo_u / kTile;
  const int t_end = L > 0 ? (L + kTile - 1) / kTile : 0;
  const int ntiles = max(0, t_end - t_first);
  // splits start at t_first, or (row-exact mode) at multiples of tps so that a key meets the
  // same split and key lane in every call
  const int t_base = a.align_splits ? t_first / tps * tps : t_first;
  const int nsplit = (t_end - t_base + tps - 1) / tps;
  if (ntiles == 0) {
    // no visible key for any row: split 0, row group 0 writes the rows as zeros
    if (s == 0 && rg == 0) {
      for (int idx = threadIdx.x; idx < GM * (kHeadDim / 4); idx += S::kThreads) {
        const int r = idx / (kHeadDim / 4), d4 = idx % (kHeadDim / 4);
        const int i = r / G, hq = g * G + (r - i * G);
        store_out4(a.out, a.out_bf16, (((int64_t)b * M + i) * a.num_q_heads + hq) * kHeadDim + 4 * d4,
            f32x4_t{0.f, 0.f, 0.f, 0.f});
      }
    }
    return;
  }
  if (s >= nsplit) return;
  // in-kernel split merge: count the resident work groups of the pair
  uint32_t* const ctl = a.ws_ctl + kCtlStride * (int64_t)bg;  // counters and claim bits of the pair
  const bool fused = a.fused_combine && nsplit > 1;
  const int group_wgs = nsplit * RG;  // work groups that write partials of this pair
  if (fused && threadIdx.x == 0)
    __hip_atomic_fetch_add(&ctl[kCtlStarted], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int tb = t_base + s * tps;
  int te = min(tb + tps, t_end);
  if (a.clip_rows) {
    // long query windows: only the tiles some row of this work group can see (past its last
    // row's position, or before its first row's window, every key is masked for all its rows).
    // The start moves by whole steps of KL tiles, so every tile keeps its key lane and the
    // result is bitwise that of the full range; an empty range still writes its split partial
    // (l = 0).
    const int p_lo = L - M + row0 / G;
    const int p_hi = L - M + (min(row0 + kRows, GM) - 1) / G;
    te = max(tb, min(te, p_hi < 0 ? 0 : p_hi / kTile + 1));
    if (wl >= 0) {
      const int t_lo = min(te, max(0, p_lo - wl) / kTile);
      if (t_lo > tb) tb += (t_lo - tb) / KL * KL;
    }
  }
  if (wl >= 0) {
    lb0 = tb >> bshift;
    if (lb0 + lane < a.max_blocks) bt_lo = btrow[lb0 + lane];
    if (lb0 + lane + 64 < a.max_blocks) bt_hi = btrow[lb0 + lane + 64];
  }
  const int lo_max = (wl < 0) ? 0 : max(0, L - 1 - wl);  // largest row window start
  const int p_min = L - M;                               // smallest row position
  if constexpr (!kEarly) load_inputs();
  // positions of the wave's query rows (-1: padding row)
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int pr = row0 + rl[r];
    rpos[r] = pr < GM ? L - M + pr / G : -1;
  }
  // Complete the page-table, Q and new-token loads through an asm that redefines their
  // registers: later reads carry no load dependence, so the compiler adds no wait on the
  // DMAs below, whose counts the loop relies on.
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(bt_lo), "+v"(bt_hi), "+v"(ks)::"memory");
#pragma unroll
  for (int r = 0; r < RW; ++r)
    asm volatile(""
                 : "+v"(qraw[r][0]), "+v"(qraw[r][1]), "+v"(qraw[r][2]), "+v"(qraw[r][3]), "+v"(qraw[r][4]),
                   "+v"(qraw[r][5]), "+v"(qraw[r][6]), "+v"(qraw[r][7])::"memory");
  if constexpr (kIns) {
#pragma unroll
    for (int u = 0; u < kInsPer; ++u) asm volatile("" : "+v"(nraw[u])::"memory");
    asm volatile("" : "+v"(vs_ins)::"memory");
  }
  if constexpr (kIns) {
    if (a.cos_sin) {
      // Q/K RMSNorm + RoPE of the raw new tokens, as fkv_qk_norm_rope_insert computes them. New
      // K rows: 16 consecutive threads per token (the V chunks' threads compute and discard);
      // table rows are clamped into the table for threads without a token.
#pragma unroll
      for (int u = 0; u < kInsPer; ++u) {
        const int p = min(max(L - M + (ci[u] >> 4), 0), a.max_seq_len - 1);
        const u32x4_t wk = *reinterpret_cast<const u32x4_t*>(a.k_w + 8 * (ci[u] & 15));
        const u32x4_t z = norm_rope16(nraw[u], wk, ci[u] & 15, a.eps, a.cos_sin + (int64_t)p * kHeadDim);
        if (!ins_v_chunk[u]) nraw[u] = z;
      }
      // the wave's query rows (padding rows stay zero)
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        u32x4_t qn[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) qn[c] = qraw[r][c];
        norm_rope_q64(qn, a.q_w, hh, a.eps, a.cos_sin + (int64_t)max(rpos[r], 0) * kHeadDim);
        if (rpos[r] >= 0)
#pragma unroll
          for (int c = 0; c < 8; ++c) qraw[r][c] = qn[c];
      }
    }
  }
  const float C = a.softmax_scale * ks * kLog2e;
  auto block_of = [&](int tile) -> int {
    const int e = (tile >> bshift) - lb0;
    return __builtin_amdgcn_readlane(e < 64 ? bt_lo : bt_hi, e & 63);
  };

  // ---- this wave's DMA chunks: kPerWave fixed (key lane, chunk) pairs per step
  const int nsteps = (te - tb + KL - 1) / KL;
  const int64_t slab_bytes = (int64_t)a.block_size * kHeadDim;
  uint32_t src_off[S::kPerWave];
  int dma_tl[S::kPerWave];
  const unsigned char* dma_pool[S::kPerWave];
  uint32_t dma_lds[S::kPerWave];
#pragma unroll
  for (int u = 0; u < S::kPerWave; ++u) {
    const int qq = w * S::kPerWave + u;
    const int tl = qq / S::kChunks, j = qq % S::kChunks;
    dma_tl[u] = tl;
    dma_pool[u] = j >= 4 ? a.v_pool : a.k_pool;
    dma_lds[u] = (uint32_t)(tl * S::kTileBytes + j * 1024);
    if (j < 4) {
      src_off[u] = (uint32_t)(key_of_row(n) * kHeadDim + 32 * j + 16 * hh);
    } else {
      const int cp = (j - 4) >> 1, aa = (j - 4) & 1;
      src_off[u] = (uint32_t)((2 * cp + hh) * 1024 + 512 * aa + 16 * n);
    }
  }
  auto issue = [&](int i) {
    unsigned char* slot = body + (i % S::kDepth) * S::kStepBytes;
#pragma unroll
    for (int u = 0; u < S::kPerWave; ++u) {
      // a tile past the split's end re-fetches its last tile (same instruction count per step)
      const int tile = min(tb + KL * i + dma_tl[u], te - 1);
      int blk = block_of(tile);
      blk = ((unsigned)blk < (unsigned)a.num_blocks) ? blk : 0;
      const int64_t off = ((int64_t)blk * a.num_kv_heads + g) * slab_bytes + (int64_t)(tile & bshift) * (kTile * kHeadDim);
      const unsigned char* src = dma_pool[u] + off + src_off[u];
      // explicit void pointers: the host pass otherwise drops the kernel's launch stub
      __builtin_amdgcn_global_load_lds((const void*)src, (void*)(slot + dma_lds[u]), 16, 0, 0);
    }
  };
  const uint32_t ring_lane = (uint32_t)(uintptr_t)body + (uint32_t)(kl * S::kTileBytes) + 16u * (uint32_t)lane;

  // ---- online-softmax state of the lane's rows (one per row tile of the wave)
  f32x16_t o[RW][4];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[r][dt][v] = 0.f;
  float m_ref[RW], lsum[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    m_ref[r] = kRefInit;
    lsum[r] = 0.f;
  }

  // ---- S^T = K Q^T of one tile for every row tile of the wave (each fp8 -> bf16 K chunk
  // is converted once and feeds one MFMA per row tile)
  auto qk = [&](const TileRegs32<true>& x, f32x16_t (&sc)[RW]) {
    const u32x4_t kraw[4] = {x.k[0][0], x.k[0][1], x.k[1][0], x.k[1][1]};
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[r][v] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const u32x4_t& kr = kraw[c >> 1];
      const bf16x8_t kf = fp8x8_to_bf16x8(kr[(c & 1) * 2], kr[(c & 1) * 2 + 1]);
#pragma unroll
      for (int r = 0; r < RW; ++r) sc[r] = mfma32_bf16(kf, __builtin_bit_cast(bf16x8_t, qraw[r][c]), sc[r]);
    }
  };
  // ---- masking of a tile that is not visible to every row of the KV head: invisible
  // scores become -inf; keys outside [lo_u, L), and every key of an invalid block, may hold
  // stale bytes, so their V bytes are zeroed (0 * NaN cannot occur)
  auto mask = [&](int tile, f32x16_t (&sc)[RW], TileRegs32<true>& x) {
    const int kt = tile * kTile;
    const bool valid = (unsigned)block_of(tile) < (unsigned)a.num_blocks;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int hi = valid ? rpos[r] : -1;
      const int lo = (wl < 0) ? 0 : max(0, rpos[r] - wl);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = kt + 16 * (v >> 3) + 8 * hh + (v & 7);
        const uint32_t bad = (uint32_t)(((j - lo) | (hi - j)) >> 31);
        sc[r][v] = __uint_as_float((bad & 0xFF800000u) | (~bad & __float_as_uint(sc[r][v])));
      }
    }
#pragma unroll
    for (int cp = 0; cp < 2; ++cp) {
      const int k0 = kt + 16 * cp + 8 * hh;
      const int e0 = valid ? min(8, max(0, lo_u - k0)) : 8;
      const int e1 = min(8, max(0, L - k0));
      if (e0 > 0 || e1 < 8) {
        const uint64_t keep =
            (e1 >= 8 ? ~0ull : ((1ull << (8 * e1)) - 1)) & (e0 >= 8 ? 0ull : ~((1ull << (8 * e0)) - 1));
        const uint32_t klo = (uint32_t)keep, khi = (uint32_t)(keep >> 32);
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
          x.v[2 * cp + aa][0] &= klo;
          x.v[2 * cp + aa][1] &= khi;
          x.v[2 * cp + aa][2] &= klo;
          x.v[2 * cp + aa][3] &= khi;
        }
      }
    }
  };
  auto interior = [&](int tile) -> bool {
    const int kt = tile * kTile;
    return ((unsigned)block_of(tile) < (unsigned)a.num_blocks) && (kt >= lo_max) && (kt + kTile - 1 <= p_min);
  };
  // ---- probabilities of row tile r against its current reference; the lane's sum is the
  // range check
  auto probs = [&](const f32x16_t& sc, float mr, uint32_t (&hw)[8]) -> float {
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(fmaf(sc[v], C, -mr));
#pragma unroll
    for (int k = 0; k < 8; ++k) hw[k] = pack_f16(p[2 * k], p[2 * k + 1]);
    // the row sum uses the same rounded probabilities the PV product sees
    const f16x2_t one2 = __builtin_bit_cast(f16x2_t, 0x3C003C00u);
    float l = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, hw[k]), one2, l, false);
    return l;
  };
  // cold path: exact row maximum; raise the reference of rows exceeded by more than
  // kLazyTau, rescale those rows, recompute the probabilities
  auto raise = [&](int r, const f32x16_t& sc, uint32_t (&hw)[8], float& lt) {
    float mx = sc[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sc[v]);
    const float cand = pair_max(mx) * C;  // -inf when the row sees no key of this tile
    const bool up = cand > m_ref[r] + kLazyTau;
    if (__builtin_amdgcn_ballot_w64(up) != 0) {
      const float alpha = up ? __builtin_amdgcn_exp2f(m_ref[r] - cand) : 1.0f;
      lsum[r] *= alpha;
      if constexpr (RW == 2) acc_fence32(o[r]);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[r][dt] *= alpha;
      m_ref[r] = up ? cand : m_ref[r];
      lt = probs(sc, m_ref[r], hw);
    }
  };
  // ---- O^T += V^T P^T: d-tile 2a+b, key half c' reads bytes 8b..8b+7 of V chunk (c', a);
  // each converted V operand feeds one MFMA per row tile
  auto pv = [&](const TileRegs32<true>& x, const uint32_t (&hw)[RW][8]) {
    f16x8_t P0[RW], P1[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      P0[r] = __builtin_bit_cast(f16x8_t, u32x4_t{hw[r][0], hw[r][1], hw[r][2], hw[r][3]});
      P1[r] = __builtin_bit_cast(f16x8_t, u32x4_t{hw[r][4], hw[r][5], hw[r][6], hw[r][7]});
    }
    if constexpr (RW == 2) {
      f16x8_t va[4], vb[4];  // d-tile 2a+b: key half 0, key half 1
#pragma unroll
      for (int aa = 0; aa < 2; ++aa)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          va[2 * aa + bb] = fp8x8_to_f16x8(x.v[aa][2 * bb], x.v[aa][2 * bb + 1]);
          vb[2 * aa + bb] = fp8x8_to_f16x8(x.v[2 + aa][2 * bb], x.v[2 + aa][2 * bb + 1]);
        }
      pv32_f16_agpr_rw2(o[0], o[RW - 1], va, vb, P0[0], P1[0], P0[RW - 1], P1[RW - 1]);
    } else {
#pragma unroll
      for (int aa = 0; aa < 2; ++aa)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const u32x4_t& v0 = x.v[aa];
          const u32x4_t& v1 = x.v[2 + aa];
          const f16x8_t va = fp8x8_to_f16x8(v0[2 * bb], v0[2 * bb + 1]);
          const f16x8_t vb = fp8x8_to_f16x8(v1[2 * bb], v1[2 * bb + 1]);
          pv32_f16(o[0][2 * aa + bb], va, P0[0]);
          pv32_f16(o[0][2 * aa + bb], vb, P1[0]);
        }
    }
  };

  // ---- fused insert ("Laguna S 2.1 INT4 -- calibrated FP8 KV on Intel B70", section "Initial
  // optimization order": scaled E4M3 insertion; its fusion into the attention call is the
  // next step named there). New token i sits at position L - M + i. Every group whose key
  // range holds new positions encodes them and stores their codes into the pool itself (the
  // row groups of a split store the same bytes), before it requests a ring step holding a
  // new key: its later DMAs then read the codes from memory like any other key.
  // Ordering, all within the work group: the stores are issued before the DMAs of those
  // steps; vector memory operations complete in issue order, so once a wave's wait shows a
  // DMA issued after its stores complete, the stores are complete too, and the barrier that
  // follows the wait extends that to every wave of the group (workgroup-scope release and
  // acquire: the group's waves share one CU and its L1, which the stores write through).
  const int pn0 = max(0, L - M);  // first new position
  const int tn0 = pn0 / kTile;    // first tile holding a new key
  const bool ins = fuse_ins && L > pn0 && pn0 < te * kTile && L > tb * kTile;  // uniform
  // first step holding a new key; steps from it on are requested after the stores complete
  const int sn0 = ins ? max(0, tn0 - tb) / KL : S::kDepth;
  // steps requested before the encode (one, so the encode is not queued behind the others),
  // and before the first barrier (the rest right after it)
  const int pre = !ins ? S::kDepth - 1 : (sn0 == 0 ? 0 : 1);
  const int lim = (!ins || sn0 == 0) ? S::kDepth - 1 : min(sn0, S::kDepth - 1);

  // ---- the ring's first steps are requested before anything else: they need only the
  // page table
  const uint32_t slot0 = ring_lane;
#pragma unroll
  for (int p = 0; p < S::kDepth - 1; ++p)
    if (p < pre && p < nsteps) issue(p);
  if (ins) {
#pragma unroll
    for (int u = 0; u < kInsPer; ++u) {
      const int p = L - M + (ci[u] >> 4);  // this chunk's token position
      // physical block of p from the split's page-table window (lanes hold entries lb0 +
      // lane and lb0 + 64 + lane); only positions in this group's key range are stored
      const int e = min(max((p >> (5 + bshift)) - lb0, 0), 127);
      const int blo = __builtin_amdgcn_ds_bpermute((e & 63) * 4, bt_lo);
      const int bhi = __builtin_amdgcn_ds_bpermute((e & 63) * 4, bt_hi);
      const int blk = e < 64 ? blo : bhi;
      if (ins_chunk[u] && p >= 0 && p >= tb * kTile && p < te * kTile && (unsigned)blk < (unsigned)a.num_blocks) {
        uint32_t c0, c1;
        e4m3_encode8(nraw[u], ins_v_chunk[u] ? vs_ins : ks, c0, c1);
        const int d0 = 8 * (ci[u] & 15);
        const int off = p & (a.block_size - 1);
        const int64_t slab = ((int64_t)blk * a.num_kv_heads + g) * slab_bytes;
        if (!ins_v_chunk[u]) {
          *reinterpret_cast<u32x2_t*>(const_cast<uint8_t*>(a.k_pool) + slab + off * kHeadDim + d0) = u32x2_t{c0, c1};
        } else {
          uint8_t* vp = const_cast<uint8_t*>(a.v_pool) + slab + (off >> 3) * 1024 + d0 * 8 + (off & 7);
#pragma unroll
          for (int j = 0; j < 8; ++j) vp[j * 8] = (uint8_t)((j < 4 ? c0 : c1) >> (8 * (j & 3)));
        }
      }
    }
    // the first step holds a new key: every store completes before any DMA
    if (sn0 == 0) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  }
#pragma unroll
  for (int p = 0; p < S::kDepth - 1; ++p)
    if (p >= pre && p < lim && p < nsteps) issue(p);

  // ---- the pipeline. kDepth steps are in flight; one barrier per step publishes a step
  // and certifies that every wave has read the slot the next request overwrites. A wave
  // computes S^T of tile i+1 in the same block as the probabilities of tile i, so MFMA and
  // VALU work interleave, then O^T += V^T P^T of tile i.
  const int nfull = wave_rows ? (te - tb - kl + KL - 1) / KL : 0;  // this wave's tiles
  wait_steps<S::kPerWave, S::kDepth - 2>(min(nsteps - 1, lim - 1));
  asm volatile("s_barrier" ::: "memory");
#pragma unroll
  for (int p = 1; p < S::kDepth; ++p)
    if (p >= lim && p < nsteps) issue(p);
  TileRegs32<true> xa, xb;
  f32x16_t sa[RW], sb[RW];
  if (nfull > 0) {
    read_slot<true>(slot0, xa);
    qk(xa, sa);
  }
  // The barrier part of step i (every wave takes part in every step's barrier).
  auto sync_step = [&](int i) {
    if (i + 1 < nsteps) {
      wait_steps<S::kPerWave, S::kDepth - 2>(min(nsteps - 2 - i, S::kDepth - 2));
      asm volatile("s_barrier" ::: "memory");
      if (i + S::kDepth < nsteps) issue(i + S::kDepth);
    }
  };
  // probabilities of the current tile, the rare raise, then O^T += V^T P^T
  auto finish_tile = [&](const TileRegs32<true>& xc, uint32_t (&hw)[RW][8], float (&lt)[RW], f32x16_t (&sc)[RW]) {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      if (__builtin_amdgcn_ballot_w64(!(lt[r] <= kAcceptSum)) != 0) raise(r, sc[r], hw[r], lt[r]);
      lsum[r] += lt[r];
    }
    pv(xc, hw);
  };
  // Step i of a wave that has a tile at i + 1 too: S^T of the next tile and the
  // probabilities of this one come in one straight-line block, so their MFMA and VALU work
  // can interleave.
  auto full_step = [&](int i, TileRegs32<true>& xc, TileRegs32<true>& xn, f32x16_t (&sc)[RW], f32x16_t (&sn)[RW]) {
    sync_step(i);
    const int tile = tb + KL * i + kl;
    if (!interior(tile)) mask(tile, sc, xc);
    read_slot<true>(slot0 + (uint32_t)(((i + 1) % S::kDepth) * S::kStepBytes), xn);
    uint32_t hw[RW][8];
    float lt[RW];
    // the block of S^T products and probabilities issues at raised wave priority, the P.V
    // products at the normal one (measured: about 1 % faster steps at 8k and 32k than
    // without, slower with the priority on the P.V block or alternating between the waves)
    __builtin_amdgcn_s_setprio(1);
    qk(xn, sn);
#pragma unroll
    for (int r = 0; r < RW; ++r) lt[r] = probs(sc[r], m_ref[r], hw[r]);
    __builtin_amdgcn_s_setprio(0);
    finish_tile(xc, hw, lt, sc);
  };
  // the wave's last tile
  auto last_step = [&](int i, TileRegs32<true>& xc, f32x16_t (&sc)[RW]) {
    sync_step(i);
    const int tile = tb + KL * i + kl;
    if (!interior(tile)) mask(tile, sc, xc);
    uint32_t hw[RW][8];
    float lt[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) lt[r] = probs(sc[r], m_ref[r], hw[r]);
    finish_tile(xc, hw, lt, sc);
  };
  int i = 0;
  for (; i + 1 < nfull; ++i) {
    full_step(i, xa, xb, sa, sb);
    xa = xb;
#pragma unroll
    for (int r = 0; r < RW; ++r) sa[r] = sb[r];
  }
  if (i < nfull) {
    last_step(i, xa, sa);
    ++i;
  }
  for (; i < nsteps; ++i) sync_step(i);  // no tile of this wave left (barriers still counted)
  // The exchange area and the staged rows below overlay the ring. After the last step barrier
  // another wave (one with more tiles, or a slower one) may still read the ring slot of the
  // last step. Where they fit (kWrap), the exchange area takes the ring's other slots, from
  // the slot after that one on (addresses modulo the ring), and the staged rows follow it,
  // so a wave writes its exchange data as soon as its loop ends; else a barrier first.
  constexpr int kStageRow = kHeadDim * 4;  // bytes of a staged row (no padding: swizzled)
  constexpr bool kWrap = S::kXch <= S::kRing - S::kStepBytes && S::kXch + 32 * RT * kStageRow <= S::kRing &&
                         (S::kRing & (S::kRing - 1)) == 0;
  const uint32_t xbase = kWrap ? (uint32_t)((max(nsteps, 1) % S::kDepth) * S::kStepBytes) : 0u;
  if constexpr (!kWrap) __syncthreads();

  // ---- merge the KL key lanes of each row tile in a fixed order. Every wave writes its
  // (m, l) and its unscaled accumulators of the groups other key lanes own once every wave
  // has left the loop; after one more barrier each owner rescales and sums its groups over
  // the key lanes in lane order and stages the merged rows.
  if constexpr (RW == 2) {
    acc_fence32(o[0]);
    acc_fence32(o[1]);
  }
  // Output group gi = 4a + i holds dims 64a + 16i + 8hh + 0..7: elements 4i..4i+3 of d-tiles
  // 2a and 2a + 1. Key lane kl owns groups kl*GPK .. +GPK-1 and receives them from the others.
  constexpr int kGpk = 8 / KL;
  // [owner][row tile][source, owner skipped][kGpk*2 quads][64 lanes][4 floats]: 16-byte,
  // lane-contiguous accesses
  auto xch = [&](int owner, int rt, int src, int f4) -> f32x4_t& {
    const int slot = src < owner ? src : src - 1;
    uint32_t off = (uint32_t)((((owner * RT + rt) * (KL - 1) + slot) * (kGpk * 2) + f4) * 64 + lane) * 16u;
    if constexpr (kWrap) off = (xbase + off) & (uint32_t)(S::kRing - 1);
    return *reinterpret_cast<f32x4_t*>(body + off);
  };
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const float lrow = pair_sum(lsum[r]);
    if (hh == 0) {
      sm_m[kl * kRows + rl[r]] = m_ref[r];
      sm_l[kl * kRows + rl[r]] = lrow;
    }
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) {
      const int owner = gi / kGpk;
      if (owner == kl) continue;
      const int aa = gi >> 2, ii = gi & 3;
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const f32x16_t& acc = o[r][2 * aa + bb];
        xch(owner, rtg * RW + r, kl, (gi % kGpk) * 2 + bb) =
            f32x4_t{acc[4 * ii], acc[4 * ii + 1], acc[4 * ii + 2], acc[4 * ii + 3]};
      }
    }
  }
  __syncthreads();  // every exchange write is done
  const bool direct = (nsplit == 1);
  const float vsc = *a.v_scale;
  const int64_t part = ((int64_t)b * a.num_kv_heads + g) * a.max_splits + s;
  // The merged rows are staged row-major in LDS so that the group's stores write whole
  // contiguous rows: 4-float column c of row r at c ^ (r % 32) (kWrap: conflict-free without
  // padding, placed after the exchange area modulo the ring), else at rows padded to
  // kStageStride floats.
  constexpr int kStageStride = S::kStageStride;
  auto stage = [&](int row, int col) -> float* {  // col: a multiple of 4
    if constexpr (kWrap) {
      const uint32_t c4 = (uint32_t)(col >> 2) ^ (uint32_t)(row & 31);
      const uint32_t off = (xbase + (uint32_t)S::kXch + (uint32_t)row * kStageRow + c4 * 16u) & (uint32_t)(S::kRing - 1);
      return reinterpret_cast<float*>(body + off);
    } else {
      return reinterpret_cast<float*>(body + S::kXch) + row * kStageStride + col;
    }
  };
  __shared__ float sm_row[2 * kRows];                       // merged (M, L) per row
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    // weight of key lane k: 2^(m_k - M); the lane's own weight scales its accumulators
    float ew[KL];
    float Mrow = sm_m[rl[r]];
#pragma unroll
    for (int k = 1; k < KL; ++k) Mrow = fmaxf(Mrow, sm_m[k * kRows + rl[r]]);
    float Lrow = 0.f;
#pragma unroll
    for (int k = 0; k < KL; ++k) {
      ew[k] = __builtin_amdgcn_exp2f(sm_m[k * kRows + rl[r]] - Mrow);
      Lrow += sm_l[k * kRows + rl[r]] * ew[k];
    }
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) {
      // compile-time group index (the accumulators are only indexed by constants)
      if (gi / kGpk != kl) continue;
      const int gl = gi % kGpk;
      const int aa = gi >> 2, ii = gi & 3;
      float o8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o8[e] = 0.f;
#pragma unroll
      for (int src = 0; src < KL; ++src) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const f32x16_t& acc = o[r][2 * aa + bb];
          const f32x4_t val = (src == kl) ? f32x4_t{acc[4 * ii], acc[4 * ii + 1], acc[4 * ii + 2], acc[4 * ii + 3]}
                                          : xch(kl, rtg * RW + r, src, gl * 2 + bb);
#pragma unroll
          for (int k = 0; k < 4; ++k) o8[2 * k + bb] += val[k] * ew[src];
        }
      }
      const int d0 = 64 * (gi >> 2) + 16 * (gi & 3) + 8 * hh;
      *reinterpret_cast<f32x4_t*>(stage(rl[r], d0)) = f32x4_t{o8[0], o8[1], o8[2], o8[3]};
      *reinterpret_cast<f32x4_t*>(stage(rl[r], d0 + 4)) = f32x4_t{o8[4], o8[5], o8[6], o8[7]};
    }
    if (kl == 0 && hh == 0) {
      sm_row[rl[r]] = Mrow;
      sm_row[kRows + rl[r]] = Lrow;
    }
  }
  __syncthreads();
  const int nrows = max(0, min(kRows, GM - row0));  // real rows of this work group
  if (direct) {
    for (int idx = threadIdx.x; idx < nrows * (kHeadDim / 4); idx += S::kThreads) {
      const int rr = idx / (kHeadDim / 4), d4 = idx % (kHeadDim / 4);
      const int i = (row0 + rr) / G, hq = g * G + (row0 + rr - i * G);
      const float lw = sm_row[kRows + rr];
      const float mul = lw > 0.f ? vsc / lw : 0.f;
      store_out4(a.out, a.out_bf16, (((int64_t)b * M + i) * a.num_q_heads + hq) * kHeadDim + 4 * d4,
          *reinterpret_cast<const f32x4_t*>(stage(rr, 4 * d4)) * mul);
    }
  } else {
    // the partial: rows_pad x 128 fp32 (only the GM real rows written), then (M, L) per row
    const __amdgpu_buffer_rsrc_t prsrc =
        coherent_rsrc(a.ws_o + part * a.rows_pad * kHeadDim, (uint32_t)(a.rows_pad * kHeadDim * 4));
    for (int idx = threadIdx.x; idx < nrows * (kHeadDim / 4); idx += S::kThreads) {
      const int rr = idx / (kHeadDim / 4), d4 = idx % (kHeadDim / 4);
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stage(rr, 4 * d4));
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), prsrc, (row0 * (kHeadDim / 4) + idx) * 16, 0,
                                             kCoherent);
    }
    const __amdgpu_buffer_rsrc_t mlrsrc = coherent_rsrc(a.ws_ml + part * 2 * a.rows_pad, 2 * a.rows_pad * 4);
    for (int idx = threadIdx.x; idx < 2 * nrows; idx += S::kThreads) {
      const int which = idx / nrows, rr = idx % nrows;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sm_row[which * kRows + rr]), mlrsrc,
                                            (which * a.rows_pad + row0 + rr) * 4, 0, kCoherent);
    }
  }

  // ---- in-kernel merge of the pair's splits (grids that fit on the chip at once). The
  // output is cut into one slice per work group of the pair; a slice is merged by whoever
  // sets its claim bit first. A work group waits for the other splits only when all of them
  // have started, i.e. are resident and will finish without needing this CU; it then claims
  // its own slice (finish ticket f) and requests the partials in the same round trip. The
  // last work group to finish merges its own slice and then claims every other slice at
  // once, so waiting is never needed for completion and every output quad is written exactly
  // once. The last work group to leave returns the counters to zero for the next call.
  if (fused) {
    __shared__ int sh_role, sh_f, sh_claim;
    __shared__ uint32_t sh_won[8];
    const int quads = GM * 32;
    const int per = max((quads + group_wgs - 1) / group_wgs, (quads + 255) / 256);
    const int nslices = (quads + per - 1) / per;  // <= group_wgs, <= 256
    const int nwords = (nslices + 31) / 32;
    const bool fast = nsplit <= kFastSplits;
    const uint32_t ns = (uint32_t)group_wgs;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's coherent partial stores are done
    __syncthreads();                                   // ... and every other thread's
    if (threadIdx.x == 0) {
      const uint32_t f = __hip_atomic_fetch_add(&ctl[kCtlFinished], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t started = __hip_atomic_load(&ctl[kCtlStarted], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int role = (f == ns - 1) ? 2 : 0;  // 0: leave, 1: merge the own slice if still unclaimed, 2: last
      if (!role && started == ns) {
        for (int it = 0; it < kSpinLimit; ++it) {
          if (__hip_atomic_load(&ctl[kCtlFinished], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ns) {
            role = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(4);
        }
      }
      sh_role = role;
      sh_f = (int)f;
    }
    __syncthreads();
    const int role = sh_role, f = sh_f;
    // merges slice k; claimed says whether this group owns it (read after the loads are in flight)
    auto merge_own = [&](int k, bool claim) {
      const int q0 = k * per, cnt = min(per, quads - q0);
      const int t = threadIdx.x;
      if (fast) {
        // a slice can hold more quads than the group has threads (few work groups per pair)
        for (int t0 = 0; t0 < cnt; t0 += S::kThreads) {
          const int tq = t0 + t;
          QuadLoads x;
          if (tq < cnt) quad_issue(a, b, g, nsplit, q0 + tq, x);
          if (claim && t0 == 0) {
            if (t == 0) {
              const uint32_t bit = 1u << (k & 31);
              const uint32_t old =
                  __hip_atomic_fetch_or(&ctl[kCtlClaim + (k >> 5)], bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              sh_claim = (old & bit) == 0;
            }
            __syncthreads();
            if (!sh_claim) break;  // uniform: the last finisher took the slice
          }
          if (tq < cnt) quad_finish(a, b, g, nsplit, q0 + tq, x, vsc);
        }
      } else {
        if (claim) {
          if (t == 0) {
            const uint32_t bit = 1u << (k & 31);
            const uint32_t old =
                __hip_atomic_fetch_or(&ctl[kCtlClaim + (k >> 5)], bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sh_claim = (old & bit) == 0;
          }
          __syncthreads();
        }
        if (!claim || sh_claim) merge_slice<S::kThreads>(a, b, g, nsplit, q0, cnt, vsc, reinterpret_cast<float*>(body));
      }
    };
    // one merge site: the own slice first, then (last finisher) every slice won in the batch claim
    int k = (role != 0 && f < nslices) ? f : -1;
    bool claim = role == 1, batch = role == 2;
    int wd = 0;
    uint32_t won = 0u;
    for (;;) {
      if (k >= 0) merge_own(k, claim);
      if (batch) {
        batch = false;
        claim = false;
        if ((int)threadIdx.x < nwords) {
          const int w0 = 32 * threadIdx.x;
          const int nb = min(32, nslices - w0);
          uint32_t mask = nb >= 32 ? ~0u : ((1u << nb) - 1u);
          if (f >= w0 && f < w0 + 32) mask &= ~(1u << (f - w0));
          const uint32_t old =
              __hip_atomic_fetch_or(&ctl[kCtlClaim + threadIdx.x], mask, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          sh_won[threadIdx.x] = mask & ~old;
        }
        __syncthreads();
        won = role == 2 ? sh_won[0] : 0u;
      } else if (role != 2) {
        break;
      }
      while (won == 0u && role == 2 && ++wd < nwords) won = sh_won[wd];
      if (won == 0u) break;
      k = 32 * wd + __builtin_ctz(won);
      won &= won - 1u;
    }
    if (threadIdx.x == 0) {
      const uint32_t e = __hip_atomic_fetch_add(&ctl[kCtlExited], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (e == ns - 1) {
        __hip_atomic_store(&ctl[kCtlStarted], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctl[kCtlFinished], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctl[kCtlExited], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int wd = 0; wd < nwords; ++wd)
          __hip_atomic_store(&ctl[kCtlClaim + wd], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

}  // namespace

template <int RT, int KL, int RW>
static hipError_t launch_m32_t(const DecodeArgs& a, hipStream_t stream) {
  const int64_t pairs = (int64_t)a.num_seqs * a.num_kv_heads;
  const int64_t per_pair = (int64_t)a.max_splits * a.row_groups;
  const int64_t grid = a.xcd_pairs ? (pairs + 7) / 8 * 8 * per_pair : pairs * per_pair;
  constexpr int kThreads = M32Shape<RT, KL, RW, true>::kThreads;
  // early input loads pay when the grid is about one wave of work groups over the chip (a
  // layer of one sequence); in a large batch grid many work groups leave at once (measured:
  // 8k step -0.9 us, 32-sequence batch +5 % with early loads)
  const bool early = grid <= 2 * 256;
  if (a.k_new) {
    if (early)
      hipLaunchKernelGGL((decode_m32_kernel<RT, KL, RW, true, true, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_m32_kernel<RT, KL, RW, true, true, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  } else {
    if (early)
      hipLaunchKernelGGL((decode_m32_kernel<RT, KL, RW, true, false, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_m32_kernel<RT, KL, RW, true, false, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_m32(const DecodeArgs& a, int rt, int rw, int kl, bool fp8, hipStream_t stream) {
  if (!fp8) return hipErrorInvalidValue;
  if (rw == 2) return (rt == 2 && kl == 4) ? launch_m32_t<2, 4, 2>(a, stream) : hipErrorInvalidValue;
  if (rt == 1 && kl == 8) return launch_m32_t<1, 8, 1>(a, stream);
  if (rt == 1 && kl == 4) return launch_m32_t<1, 4, 1>(a, stream);  // one row tile, four waves
  if (rt == 2 && kl == 4) return launch_m32_t<2, 4, 1>(a, stream);
  if (rt == 4 && kl == 2) return launch_m32_t<4, 2, 1>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fkv
