// Device-side building blocks for gfx950: vector types, the E4M3FN encoder, fp8
// converters, MFMA wrappers and cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fkv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

// Stores output elements e .. e+3 of a [seq][M][Hq][128] result: fp32, or BF16 rounded to
// nearest even (the branch is uniform: one output type per call).
__device__ __forceinline__ void store_out4(float* out, bool bf16, int64_t e, f32x4_t v) {
  if (bf16) {
    const bf16x2_t lo = __builtin_convertvector(f32x2_t{v[0], v[1]}, bf16x2_t);
    const bf16x2_t hi = __builtin_convertvector(f32x2_t{v[2], v[3]}, bf16x2_t);
    *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(out) + e) =
        u32x2_t{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  } else {
    *reinterpret_cast<f32x4_t*>(out + e) = v;
  }
}

constexpr int kHeadDim = 128;
constexpr int kTile = 32;     // keys per attention tile

// ---- E4M3FN encoder --------------------------------------------------------------------
// Round an fp32 value to the nearest E4M3FN code, ties to even, saturating to +-448 for
// |y| >= 448 (infinities included); NaN -> 0x7F | sign. The sign of zero is kept.
// Integer formulation: normals keep the top 3 mantissa bits after adding the
// round-to-nearest-even bias; values below 2^-6 live on the 2^-9 subnormal grid.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t b = __float_as_uint(y);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;          // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;         // >= 448 (0x43E00000), inf included
  if (a < 0x3C800000u) {                             // < 2^-6: multiples of 2^-9
    const float q = __uint_as_float(a) * 512.0f;     // exact power-of-two scaling
    return sign | (uint32_t)__builtin_rintf(q);      // RNE to an integer 0..8 (8 = 2^-6)
  }
  const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;  // RNE to 3 mantissa bits
  return sign | (r - (120u << 3));                   // rebias exponent 127 -> 7
}

// Two fp32 values -> two E4M3FN bytes by the hardware conversion (v_cvt_pk_fp8_f32, round to
// nearest even), placed in the low (kHigh = false) or high half of old. For every fp32 input
// with |y| < 448 (NaN excluded) its byte equals e4m3_encode(y): checked on the box over all
// 2^32 patterns (csrc/probe/e4m3_check.hip, run by the GPU conversion test). It does not
// saturate like e4m3_encode, and a NaN's code loses its sign, so the callers route such
// values to e4m3_encode.
template <bool kHigh>
__device__ __forceinline__ uint32_t e4m3_cvt2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, kHigh);
}

// Eight BF16 values (16 bytes; element j in the high or low half of word j/2) -> eight
// E4M3FN codes: code j = e4m3_encode(fp32(x_j) / scale) with the correctly rounded fp32
// quotient, in byte j%4 of lo (j < 4) or hi (j >= 4). Cache insertion, standalone or fused
// into decode, stores exactly these bytes.
//
// Quotient. For scales in [2^-32, 2^32] it comes from one reciprocal r = RN(1/scale) and
// Markstein's residual correction (P. Markstein, "IA-64 and Elementary Functions", 2000):
// q0 = RN(x r), e = RN(x - q0 scale) (exact, one FMA), q = RN(q0 + e r) (one FMA). With a
// BF16 dividend (8 significant bits) one correction gives the correctly rounded quotient for
// every pair of significands (checked exhaustively against IEEE division on the CPU, with
// every BF16 dividend against scales sampled over the whole range: the host division test).
// Where that argument does not reach, the codes still agree: for |q0| >= 1024 both quotients
// saturate (q0 is kept; it may be infinite), and for |x| < 2^-100 the residual may underflow
// but the quotient lies far below the smallest E4M3 subnormal, so both encode to zero. The
// sign is x's (scale > 0), NaN included. Other scales (zero, negative, tiny, huge, NaN) take
// the IEEE division.
// Code. When all eight quotients have |q| < 448 (an integer test on the magnitude bits, which
// also catches infinities and NaN) the hardware conversion makes the bytes; else e4m3_encode.
__device__ __forceinline__ void e4m3_encode8(const u32x4_t& in, float scale, uint32_t& lo, uint32_t& hi) {
  float x[8], q[8], q0[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t w = in[j >> 1];
    x[j] = __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
  const bool recip = scale >= 0x1p-32f && scale <= 0x1p32f;
  if (recip) {
    const float r = __fdiv_rn(1.0f, scale);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      q0[j] = x[j] * r;
      q[j] = __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0[j], scale, x[j]), r, q0[j]), x[j]);
    }
  } else {
    // a side effect the compiler cannot speculate: without it the eight divisions of this
    // rare branch are hoisted and computed for every chunk, then discarded by selects
    asm volatile("");
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = q0[j] = __fdiv_rn(x[j], scale);
  }
  // largest magnitude, as bits shifted past the sign: NaN > infinity > every finite value
  uint32_t m = 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = max(m, __float_as_uint(q[j]) << 1);
  if (m < (0x43E00000u << 1)) {
    lo = e4m3_cvt2<true>(q[2], q[3], e4m3_cvt2<false>(q[0], q[1], 0u));
    hi = e4m3_cvt2<true>(q[6], q[7], e4m3_cvt2<false>(q[4], q[5], 0u));
  } else {
    uint32_t c[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float qq = (recip && __builtin_fabsf(q0[j]) >= 1024.0f) ? q0[j] : q[j];
      c[j >> 2] |= e4m3_encode(qq) << (8 * (j & 3));
    }
    lo = c[0];
    hi = c[1];
  }
}

// ---- per-head RMSNorm + rotate-half RoPE in one fixed float32 order ------------------------
// ("Laguna S 2.1 INT4 -- calibrated FP8 KV on Intel B70", section "Initial optimization
// order": the scaled insert sits at the Q/K norm + RoPE step.) The order, followed exactly so
// that BF16 roundings and E4M3 codes are reproducible: each group of 8 consecutive dims sums
// its squares in dim order; the 16 group sums combine pairwise at group distances 1, 2, 4, 8;
// r = 1 / sqrt(s / 128 + eps) with the correctly rounded square root (sqrtf here; HIP's
// __fsqrt_rn maps to the native one) and IEEE division; y = bf16((x r) w); for d < 64,
// z_d = bf16(y_d c_d - y_(d+64) s_d) and z_(d+64) = bf16(y_(d+64) c_d + y_d s_d), every product
// and sum rounded on its own (no FMA contraction).

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// One head vector over 16 consecutive lanes, lane c holding dims 8c .. 8c+7 (xin: BF16 x, win:
// BF16 weights of those dims), row: the position's table row (64 cosines, then 64 sines).
// Every lane of the wave must call it (16-wide shuffles). Returns the lane's 8 BF16 results.
__device__ __forceinline__ u32x4_t norm_rope16(const u32x4_t& xin, const u32x4_t& win, int c, float eps,
                                               const float* row) {
#pragma clang fp contract(off)
  float x[8], w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = (j & 1) ? bf16_hi(xin[j >> 1]) : bf16_lo(xin[j >> 1]);
    w[j] = (j & 1) ? bf16_hi(win[j >> 1]) : bf16_lo(win[j >> 1]);
  }
  float s = x[0] * x[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) s = s + x[j] * x[j];
#pragma unroll
  for (int k = 1; k < 16; k <<= 1) s = s + __shfl_xor(s, k, 16);
  const float rr = __fdiv_rn(1.0f, sqrtf(__fdiv_rn(s, 128.0f) + eps));
  float y[8];
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const uint32_t yb = bf16x2_rne((x[j] * rr) * w[j], (x[j + 1] * rr) * w[j + 1]);
    y[j] = bf16_lo(yb);
    y[j + 1] = bf16_hi(yb);
  }
  const float* cr = row + 8 * (c & 7);
  const f32x4_t c0 = *reinterpret_cast<const f32x4_t*>(cr), c1 = *reinterpret_cast<const f32x4_t*>(cr + 4);
  const f32x4_t s0 = *reinterpret_cast<const f32x4_t*>(cr + 64), s1 = *reinterpret_cast<const f32x4_t*>(cr + 68);
  const float cs[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
  const float sn[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  uint32_t zw[4];
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    float z[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float yp = __shfl_xor(y[j + e], 8, 16);  // dim d + 64 (lanes 0-7) or d - 64 (lanes 8-15)
      const float a0 = y[j + e] * cs[j + e], a1 = yp * sn[j + e];
      z[e] = c < 8 ? a0 - a1 : a0 + a1;
    }
    zw[j >> 1] = bf16x2_rne(z[0], z[1]);
  }
  return u32x4_t{zw[0], zw[1], zw[2], zw[3]};
}

// ---- fp8 -> bf16 / f16 (hardware, exact for every E4M3FN code) -------------------------
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ f16x8_t fp8x8_to_f16x8(uint32_t lo, uint32_t hi) {
  const f16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const f16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const f16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const f16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return f16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// ---- MFMA 16x16x32 ------------------------------------------------------------------------
// Lane l holds A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16] and
// D[4*(l/16) .. +3][l%16] (row index first).
__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f16(f16x8_t a, f16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---- cross-lane reductions over the four 16-lane groups ------------------------------------
// permlane16_swap pairs lane l with l^16, permlane32_swap pairs l with l^32. Both lanes
// of a pair receive (value of the lower lane, value of the upper lane), so the result
// is bitwise identical on all four lanes of a column.
__device__ __forceinline__ float group_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float group_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Two fp32 values -> packed f16, round to nearest even (one v_cvt_pk_f16_f32 on gfx950):
// the attention weights fed to the f16 P.V product and to the row sums.
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)a, (_Float16)b});
}

}  // namespace fkv
