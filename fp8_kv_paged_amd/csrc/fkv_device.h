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

// Eight BF16 values (16 bytes; element j in the high or low half of word j/2) -> eight
// E4M3FN codes: code j = e4m3_encode(fp32(x_j) / scale) with one correctly rounded fp32
// division, in byte j%4 of lo (j < 4) or hi (j >= 4). Cache insertion, standalone or fused
// into decode, stores exactly these bytes.
__device__ __forceinline__ void e4m3_encode8(const u32x4_t& in, float scale, uint32_t& lo, uint32_t& hi) {
  uint32_t c[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t w = in[j >> 1];
    const float x = __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
    c[j >> 2] |= e4m3_encode(__fdiv_rn(x, scale)) << (8 * (j & 3));
  }
  lo = c[0];
  hi = c[1];
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
