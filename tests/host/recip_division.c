/* The quantiser's quotient for scales in [2^-32, 2^32]: r = RN(1/s), q0 = RN(x r),
 * q = RN(q0 + RN(x - q0 s) r) (the last two steps fused multiply-adds; P. Markstein,
 * "IA-64 and Elementary Functions", 2000), with q0 kept where |q0| >= 1024 and the sign of x.
 * Part 1: for every BF16 significand x in [1, 2) and [1/2, 1) and every float32 significand
 * s in [1, 2), q equals the IEEE quotient x / s bit for bit (the step is invariant under
 * power-of-two scaling of x and s while nothing under- or overflows).
 * Part 2: for every BF16 pattern x and 260 scales per binade 2^-32..2^31 (1, the all-ones
 * significand and seeded random ones), the E4M3FN code of q equals that of x / s, and q equals
 * x / s bit for bit wherever |x| >= 2^-100 and x / s is a normal float32 below 1024.
 * The E4M3FN rounding here is written from the format (bias 7, 3 mantissa bits, ties to even,
 * saturation at 448, NaN 0x7F) for this check alone. Prints "mismatches N". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t b) { float x; memcpy(&x, &b, 4); return x; }
static uint32_t to_bits(float x) { uint32_t b; memcpy(&b, &x, 4); return b; }

static uint32_t e4m3(float y) {
  const uint32_t b = to_bits(y), sign = (b >> 24) & 0x80u, a = b & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;
  if (a < 0x3C800000u) return sign | (uint32_t)rintf(from_bits(a) * 512.0f);
  return sign | ((((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20)) - (120u << 3));
}

static float quotient(float x, float s, float r) {
  volatile float q0 = x * r; /* a separate rounding, never contracted into the FMA below */
  const float q1 = fmaf(fmaf(-q0, s, x), r, q0);
  return copysignf(fabsf(q0) >= 1024.0f ? q0 : q1, x);
}

int main(void) {
  long bad = 0, total = 0;
#pragma omp parallel for reduction(+ : bad, total) schedule(static)
  for (uint32_t m = 0; m < (1u << 23); ++m) {
    const float s = from_bits(0x3F800000u | m);
    const float r = 1.0f / s;
    for (uint32_t e = 126; e <= 127; ++e)
      for (uint32_t xm = 0; xm < 128; ++xm) {
        const float x = from_bits((e << 23) | (xm << 16));
        bad += to_bits(quotient(x, s, r)) != to_bits(x / s);
        ++total;
      }
  }
  printf("part 1: %ld pairs\n", total);
#pragma omp parallel for reduction(+ : bad, total) schedule(dynamic)
  for (int e = -32; e <= 31; ++e) {
    uint32_t seed = (uint32_t)(e + 1000) * 2654435761u;
    for (int t = 0; t < 260; ++t) {
      uint32_t m = t == 1 ? 0x7FFFFFu : 0u;
      if (t >= 2) { seed = seed * 1664525u + 1013904223u; m = seed >> 9; }
      const float s = from_bits(((uint32_t)(e + 127) << 23) | m);
      const float r = 1.0f / s;
      for (uint32_t p = 0; p < 65536; ++p) {
        const float x = from_bits(p << 16);
        const float qd = x / s, qf = quotient(x, s, r);
        const uint32_t cd = e4m3(qd), cf = e4m3(qf);
        if (isnan(x)) bad += (cf & 0x7F) != 0x7F || (cf & 0x80) != (cd & 0x80);
        else bad += cd != cf;
        if (!isnan(x) && fabsf(x) >= 0x1p-100f && fabsf(qd) >= 0x1p-126f && fabsf(qd) < 1024.0f)
          bad += to_bits(qd) != to_bits(qf);
        ++total;
      }
    }
  }
  printf("total %ld mismatches %ld\n", total, bad);
  return bad != 0;
}
