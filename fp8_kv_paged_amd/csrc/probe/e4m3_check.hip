// Check of the library's E4M3 conversion helper (not part of libfkv.so): for every fp32 bit
// pattern x, e4m3_cvt2 (the hardware conversion the quantiser uses when every quotient of a
// chunk is below 448 in magnitude) must give the bytes of e4m3_encode (the integer encoder that
// follows the format's definition) for x and -x, each in its own byte of the packed word.
// Counts by class of |x|: below 448, 448 and above (finite), infinite, NaN; and the NaN
// patterns whose byte is not a NaN code. The first 32 mismatching patterns below 448 are kept.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../fkv_device.h"

namespace {

__global__ __launch_bounds__(256) void e4m3_check_kernel(unsigned long long* counts, uint32_t* examples,
                                                         uint32_t top) {
  // patterns (top << 28) + 1024 * thread + k, k < 1024: 2^18 threads cover 2^28 patterns
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  uint32_t local[5] = {0u, 0u, 0u, 0u, 0u};
  for (uint32_t k = 0; k < 1024u; ++k) {
    const uint32_t p = (top << 28) + t * 1024u + k;
    const float x = __uint_as_float(p), y = __uint_as_float(p ^ 0x80000000u);
    const uint32_t w = fkv::e4m3_cvt2<true>(y, x, fkv::e4m3_cvt2<false>(x, y, 0u));
    const uint32_t ex = fkv::e4m3_encode(x), ey = fkv::e4m3_encode(y);
    const uint32_t want = ex | (ey << 8) | (ey << 16) | (ex << 24);
    const uint32_t a = p & 0x7FFFFFFFu;
    const int cls = a > 0x7F800000u ? 3 : a == 0x7F800000u ? 2 : a >= 0x43E00000u ? 1 : 0;
    if (w != want) {
      ++local[cls];
      if (cls == 0) {
        const uint32_t i = atomicAdd(&examples[0], 1u);
        if (i < 32u) {
          examples[1 + 3 * i] = p;
          examples[2 + 3 * i] = w;
          examples[3 + 3 * i] = want;
        }
      }
    }
    if (cls == 3 && ((w & 0x7Fu) != 0x7Fu || ((w >> 8) & 0x7Fu) != 0x7Fu)) ++local[4];
  }
  for (int c = 0; c < 5; ++c)
    if (local[c]) atomicAdd(&counts[c], (unsigned long long)local[c]);
}

}  // namespace

// counts: 5 device words, examples: 97 device words, both zeroed by the caller. Runs the
// 16 launches on `stream` and returns 0, 1 for bad arguments, 2 for a launch error.
extern "C" int fkv_probe_e4m3_check(unsigned long long* counts, uint32_t* examples, void* stream) {
  if (!counts || !examples) return 1;
  for (uint32_t top = 0; top < 16u; ++top) {
    hipLaunchKernelGGL(e4m3_check_kernel, dim3(1024), dim3(256), 0, static_cast<hipStream_t>(stream), counts,
                       examples, top);
    if (hipGetLastError() != hipSuccess) return 2;
  }
  return 0;
}
