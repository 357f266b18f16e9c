// Attainable HBM read bandwidth probe for the benchmark (not part of libfkv.so): every byte of
// a buffer read once with 16-byte nontemporal vector loads, each work group streaming one
// contiguous chunk with eight loads per thread in flight, folded with XOR so the loads cannot
// be dropped, one word per work group written to a sink. (Measured on MI355X over 2 GiB:
// grid-stride order with four loads in flight 5.1-5.7 TB/s, contiguous chunks 6.0-6.3 TB/s,
// contiguous chunks with nontemporal loads 6.9-7.0 TB/s at 1,024-8,192 work groups.)
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int kInFlight = 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ src, uint64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const uint64_t b0 = (uint64_t)blockIdx.x * per;
  const uint64_t b1 = b0 + per < n16 ? b0 + per : n16;
  uint64_t i = b0 + threadIdx.x;
  u32x4_t acc{0u, 0u, 0u, 0u};
  for (; i + (kInFlight - 1) * 256 < b1; i += kInFlight * 256) {
    u32x4_t v[kInFlight];
#pragma unroll
    for (int f = 0; f < kInFlight; ++f) v[f] = __builtin_nontemporal_load(src + i + f * 256);
#pragma unroll
    for (int f = 0; f < kInFlight; ++f) acc ^= v[f];
  }
  for (; i < b1; i += 256) acc ^= __builtin_nontemporal_load(src + i);
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Reads `bytes` (a multiple of 16, 16-byte aligned) at src with `blocks` work groups of 256
// threads; sink receives `blocks` words. Returns 0, or 1 for bad arguments, 2 for a launch error.
extern "C" int fkv_probe_stream_read(const void* src, uint64_t bytes, uint32_t* sink, int blocks, void* stream) {
  if (!src || !sink || blocks < 1 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) != 0) return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
