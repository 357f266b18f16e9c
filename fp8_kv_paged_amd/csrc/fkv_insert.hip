// Cache insertion: BF16 K/V -> (FP8 E4M3FN with a per-tensor scale | BF16) scattered into
// paged pools through a slot mapping.
//
// Operation: "Laguna S 2.1 INT4 -- calibrated FP8 KV on Intel B70", section Contract (E4M3
// KV with the checkpoint's calibrated scalar K/V scales, unit scales for the draft cache
// layers, no runtime scale calculation); the encode rule (true division, RNE, saturation
// at +-448) is the library's documented reading.
//
// One thread converts 8 consecutive dimensions (16 bytes of BF16) of one (token, KV head)
// for both K and V: a 16-byte load each, an 8-byte store for the K row and byte stores
// into the dimension-major 8-key groups of the V slab.
#include "fkv_device.h"
#include "fkv_internal.h"

namespace fkv {

template <bool kFp8>
__global__ __launch_bounds__(256) void cache_insert_kernel(InsertArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.num_tokens * a.num_kv_heads * 16;
  if (tid >= total) return;
  const int c = (int)(tid & 15);              // 8-dimension chunk
  const int64_t th = tid >> 4;                // token * Hkv + head
  const int h = (int)(th % a.num_kv_heads);
  const int64_t t = th / a.num_kv_heads;
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot / a.block_size;
  const int o = (int)(slot - blk * a.block_size);
  const int64_t slab = (blk * a.num_kv_heads + h) * (int64_t)a.block_size * kHeadDim;
  const int64_t k_off = slab + (int64_t)o * kHeadDim + c * 8;
  const int64_t v_off = slab + (o >> 3) * (8 * kHeadDim) + (c * 8) * 8 + (o & 7);

  const u32x4_t kin = *reinterpret_cast<const u32x4_t*>(a.k + th * kHeadDim + c * 8);
  const u32x4_t vin = *reinterpret_cast<const u32x4_t*>(a.v + th * kHeadDim + c * 8);

  if constexpr (kFp8) {
    uint32_t kc[2], vc[2];
    e4m3_encode8(kin, *a.k_scale, kc[0], kc[1]);
    e4m3_encode8(vin, *a.v_scale, vc[0], vc[1]);
    uint8_t* vp = static_cast<uint8_t*>(a.v_pool) + v_off;
#pragma unroll
    for (int j = 0; j < 8; ++j) vp[j * 8] = (uint8_t)(vc[j >> 2] >> (8 * (j & 3)));
    *reinterpret_cast<u32x2_t*>(static_cast<uint8_t*>(a.k_pool) + k_off) = u32x2_t{kc[0], kc[1]};
  } else {
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.k_pool) + k_off) = kin;
    uint16_t* vp = static_cast<uint16_t*>(a.v_pool) + v_off;
#pragma unroll
    for (int j = 0; j < 8; ++j) vp[j * 8] = (uint16_t)(vin[j >> 1] >> (16 * (j & 1)));
  }
}

hipError_t launch_insert(const InsertArgs& a, bool fp8, hipStream_t stream) {
  const int64_t total = (int64_t)a.num_tokens * a.num_kv_heads * 16;
  const int64_t blocks = (total + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (fp8)
    hipLaunchKernelGGL(cache_insert_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(cache_insert_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fkv
