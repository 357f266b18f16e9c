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
// into the dimension-major 8-key groups of the V slab. The same stores serve the Q/K
// RMSNorm + RoPE kernel below, which inserts the normalised, rotated keys.
#include "fkv_device.h"
#include "fkv_internal.h"

namespace fkv {

// Stores 8 dimensions (chunk c) of one (token, KV head) of K and V at offset o of the
// (block, head) slab starting at element slab: 8 bytes (FP8) or 16 (BF16) of the K row, and
// one element into each of 8 rows of the V slab's dimension-major 8-key group.
template <bool kFp8>
__device__ __forceinline__ void put_kv_chunk(void* k_pool, void* v_pool, int64_t slab, int o, int c, const u32x4_t& kin,
                                             const u32x4_t& vin, const float* k_scale, const float* v_scale) {
  const int64_t k_off = slab + (int64_t)o * kHeadDim + c * 8;
  const int64_t v_off = slab + (o >> 3) * (8 * kHeadDim) + (c * 8) * 8 + (o & 7);
  if constexpr (kFp8) {
    uint32_t kc[2], vc[2];
    e4m3_encode8(kin, *k_scale, kc[0], kc[1]);
    e4m3_encode8(vin, *v_scale, vc[0], vc[1]);
    uint8_t* vp = static_cast<uint8_t*>(v_pool) + v_off;
#pragma unroll
    for (int j = 0; j < 8; ++j) vp[j * 8] = (uint8_t)(vc[j >> 2] >> (8 * (j & 3)));
    *reinterpret_cast<u32x2_t*>(static_cast<uint8_t*>(k_pool) + k_off) = u32x2_t{kc[0], kc[1]};
  } else {
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(k_pool) + k_off) = kin;
    uint16_t* vp = static_cast<uint16_t*>(v_pool) + v_off;
#pragma unroll
    for (int j = 0; j < 8; ++j) vp[j * 8] = (uint16_t)(vin[j >> 1] >> (16 * (j & 1)));
  }
}

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
  const u32x4_t kin = *reinterpret_cast<const u32x4_t*>(a.k + th * kHeadDim + c * 8);
  const u32x4_t vin = *reinterpret_cast<const u32x4_t*>(a.v + th * kHeadDim + c * 8);
  put_kv_chunk<kFp8>(a.k_pool, a.v_pool, slab, o, c, kin, vin, a.k_scale, a.v_scale);
}

// ---- Q/K RMSNorm + RoPE + insert ("Laguna S 2.1 INT4 -- calibrated FP8 KV on Intel B70",
// section "Initial optimization order": the scaled E4M3 insert at the Q/K norm + RoPE step;
// "Laguna S 2.1 B70 campaign transfer ledger", section "Result progression and what actually
// worked": an exact fused Q/K RMSNorm/RoPE stack). Sixteen lanes take one 128-dim head vector
// of Q or K, 8 consecutive dims each (norm_rope16). A K row then inserts its result and the
// token's V row of that head.
template <bool kFp8>
__global__ __launch_bounds__(256) void norm_rope_insert_kernel(NormRopeArgs a) {
  const int rows = a.num_q_heads + a.num_kv_heads;  // normalised head vectors per token
  const int64_t job = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int c = (int)(threadIdx.x & 15);
  const bool live = job < (int64_t)a.num_tokens * rows;
  const int64_t jj = live ? job : 0;  // lanes past the end compute row 0 for the shuffles, store nothing
  const int64_t t = jj / rows;
  const int r = (int)(jj - t * rows);
  const bool is_q = r < a.num_q_heads;
  const int h = is_q ? r : r - a.num_q_heads;
  const uint16_t* src = is_q ? a.q + (t * a.num_q_heads + h) * kHeadDim : a.k + (t * a.num_kv_heads + h) * kHeadDim;
  const u32x4_t xin = *reinterpret_cast<const u32x4_t*>(src + c * 8);
  const u32x4_t win = *reinterpret_cast<const u32x4_t*>((is_q ? a.q_w : a.k_w) + c * 8);
  const int pos = a.positions[t];
  const bool valid = pos >= 0 && pos < a.rope_rows;
  const u32x4_t z = norm_rope16(xin, win, c, a.eps, a.cos_sin + (int64_t)(valid ? pos : 0) * kHeadDim);
  if (!live) return;
  const u32x4_t zb = valid ? z : u32x4_t{0u, 0u, 0u, 0u};
  if (is_q) {
    *reinterpret_cast<u32x4_t*>(a.q_out + (t * a.num_q_heads + h) * kHeadDim + c * 8) = zb;
    return;
  }
  const int64_t slot = a.slots[t];
  if (!valid || slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot / a.block_size;
  const int o = (int)(slot - blk * a.block_size);
  const int64_t slab = (blk * a.num_kv_heads + h) * (int64_t)a.block_size * kHeadDim;
  const u32x4_t vin = *reinterpret_cast<const u32x4_t*>(a.v + (t * a.num_kv_heads + h) * kHeadDim + c * 8);
  put_kv_chunk<kFp8>(a.k_pool, a.v_pool, slab, o, c, zb, vin, a.k_scale, a.v_scale);
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

hipError_t launch_norm_rope_insert(const NormRopeArgs& a, bool fp8, hipStream_t stream) {
  const int64_t total = (int64_t)a.num_tokens * (a.num_q_heads + a.num_kv_heads) * 16;
  const int64_t blocks = (total + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (fp8)
    hipLaunchKernelGGL(norm_rope_insert_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(norm_rope_insert_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fkv
