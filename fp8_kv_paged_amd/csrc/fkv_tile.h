// Shared pieces of the split kernels: the 32-key tile geometry of the paged pools, the
// per-lane chunk offsets that the LDS DMA and the register reads agree on, the LDS read
// of one tile and the DMA that fills it.
#pragma once

#include "fkv_device.h"

namespace fkv {

constexpr float kLazyTau = 8.0f;  // log2 units a tile maximum may exceed the reference by
constexpr float kLog2e = 1.4426950408889634f;
// Reference maximum of a row that has seen no visible key: finite, so that a masked score
// (-inf) still gives probability 0 while a visible one overflows the range check below.
constexpr float kRefInit = -1.0e30f;
// A lane's eight probabilities of one row tile are accepted when they sum to at most 2^15:
// each then fits f16 (max 65504). Larger sums send the tile through the exact-maximum path.
constexpr float kAcceptSum = 32768.f;

template <bool kFp8>
struct TileGeom {
  static constexpr int kChunks = kFp8 ? 8 : 16;  // 1 KB pieces per 32-key tile: K half, then V half
  static constexpr int kBytes = kChunks * 1024;
  static constexpr int kKVec = kFp8 ? 2 : 4;     // u32x4 per lane per 16-key half of K
  static constexpr int kVVec = kFp8 ? 4 : 8;     // u32x4 per lane of V
};

// Byte offset, within a tile's K slab (j < kChunks/2) or V group base (j >= kChunks/2), of
// the 16 bytes lane (n, q) owns in chunk j.
template <bool kFp8>
__device__ __forceinline__ uint32_t tile_chunk_offset(int j, int n, int q) {
  constexpr int kHalf = TileGeom<kFp8>::kChunks / 2;
  constexpr int kEs = kFp8 ? 1 : 2;
  if (j < kHalf) {
    const int per_tt = kHalf / 2;
    const int tt = j / per_tt, piece = j % per_tt;
    const int key = 8 * (n >> 2) + 4 * tt + (n & 3);
    return (uint32_t)((key * kHeadDim + 32 * q) * kEs + 16 * piece);
  }
  return (uint32_t)((q * 8 * kHeadDim + 64 * n) * kEs + 16 * (j - kHalf));
}

template <bool kFp8>
struct TileRegs32 {
  u32x4_t k[2][TileGeom<kFp8>::kKVec];
  u32x4_t v[TileGeom<kFp8>::kVVec];
};

// ds_read of one tile slot: lane l reads bytes 16*l of every 1 KB chunk. Inline asm so
// that the compiler does not add a wait on every outstanding DMA before it; the caller
// has waited for the slot's own DMAs. The outputs are early-clobber: a later read of the
// sequence still needs the address after an earlier one has been issued into its output.
template <bool kFp8>
__device__ __forceinline__ void read_slot(uint32_t addr, TileRegs32<kFp8>& r) {
  if constexpr (kFp8) {
    asm volatile(
        "ds_read_b128 %0, %8 offset:0\n\t"
        "ds_read_b128 %1, %8 offset:1024\n\t"
        "ds_read_b128 %2, %8 offset:2048\n\t"
        "ds_read_b128 %3, %8 offset:3072\n\t"
        "ds_read_b128 %4, %8 offset:4096\n\t"
        "ds_read_b128 %5, %8 offset:5120\n\t"
        "ds_read_b128 %6, %8 offset:6144\n\t"
        "ds_read_b128 %7, %8 offset:7168\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r.k[0][0]), "=&v"(r.k[0][1]), "=&v"(r.k[1][0]), "=&v"(r.k[1][1]), "=&v"(r.v[0]), "=&v"(r.v[1]),
          "=&v"(r.v[2]), "=&v"(r.v[3])
        : "v"(addr)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %8 offset:0\n\t"
        "ds_read_b128 %1, %8 offset:1024\n\t"
        "ds_read_b128 %2, %8 offset:2048\n\t"
        "ds_read_b128 %3, %8 offset:3072\n\t"
        "ds_read_b128 %4, %8 offset:4096\n\t"
        "ds_read_b128 %5, %8 offset:5120\n\t"
        "ds_read_b128 %6, %8 offset:6144\n\t"
        "ds_read_b128 %7, %8 offset:7168\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r.k[0][0]), "=&v"(r.k[0][1]), "=&v"(r.k[0][2]), "=&v"(r.k[0][3]), "=&v"(r.k[1][0]),
          "=&v"(r.k[1][1]), "=&v"(r.k[1][2]), "=&v"(r.k[1][3])
        : "v"(addr)
        : "memory");
    asm volatile(
        "ds_read_b128 %0, %8 offset:8192\n\t"
        "ds_read_b128 %1, %8 offset:9216\n\t"
        "ds_read_b128 %2, %8 offset:10240\n\t"
        "ds_read_b128 %3, %8 offset:11264\n\t"
        "ds_read_b128 %4, %8 offset:12288\n\t"
        "ds_read_b128 %5, %8 offset:13312\n\t"
        "ds_read_b128 %6, %8 offset:14336\n\t"
        "ds_read_b128 %7, %8 offset:15360\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r.v[0]), "=&v"(r.v[1]), "=&v"(r.v[2]), "=&v"(r.v[3]), "=&v"(r.v[4]), "=&v"(r.v[5]), "=&v"(r.v[6]),
          "=&v"(r.v[7])
        : "v"(addr)
        : "memory");
  }
}

// Requests one 32-key tile (K half then V half) into an LDS slot with global_load_lds:
// chunk j of the tile lands at dst + 1024*j, lane l's 16 bytes at offset 16*l. kb / vb
// already include the lane's chunk-0 offsets within the K slab and the V group.
template <bool kFp8>
__device__ __forceinline__ void dma_tile(const unsigned char* kb, const unsigned char* vb, unsigned char* dst) {
  constexpr int kHalf = TileGeom<kFp8>::kChunks / 2;
  constexpr int kEs = kFp8 ? 1 : 2;
#pragma unroll
  for (int j = 0; j < kHalf; ++j) {
    const int per_tt = kHalf / 2, tt = j / per_tt, piece = j % per_tt;
    __builtin_amdgcn_global_load_lds(kb + tt * 4 * kHeadDim * kEs + 16 * piece, dst + j * 1024, 16, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < kHalf; ++j) __builtin_amdgcn_global_load_lds(vb + 16 * j, dst + (kHalf + j) * 1024, 16, 0, 0);
}

}  // namespace fkv
