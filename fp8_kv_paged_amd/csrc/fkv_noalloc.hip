// fkv_decode_attn_noalloc: fkv_decode_attn with its split-KV scratch (partials and merge
// counters) in a static device array of this library instead of a caller workspace, for callers
// that cannot allocate device memory (code under HIP graph capture, tight serving loops). No
// allocation of any kind happens on this path.
#include <mutex>

#include "../../include/fkv.h"
#include "fkv_internal.h"

namespace {

constexpr uint64_t kScratchBytes = FKV_NOALLOC_SCRATCH_BYTES;
constexpr uint64_t kCtlBytes = (uint64_t)FKV_NOALLOC_MAX_PAIRS * 256;  // merge counters, at the start
constexpr int kMaxDevices = 64;
static_assert(kCtlBytes % 256 == 0 && kCtlBytes < kScratchBytes, "counters, then partials");

// One copy per GPU, resident until the process ends. Static storage: zero when the code
// object is loaded. The counter area must be zero before every call; every call leaves it so.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_setup;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device; null until set up

// Device address of this device's scratch. Set up once per device, with the device current:
// the symbol's address (the array's name is only a host-side stand-in), then the counter area
// cleared on the caller's stream unless that stream is being captured into a graph (then the
// zero of static storage stands: nothing has used the area yet).
void* acquire(void* stream, int* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = FKV_EHIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_setup);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *status = FKV_EHIP;
      return nullptr;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cs) != hipSuccess) {
      *status = FKV_EHIP;
      return nullptr;
    }
    if (cs == hipStreamCaptureStatusNone && hipMemsetAsync(p, 0, kCtlBytes, static_cast<hipStream_t>(stream)) != hipSuccess) {
      *status = FKV_EHIP;
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  *status = FKV_OK;
  return g_scratch[dev];
}

}  // namespace

extern "C" int fkv_decode_attn_noalloc(const fkv_cache* cache, const fkv_decode_desc* desc, const uint16_t* q,
                                       const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                                       const float* v_scale, void* out, void* stream) {
  const fkv::FixedScratch fs{acquire, kScratchBytes, kCtlBytes};
  return fkv::decode_attn_fixed_scratch(cache, desc, q, block_table, seq_lens, k_scale, v_scale, out, fs, stream);
}
