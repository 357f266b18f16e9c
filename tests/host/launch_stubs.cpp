// Stand-ins for the kernel launchers: they record the call and report success, so that every
// host-side path of the C ABI (planning, validation, launch counters) runs on a machine
// without a GPU. Test infrastructure only.
#include "../../fp8_kv_paged_amd/csrc/fkv_internal.h"

namespace fkv {

unsigned long long g_stub_decode_calls = 0;

hipError_t launch_insert(const InsertArgs&, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_norm_rope_insert(const NormRopeArgs&, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_decode(const DecodeArgs& a, const SplitShapeInfo&, bool, hipStream_t, bool* launched_combine) {
  ++g_stub_decode_calls;
  *launched_combine = a.max_splits > 1 && !a.fused_combine;
  return hipSuccess;
}

}  // namespace fkv
