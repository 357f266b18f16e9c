// The C-ABI host layer compiled on its own for CPU checks (no device code): the launchers it
// calls are replaced by stubs in launch_stubs.cpp.
#include "../../fp8_kv_paged_amd/csrc/fkv_api.hip"
