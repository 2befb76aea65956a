#include <hip/hip_runtime.h>

#include "launch.h"

namespace gdnq {
size_t prefill_ssd_workspace_bytes(const PrefillLaunch&) { return 0; }
hipError_t launch_prefill_ssd(const PrefillLaunch&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace gdnq
