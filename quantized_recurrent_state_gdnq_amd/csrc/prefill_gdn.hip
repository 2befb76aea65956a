#include <hip/hip_runtime.h>
#include "launch.h"
namespace gdnq {
hipError_t launch_prefill_gdn(const PrefillLaunch&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prefill_ssd(const PrefillLaunch&, hipStream_t) { return hipErrorNotSupported; }
size_t prefill_workspace_bytes(const PrefillLaunch&) { return 0; }
}
