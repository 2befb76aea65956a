// Device scratch of the allocation-free entry point (gdnq_prefill_chunked_noalloc):
// a fixed array in device memory that replaces the caller's workspace, for
// callers that cannot allocate.  Every GPU the library runs on holds its own
// copy from module load until the process ends.
//
// In host code the name `scratch` is a host-side stand-in, never a device
// address: the address of each device's copy is looked up once per device
// with hipGetSymbolAddress (that device current) and only that pointer is
// handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gdnq.h"
#include "launch.h"

namespace gdnq {

constexpr size_t SCRATCH_BYTES = GDNQ_NOALLOC_SCRATCH_BYTES;  // per device

static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES];  // device address of `scratch` per device, looked up once
}  // namespace

size_t scratch_capacity() { return SCRATCH_BYTES; }

hipError_t scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace gdnq
