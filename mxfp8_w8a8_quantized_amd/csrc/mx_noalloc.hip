// The library-owned scratch array behind mx_linear_noalloc: one copy per
// GPU, in the code object's zero-initialised data, held until the process
// ends. A host-side reference to `scratch` names a host stand-in, not the
// device memory, so the device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mx_internal.h"

namespace {

// Activation slab and plan partial sums of one
// mx_linear_noalloc call (the layout of mx_linear's workspace).
static __device__ __align__(256) uint8_t scratch[mx::kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device; null until looked up

}  // namespace

namespace mx {

hipError_t scratch_buffer(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace mx
