// noalloc.hip -- the fixed device scratch array behind gattn_forward_noalloc.
//
// The balanced partition of the gather path keeps its per-part softmax
// states and flags in a workspace.  Callers that cannot allocate (code under
// HIP graph capture, tight serving loops) get this file-scope array instead:
// one copy per GPU, alive until the process ends.  Its name is a host-side
// stand-in in host code; the device address of each GPU's copy comes from
// hipGetSymbolAddress, called once per device with that device current, and
// only that address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.hpp"

namespace gattn {

namespace {

__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace gattn
