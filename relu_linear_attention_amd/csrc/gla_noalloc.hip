// Scratch memory of gla_forward_noalloc: a device array that the library
// reserves when its code object is loaded on a device, so that the entry
// point needs no allocation at call time.  Each device holds its own copy at
// its own address until the process ends.

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "gla_internal.h"

namespace gla {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::vector<void *> g_scratch_ptr;  // per device id; nullptr until looked up
}  // namespace

// Device address of the current device's copy of `scratch`.  The array's
// name is a host-side stand-in in host code, never a device address: the
// kernels get the address looked up here, once per device, with that device
// current.
hipError_t noalloc_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || ((uintptr_t)p & 255) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace gla
