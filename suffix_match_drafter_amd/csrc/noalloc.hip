// noalloc.hip -- the workspace of the allocation-free suffix-array build: one file-scope device
// array, sized for kNoAllocMaxTokens tokens.
//
// In host code the array's name is a host-side stand-in, not a device address: it is never
// passed to a kernel or a copy.  The device address comes from hipGetSymbolAddress, looked up
// once per device with that device current, and every use goes through it.
#include "noalloc.h"

#include <mutex>

#include "sa_build.h"

namespace sfx {

namespace {

constexpr size_t kNoAllocBytes = sa_ws_bytes(kNoAllocMaxTokens);
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_workspace(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  *bytes = kNoAllocBytes;
  return hipSuccess;
}

}  // namespace sfx
