// noalloc.h -- the device workspace of the allocation-free suffix-array build (internal to
// libsfx).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfx {

// Largest text the allocation-free build takes: 2^20 tokens (its workspace, about 40 MiB, is
// held on every device the library runs on until the process ends).
constexpr int64_t kNoAllocMaxTokens = int64_t(1) << 20;

// Device address and size of that workspace on the current device.  The first call on a
// device looks the address up (with that device current); later calls reuse it.
hipError_t noalloc_workspace(void** ptr, size_t* bytes);

}  // namespace sfx
