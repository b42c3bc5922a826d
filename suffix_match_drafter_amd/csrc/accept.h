// accept.h -- launch interface of the acceptance-estimate kernels (internal to libsfx).
#pragma once

#include "sfx_internal.h"

namespace sfx {

// Counts table: [source 2][match length kMaxD + 1][draft slot kMaxK][proposed, accepted], uint64.
constexpr int kAcceptLens = kMaxD + 1;
constexpr size_t kAcceptEntries = (size_t)2 * kAcceptLens * kMaxK * 2;

hipError_t launch_accept_feedback(int B, int32_t* pick, const int32_t* num_accepted,
                                  unsigned long long* table, hipStream_t st);
hipError_t launch_accept_estimate(int B, int k, const int32_t* pick,
                                  const unsigned long long* table, int32_t* est_ppm,
                                  hipStream_t st);
hipError_t launch_accept_reset(unsigned long long* table, int32_t* pick, int rows,
                               hipStream_t st);

}  // namespace sfx
