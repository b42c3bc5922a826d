// call_forms.h -- launch interface of the preparation kernels of the other call forms of the
// drafter step (internal to libsfx).
#pragma once

#include "sfx_internal.h"

namespace sfx {

// Per-row prefix length and sampled id of the masked form: the row's last token becomes its
// sampled id (-1 for a masked-off or empty row).
hipError_t launch_masked_prep(int B, int S, const int32_t* ntns, const int32_t* tok,
                              const int32_t* mask, int32_t* n_out, int32_t* s_out,
                              hipStream_t st);

// The counted form: sampled ids cut at counts[b] (clamped to [0, T]) and -1 padded.
hipError_t launch_counts_prep(int B, int T, const int32_t* sampled, const int32_t* counts,
                              int32_t* s_out, hipStream_t st);

}  // namespace sfx
