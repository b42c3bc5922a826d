// masked.h -- launch interface of the masked form's preparation kernel (internal to libsfx).
#pragma once

#include "sfx_internal.h"

namespace sfx {

// Per-row prefix length and sampled id of the masked form: the row's last token becomes its
// sampled id (-1 for a masked-off or empty row).
hipError_t launch_masked_prep(int B, int S, const int32_t* ntns, const int32_t* tok,
                              const int32_t* mask, int32_t* n_out, int32_t* s_out,
                              hipStream_t st);

}  // namespace sfx
