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

// Batch-bucket padding: empties rows [from, to) of a batch (length 0, sampled ids -1) with a
// grid sized for `to` rows, so that in a graph only the node's arguments change: set_pad_rows
// sets them in an instantiated graph's node.
hipError_t launch_pad_rows(int32_t* ntns, int32_t* samp, int T, int from, int to,
                          hipStream_t st);
hipError_t set_pad_rows(hipGraphExec_t exec, hipGraphNode_t node, int32_t* ntns, int32_t* samp,
                        int T, int from, int to);

}  // namespace sfx
