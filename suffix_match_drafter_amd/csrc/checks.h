// checks.h -- optional input checks that raise bits of a sticky device error word (internal to
// libsfx).  The calls clamp or ignore these inputs in any case; the checks only report them.
#pragma once

#include "sfx_internal.h"

namespace sfx {

// Rows b < B: length outside [0, S]; a negative id in token_ids[b, 0:clamp(n_b)]; among the
// entries sampled[b, 0:c] that count (c = T, or clamp(counts[b], 0, T) when counts is non-null;
// counts[b] outside [0, T] is a length error), a non-negative id after a negative one.  samp may
// be null when T == 0.
hipError_t launch_check_propose(int B, int S, int T, const int32_t* ntns, const int32_t* tok,
                                const int32_t* samp, const int32_t* counts, uint32_t* err,
                                hipStream_t st);
// Harvest form: row index outside [0, num_rows); length outside [0, S]; a negative id in a
// document.  Packed form (doc_offsets non-null): a decreasing offset; a negative id.
hipError_t launch_check_ingest(int R, const int32_t* rows, const int32_t* lengths, int num_rows,
                               int S, const int64_t* doc_offsets, const int32_t* tokens,
                               uint32_t* err, hipStream_t st);
hipError_t launch_clear_word(uint32_t* err, hipStream_t st);

}  // namespace sfx
