// corpus.h -- launch interface of the corpus kernels (internal to libsfx).
#pragma once

#include "sfx_internal.h"

namespace sfx {

struct IngestArgs {
  int32_t R;                  // documents in this call
  const int32_t* row_indices; // harvest form: rows of `tokens` [num_rows, S]
  const int32_t* lengths;
  int32_t num_rows, S;
  const int64_t* doc_offsets; // packed form (non-null selects it): [R+1]
  const int32_t* seg_start;   // segment form (non-null selects it): document r is
  const int32_t* seg_len;     //   row[seg_start[r] : seg_start[r] + seg_len[r]]; -1 = no document
  const int32_t* tokens;
  Ctl* ctl;
  int32_t* ring;
  int64_t cap;                // ring capacity in tokens
  int64_t* doc_start;         // doc ring: logical start of each live document
  int64_t dcap;               // doc ring size (cap + 1)
  int64_t* doc_off;           // scratch [R+1]: offsets of the new documents
  int32_t* doc_idx;           // scratch [R+1]: documents (not skipped) before each entry
};

// In-flight ingest: per-row cursors, claims that keep the first entry of a repeated row, and the
// segments the next launch_ingest appends.
struct InflightArgs {
  int32_t R;
  const int32_t* row_indices;
  const int32_t* lengths;
  const int32_t* final_flags;
  int32_t num_rows, S, min_chunk, max_rows;
  int32_t* cursor;            // [max_rows] tokens of each row already ingested
  int32_t* claim;             // [max_rows] INT32_MAX between calls
  int32_t* seg_start;         // out [R]
  int32_t* seg_len;           // out [R]
};

hipError_t launch_ingest(const IngestArgs& a, int max_doc_len_hint, hipStream_t st);
hipError_t launch_inflight_prepare(const InflightArgs& a, hipStream_t st);
hipError_t launch_claims_init(int32_t* claim, int n, hipStream_t st);
hipError_t launch_snapshot(Ctl* ctl, const int32_t* ring, int64_t cap, int32_t* text, int buf,
                           int64_t* range_out, hipStream_t st);
hipError_t launch_swap(Ctl* ctl, int buf, uint32_t mask, hipStream_t st);
hipError_t launch_ctl_init(Ctl* ctl, hipStream_t st);
hipError_t launch_live_range(const Ctl* ctl, int64_t* out, hipStream_t st);
hipError_t launch_ring_copy(const Ctl* ctl, const int32_t* ring, int64_t cap, int32_t* out,
                            int64_t out_cap, hipStream_t st);

}  // namespace sfx
