// propose.h -- launch interface of the drafter-step kernels (internal to libsfx).
#pragma once

#include "delta_index.h"
#include "sfx_internal.h"

namespace sfx {

struct ProposeArgs {
  int32_t B, S, T;
  const int32_t* ntns;
  const int32_t* tok;
  const int32_t* samp;
  int32_t* draft;
  int32_t* nvalid;
  int32_t k, D, nb, M, mode, min_self, min_corpus;
  // per-call tables filled on the host: the draft cap of a candidate of match length l,
  // and the smallest vote count that keeps a chain of c0 sites going (stop rule)
  uint8_t cap_of_len[kMaxD + 1];
  uint8_t min_count[kMaxM + 1];
  const Ctl* ctl;  // nullptr when the context has no corpus
  IndexBuf idx[2];
  const int32_t* ring;
  int64_t ring_cap;    // ring slots: slot = position % ring_cap
  int32_t stream_ctx;  // read the context from HBM instead of staging it in LDS
  int32_t* pick;       // [B] out: the winner as num_valid << 16 | source << 8 | length, or -1
  // per-call index of the delta's tail-pair occurrences (delta_index.h), or nullptr, in which
  // case a request scans the whole delta
  const int32_t* pair_group;
  const PairSeg* pair_seg;   // [kPairSlices * (B + 1)] each slice's entries of each group
  const uint32_t* pair_list;
  // the context's sticky error word (kErrSyncTimeout is raised here)
  uint32_t* err;
  // per-wavefront phase timestamps (shader clock), written only by builds with
  // SFX_PHASE_TRACE=1; nullptr otherwise
  uint64_t* trace;
};

// Error-word bit raised when a workgroup's bounded internal wait runs out (SFX_ERR_SYNC_TIMEOUT
// of include/sfx.h).
constexpr uint32_t kErrSyncTimeout = 16;

// Timestamps per wavefront in a phase trace: [B][16 wavefronts][kTracePhases].
constexpr int kTracePhases = 16;

constexpr size_t kLdsBytes = 160 * 1024;  // LDS of one gfx950 workgroup
// Dynamic LDS of one request: the staged context (when staged), the hit lists and, with a
// corpus, the delta scan's occurrence records.
size_t propose_dynamic_lds(bool staged, int S, int T, bool corpus, int nb);
// Static LDS of the propose kernel (the per-request bookkeeping).
size_t propose_static_lds();
// Whether a call with row capacity S stages the context in LDS: it does unless asked not to or
// the staged layout does not fit one workgroup's LDS.
bool propose_staged(int S, int T, bool stream_ctx, bool corpus, int nb);
// Allows the largest dynamic LDS on every propose kernel instantiation.
hipError_t propose_prepare();
// general: launch the kernel with the general path (a delta, or no live snapshot).  Without it
// the kernel ignores the delta, which is right only when no document was ingested since the
// live snapshot was taken (the call then sees no delta).
hipError_t launch_propose(const ProposeArgs& a, bool general, hipStream_t st);
hipError_t launch_update_state(int B, int S, int T, int32_t* tok, const int32_t* ntns,
                               const int32_t* samp, int32_t* nout, hipStream_t st);

}  // namespace sfx
