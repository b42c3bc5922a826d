// delta_index.h -- per-call index of the delta's two-token occurrences (internal to libsfx).
//
// The delta (documents appended since the live snapshot) has no suffix array, so its
// occurrences of a request's tail are found by position (suffix-gpu page, How it works step 2
// and Highlights: the unindexed documents are scanned directly).  Scanning the whole delta in
// every request costs B * |delta| compares.  Before a step that may see a delta, one pass sorts
// the delta's end positions by the two tokens that end there, for only those pairs that end
// some request's context.  The delta is cut into kPairSlices slices of whole 64-position runs,
// one workgroup each; every workgroup
//   1. hashes the batch's tail pairs into a table in LDS (a pair's group is named by its first
//      request, the same in every workgroup; workgroup 0 stores every request's group);
//   2. counts its slice's occurrences per group and wavefront;
//   3. turns the counts into offsets inside its slice's part of the list (groups in order, then
//      wavefronts in order), and publishes each group's offset and count in the slice;
//   4. writes its occurrences' offsets (from the delta start) there, in position order inside
//      each group.
// A request then extends only its own group's occurrences, slice by slice: exactly those the
// scan would find, in the same order.
#pragma once

#include "sfx_internal.h"

namespace sfx {

constexpr int kPairMaxBatch = 1024;  // batches above this scan the delta instead
constexpr int kPairSlices = 256;     // delta slices, one workgroup each
constexpr int kPairWaves = 8;        // wavefronts of a slice workgroup

// Hash-table slots for a batch of up to max_batch requests: a power of two, at least four
// times the batch up to 2048 slots (so at least twice any batch), which keeps the probe runs
// of the many positions whose pair is no request's short.
inline uint32_t pair_slots(int max_batch) {
  uint32_t s = 64;
  while (s < 4u * (uint32_t)max_batch && s < 2u * kPairMaxBatch) s <<= 1;
  return s;
}

// End positions per slice for a delta of nd end positions: whole 64-position runs.  Slice s
// covers end positions lo + 1 + s * seg ..., and its part of the list starts at s * seg.
__host__ __device__ inline long long pair_seg(long long nd) {
  return ((nd + kPairSlices - 1) / kPairSlices + 63) / 64 * 64;
}
// List entries for a ring of cap tokens: kPairSlices parts of pair_seg(nd) entries, nd < cap.
inline size_t pair_list_entries(int64_t cap) { return (size_t)cap + 64 * (size_t)kPairSlices; }

// A group's occurrences in one slice: offset inside the slice's part of the list, and count.
struct PairSeg {
  int32_t off;
  int32_t cnt;
};

struct PairIndexArgs {
  int32_t B, S, T, D;
  const int32_t* ntns;
  const int32_t* tok;
  const int32_t* samp;
  const Ctl* ctl;
  const int32_t* ring;
  int64_t ring_cap;
  uint32_t slots;  // LDS hash-table slots for the batch's tail pairs
  int32_t* group;  // [B] out: the request's group, or -1 when it takes no delta scan
  PairSeg* seg;    // [kPairSlices * (B + 1)] out: group g's occurrences in slice s at
                   // s * (B + 1) + g (each workgroup writes one contiguous block)
  uint32_t* list;  // [pair_list_entries(ring_cap)] occurrence offsets from the delta start
};

hipError_t launch_pair_index(const PairIndexArgs& a, hipStream_t st);

}  // namespace sfx
