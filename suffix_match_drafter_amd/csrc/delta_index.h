// delta_index.h -- per-call index of the delta's two-token occurrences (internal to libsfx).
//
// The delta (documents appended since the live snapshot) has no suffix array, so its
// occurrences of a request's tail are found by position (suffix-gpu page, How it works step 2
// and Highlights: the unindexed documents are scanned directly).  Scanning the whole delta in
// every request costs B * |delta| compares.  Before a step that may see a delta, three passes
// sort the delta's end positions by the two tokens that end there, for only those pairs that
// end some request's context:
//   1. every wavefront column of the delta hashes the batch's tail pairs into a table (a
//      pair's group is named by its first request) and counts, per group, the occurrences in
//      its slice of the delta;
//   2. one workgroup per group scans that group's counts over the columns and totals them;
//   3. every slice workgroup turns the totals into group starts, and the slices write their
//      occurrences' offsets (from the delta start), in position order.
// A request then extends only its own group's occurrences, which are exactly those the scan
// would find, in the same order.
#pragma once

#include "sfx_internal.h"

namespace sfx {

constexpr int kPairMaxBatch = 1024;     // batches above this scan the delta instead
constexpr int kPairCols = 2048;         // wavefront slices of the delta
constexpr int kPairColsPerBlock = 8;    // 512-thread workgroups of eight slices

// Hash-table slots for a batch of up to max_batch requests: a power of two, at least four
// times the batch up to 2048 slots (so at least twice any batch), which keeps the probe runs
// of the many positions whose pair is no request's short.
inline uint32_t pair_slots(int max_batch) {
  uint32_t s = 64;
  while (s < 4u * (uint32_t)max_batch && s < 2u * kPairMaxBatch) s <<= 1;
  return s;
}

struct PairIndexArgs {
  int32_t B, S, T, D;
  const int32_t* ntns;
  const int32_t* tok;
  const int32_t* samp;
  const Ctl* ctl;
  const int32_t* ring;
  int64_t ring_cap;
  uint32_t slots;            // LDS hash-table slots for the batch's tail pairs
  int32_t* group;            // [B] out: the request's group, or -1 when it takes no delta scan
  int32_t* off;              // [(B + 1) * kPairCols] counts, then their prefix within a group
  int32_t* tot;              // [B + 1] out: occurrences of each group
  int32_t* base;             // [B + 1] out: start of each group's entries in list
  uint32_t* list;            // [ring_cap] occurrence offsets from the delta start
  uint16_t* pos_group;       // [ring_cap] group of delta end position lo + 1 + i (count pass),
                             // 0xFFFF for none
};

hipError_t launch_pair_index(const PairIndexArgs& a, hipStream_t st);

}  // namespace sfx
