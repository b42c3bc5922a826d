// sa_build.h -- suffix-array construction and n-gram probe tables (internal to libsfx).
#pragma once

#include "sfx_internal.h"

namespace sfx {

// Device workspace of one construction, carved out of a caller buffer.
struct SaWork {
  uint64_t* k0;
  uint64_t* k1;
  int32_t* v0;
  int32_t* v1;
  int32_t* rank;
  int32_t* head;
  int32_t* aux;
  int32_t* act;  // positions (in suffix-array order) of the suffixes still sharing a rank
  int32_t* hist;
  int32_t* tiles;
  uint32_t* counters;
  int64_t n;
};

// Workspace bytes of a construction of n tokens (a compile-time expression as well).
constexpr int kSaRadixTile = 4096;  // keys per radix-sort tile
constexpr int kSaScanTile = 4096;   // elements per scan tile
constexpr int64_t sa_cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
constexpr size_t sa_ws_bytes(int64_t n) {
  const int64_t nn = n < 1 ? 1 : n;
  const int64_t nt = sa_cdiv(nn, kSaRadixTile);
  size_t b = 0;
  b += 2 * sizeof(uint64_t) * (size_t)nn;                              // k0, k1
  b += 2 * sizeof(int32_t) * (size_t)nn;                               // v0, v1
  b += 4 * sizeof(int32_t) * (size_t)nn;                               // rank, head, aux, act
  b += sizeof(int32_t) * (size_t)(256 * nt + 64);                      // hist
  b += sizeof(int32_t) * (size_t)(sa_cdiv(256 * nt + nn, kSaScanTile) + 64);  // scan tiles
  b += 256;                                                            // counters
  b += 16 * 256;                                                       // alignment slack
  return b;
}
size_t sa_workspace_bytes(int64_t n);
SaWork sa_carve(void* ws, int64_t n);

// Host side of the round-count reads of sa_build: pinned counts and one event per round.
constexpr int kPollRounds = 32;  // doubling rounds of n <= 2^30 tokens: at most 30
constexpr int kPollLag = 2;      // rounds between a count's enqueue and its read
struct SaPoll {
  int32_t* counts;  // pinned host memory, kPollRounds entries
  hipEvent_t ev[kPollRounds];
  int enqueued = 0;  // rounds of the last build whose count was enqueued (set by sa_build)
};

// Builds sa[0..n) of text[0..n) on `st`, with no host wait per round: every kernel reads the
// round's sort size on the device.  With poll == nullptr all ceil(log2 n) doubling rounds are
// enqueued (the ones after convergence do nothing) and the call returns without waiting; with
// a poll the host stops enqueueing kPollLag rounds after the first empty one.  *rounds_out
// (optional, needs a poll) receives the rounds that sorted something plus the first sort; it
// makes the call wait for the last enqueued round.
hipError_t sa_build(const int32_t* text, int64_t n, int32_t* sa, const SaWork& w, hipStream_t st,
                    const SaPoll* poll, int* rounds_out);

// Position lists and hash tables of the continuing 2-, 3- and 4-gram occurrences of text,
// derived from its suffix array.  ht_slots is a power of two above twice the group count.
hipError_t ngram_tables_build(const int32_t* text, const int32_t* sa, int64_t n, int32_t* pl[kNG],
                              NgramSlot* ht[kNG], uint32_t ht_slots, const SaWork& w,
                              hipStream_t st);

}  // namespace sfx
