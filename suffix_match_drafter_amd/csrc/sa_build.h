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

size_t sa_workspace_bytes(int64_t n);
SaWork sa_carve(void* ws, int64_t n);

// Builds sa[0..n) of text[0..n) on `st`.  The host waits for `st` once per doubling round to
// read the number of distinct ranks.  *rounds_out (optional) receives the rounds run.
hipError_t sa_build(const int32_t* text, int64_t n, int32_t* sa, const SaWork& w, hipStream_t st,
                    int* rounds_out);

// Position lists and hash tables of the continuing 2-, 3- and 4-gram occurrences of text,
// derived from its suffix array.  ht_slots is a power of two above twice the group count.
hipError_t ngram_tables_build(const int32_t* text, const int32_t* sa, int64_t n, int32_t* pl[kNG],
                              NgramSlot* ht[kNG], uint32_t ht_slots, const SaWork& w,
                              hipStream_t st);

}  // namespace sfx
