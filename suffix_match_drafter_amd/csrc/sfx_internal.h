// sfx_internal.h -- device-side data layout shared by the libsfx translation units.
//
// Corpus state lives on the device so that ingest, rebuild and propose never need the host to
// read a device value (suffix-gpu page, Highlights: no per-step host synchronisation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfx {

constexpr int kMaxK = 32;    // draft width limit (register windows in the vote)
// Positions allocated past a snapshot text's capacity: the propose kernel reads a corpus window
// of up to kMaxK tokens without clamping it to the text's end (the text ends with a separator,
// which ends every window, so what lies past it is never used).
constexpr int kTextSlack = 64;
constexpr int kMaxD = 64;    // max_tree_depth limit (tail staged in LDS, lengths fit a byte)
constexpr int kMaxNB = 8;    // num_backoff limit
constexpr int kMaxM = 128;   // max_occurrences limit (two sites per lane of one wavefront)
constexpr int kMaxT = 16;    // sampled width limit
constexpr int kMaxSeq = 32768;  // row capacity limit: a whole context is staged in LDS
constexpr int kNG = 3;       // probe tables for 2-, 3- and 4-grams
constexpr int kEmptyTok = -1;

// One open-addressing slot of an n-gram table: the n tokens (unused ones -1), the offset of
// the n-gram's group in the position list, the group size, and the suffix-array index of the
// group's first entry.  A group, the occurrences of the n-gram followed by a real token, is one
// contiguous range of the suffix array (a separator sorts below every token), so it is
// [sa_lo, sa_lo + cnt) there.  owner == 0 marks an empty slot.
struct alignas(32) NgramSlot {
  int32_t key[4];
  int32_t off;
  int32_t cnt;
  int32_t owner;
  int32_t sa_lo;
};

// One of the two corpus index buffers.  text holds the snapshot (live documents, each followed
// by -1); sa its suffix array; pl[g] the starts of continuing (g+2)-gram occurrences grouped by
// n-gram and ordered by position inside a group; ht[g] maps an n-gram to its group.
struct IndexBuf {
  int32_t* text;
  int32_t* sa;
  int32_t* pl[kNG];
  NgramSlot* ht[kNG];
};

// Device control block.  Logical corpus positions grow monotonically; ring slot = pos % cap.
struct Ctl {
  int64_t head;          // logical end of everything appended
  int64_t tail;          // logical start of the oldest live document
  int64_t doc_head;      // documents ever appended
  int64_t doc_tail;      // first live document
  int64_t snap_start[2]; // logical range indexed by each buffer
  int64_t snap_end[2];
  int64_t ingest_base;   // head before the most recent append (read by the scatter kernel)
  int64_t pending_start; // snapshot being built: logical range
  int64_t pending_end;
  uint32_t ht_mask[2];   // probe-table size - 1 of each buffer
  int32_t active;        // live index buffer (0/1) or -1 when no index is live
  int32_t pending;       // buffer a rebuild is filling, or -1
};

}  // namespace sfx

namespace sfx {

// Hash of an n-gram (n <= 4) for the probe tables; the same function is used when the tables
// are built and when they are probed.
__host__ __device__ inline uint32_t ngram_hash(const int32_t* key, int n) {
  uint64_t h = 0x9E3779B97F4A7C15ull ^ (uint64_t)n;
  for (int i = 0; i < n; ++i) {
    h ^= (uint32_t)key[i];
    h *= 0xff51afd7ed558ccdull;
    h ^= h >> 33;
  }
  h *= 0xc4ceb9fe1a85ec53ull;
  h ^= h >> 29;
  return (uint32_t)h;
}

// Fixed-trip form for device code: key[0..3] with the unused entries ignored.
__host__ __device__ inline uint32_t ngram_hash4(const int32_t* key, int n) {
  uint64_t h = 0x9E3779B97F4A7C15ull ^ (uint64_t)n;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < n) {
      h ^= (uint32_t)key[i];
      h *= 0xff51afd7ed558ccdull;
      h ^= h >> 33;
    }
  }
  h *= 0xc4ceb9fe1a85ec53ull;
  h ^= h >> 29;
  return (uint32_t)h;
}

}  // namespace sfx
