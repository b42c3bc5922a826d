// corpus_file.h -- host-only reading, checking and writing of corpus files, the persistence of
// the cross-request memory (suffix-gpu page, TODO: persisting the global memory; layout and
// checksum as declared with sfx_save in sfx.h).  No HIP here: this code also builds with a
// plain host compiler under the address and undefined-behaviour sanitizers.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace sfx {

struct CorpusHeader {
  char magic[8];
  int64_t capacity, head, tail, doc_head, doc_tail, snap_start, snap_end;
  uint64_t checksum;
};
static_assert(sizeof(CorpusHeader) == 72, "corpus file header is 72 bytes");

// The whole contents of a corpus file: the live tokens [tail, head), the live documents'
// starts [doc_tail, doc_head), and the index (text and suffix array) over [snap_start, snap_end).
struct CorpusImage {
  CorpusHeader h{};
  std::vector<int32_t> live;
  std::vector<int64_t> starts;
  std::vector<int32_t> text;
  std::vector<int32_t> sa;
};

// FNV-1a over the payload's 32-bit words, in file order.
uint64_t corpus_checksum(const CorpusImage& img);

// Reads `path` for a context whose corpus ring holds `capacity` tokens, and checks everything a
// kernel would later index with: the counters, the exact size, the checksum, that documents
// start right after separators, that the index text agrees with the live tokens, and that the
// suffix array is a permutation.  Returns SFX_OK, SFX_EINVAL (capacity mismatch) or SFX_EIO,
// with the reason in *err.
int read_corpus_file(const char* path, int64_t capacity, CorpusImage* img, std::string* err);

// Writes img (magic and checksum filled in here) beside `path` and renames it over `path`, so a
// failed write leaves no partial file.  SFX_OK or SFX_EIO.
int write_corpus_file(const char* path, CorpusImage* img, std::string* err);

}  // namespace sfx
