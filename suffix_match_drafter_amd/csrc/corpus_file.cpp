// corpus_file.cpp -- see corpus_file.h.
#include "corpus_file.h"

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/sfx.h"

namespace sfx {

namespace {

constexpr char kCorpusMagic[8] = {'S', 'F', 'X', 'C', 'O', 'R', 'P', '1'};

int set_err(std::string* err, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (err) *err = buf;
  return code;
}

struct Fnv32Words {
  uint64_t h = 14695981039346656037ull;
  void add(const void* p, size_t bytes) {  // bytes is a multiple of 4
    const unsigned char* b = static_cast<const unsigned char*>(p);
    for (size_t i = 0; i + 4 <= bytes; i += 4) {
      uint32_t w;
      std::memcpy(&w, b + i, 4);
      h = (h ^ w) * 1099511628211ull;
    }
  }
};

// The contents against each other: everything a kernel would later index with (document
// starts, the suffix array) is range-checked here.
int check_contents(const CorpusImage& m, std::string* err) {
  const CorpusHeader& h = m.h;
  const int64_t nl = h.head - h.tail, nd = h.doc_head - h.doc_tail, ni = h.snap_end - h.snap_start;
  if (nl > 0 && m.live[nl - 1] != -1)
    return set_err(err, SFX_EIO, "last document unterminated");
  if ((nd == 0) != (nl == 0)) return set_err(err, SFX_EIO, "documents and tokens disagree");
  for (int64_t j = 0; j < nd; ++j) {
    // the first document starts at tail; every later one after the previous start, before
    // head, and right after a separator (range first, so the lookup stays inside `live`)
    const int64_t st = m.starts[j];
    const bool good = j == 0 ? st == h.tail
                             : st > m.starts[j - 1] && st < h.head && m.live[st - h.tail - 1] == -1;
    if (!good)
      return set_err(err, SFX_EIO, "document %lld starts at %lld, not after a separator",
                     (long long)j, (long long)st);
  }
  // the indexed text agrees with the live corpus where both exist
  const int64_t lo = h.snap_start > h.tail ? h.snap_start : h.tail;
  for (int64_t q = lo; q < h.snap_end; ++q)
    if (m.text[q - h.snap_start] != m.live[q - h.tail])
      return set_err(err, SFX_EIO, "index text differs from the corpus at %lld", (long long)q);
  std::vector<unsigned char> seen(ni, 0);
  for (int64_t r = 0; r < ni; ++r) {
    const int32_t v = m.sa[r];
    if (v < 0 || v >= ni || seen[v]) return set_err(err, SFX_EIO, "suffix array is not a permutation");
    seen[v] = 1;
  }
  return SFX_OK;
}

}  // namespace

uint64_t corpus_checksum(const CorpusImage& m) {
  Fnv32Words f;
  f.add(m.live.data(), 4 * m.live.size());
  f.add(m.starts.data(), 8 * m.starts.size());
  f.add(m.text.data(), 4 * m.text.size());
  f.add(m.sa.data(), 4 * m.sa.size());
  return f.h;
}

int read_corpus_file(const char* path, int64_t capacity, CorpusImage* m, std::string* err) {
  FILE* fp = std::fopen(path, "rb");
  if (!fp) return set_err(err, SFX_EIO, "cannot open %s", path);
  CorpusHeader& h = m->h;
  auto bad = [&](int code, const char* what) {
    std::fclose(fp);
    return set_err(err, code, "corpus file %s: %s", path, what);
  };
  if (std::fread(&h, sizeof h, 1, fp) != 1) return bad(SFX_EIO, "truncated header");
  if (std::memcmp(h.magic, kCorpusMagic, 8) != 0) return bad(SFX_EIO, "not a corpus file");
  if (h.capacity != capacity) {
    std::fclose(fp);
    return set_err(err, SFX_EINVAL, "corpus file %s has capacity %lld, the context %lld", path,
                   (long long)h.capacity, (long long)capacity);
  }
  // every difference below is between values in [0, 2^62], so none overflows
  const int64_t kMaxPos = int64_t(1) << 62;
  if (h.tail < 0 || h.head < h.tail || h.head > kMaxPos || h.head - h.tail > capacity ||
      h.doc_tail < 0 || h.doc_head < h.doc_tail || h.doc_head > kMaxPos ||
      h.doc_head - h.doc_tail > h.head - h.tail || h.snap_start < 0 ||
      h.snap_end < h.snap_start || h.snap_end > h.head || h.snap_end - h.snap_start > capacity)
    return bad(SFX_EIO, "inconsistent counters");
  const int64_t nl = h.head - h.tail, nd = h.doc_head - h.doc_tail, ni = h.snap_end - h.snap_start;
  m->live.assign(nl, 0);
  m->starts.assign(nd, 0);
  m->text.assign(ni, 0);
  m->sa.assign(ni, 0);
  bool ok = nl == 0 || std::fread(m->live.data(), 4, nl, fp) == (size_t)nl;
  ok = ok && (nd == 0 || std::fread(m->starts.data(), 8, nd, fp) == (size_t)nd);
  ok = ok && (ni == 0 || std::fread(m->text.data(), 4, ni, fp) == (size_t)ni);
  ok = ok && (ni == 0 || std::fread(m->sa.data(), 4, ni, fp) == (size_t)ni);
  if (!ok) return bad(SFX_EIO, "truncated payload");
  if (std::fgetc(fp) != EOF) return bad(SFX_EIO, "trailing bytes");
  std::fclose(fp);
  if (corpus_checksum(*m) != h.checksum)
    return set_err(err, SFX_EIO, "corpus file %s: checksum mismatch", path);
  std::string why;
  const int rc = check_contents(*m, &why);
  if (rc) return set_err(err, rc, "corpus file %s: %s", path, why.c_str());
  return SFX_OK;
}

int write_corpus_file(const char* path, CorpusImage* m, std::string* err) {
  const CorpusHeader& h = m->h;
  if (h.head - h.tail != (int64_t)m->live.size() ||
      h.doc_head - h.doc_tail != (int64_t)m->starts.size() ||
      h.snap_end - h.snap_start != (int64_t)m->text.size() || m->text.size() != m->sa.size())
    return set_err(err, SFX_EIO, "corpus image sizes disagree with its counters");
  std::memcpy(m->h.magic, kCorpusMagic, 8);
  m->h.checksum = corpus_checksum(*m);
  const std::string tmp = std::string(path) + ".partial";
  FILE* fp = std::fopen(tmp.c_str(), "wb");
  if (!fp) return set_err(err, SFX_EIO, "cannot open %s for writing", tmp.c_str());
  const size_t nl = m->live.size(), nd = m->starts.size(), ni = m->text.size();
  bool ok = std::fwrite(&m->h, sizeof m->h, 1, fp) == 1;
  ok = ok && (nl == 0 || std::fwrite(m->live.data(), 4, nl, fp) == nl);
  ok = ok && (nd == 0 || std::fwrite(m->starts.data(), 8, nd, fp) == nd);
  ok = ok && (ni == 0 || std::fwrite(m->text.data(), 4, ni, fp) == ni);
  ok = ok && (ni == 0 || std::fwrite(m->sa.data(), 4, ni, fp) == ni);
  ok = (std::fclose(fp) == 0) && ok;
  if (!ok || std::rename(tmp.c_str(), path) != 0) {
    std::remove(tmp.c_str());
    return set_err(err, SFX_EIO, "writing %s failed", path);
  }
  return SFX_OK;
}

}  // namespace sfx
