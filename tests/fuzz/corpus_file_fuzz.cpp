// Corrupted-file fuzz of the corpus file reader (suffix_match_drafter_amd/csrc/corpus_file.cpp),
// built with the address and undefined-behaviour sanitizers by tests/test_corpus_file_fuzz.py.
//
// A valid image is made from seeded synthetic documents (with evicted documents before the
// ring's tail and an index that starts before it), written, and read back.  Then every
// iteration writes a mutated file: random bytes flipped, the file cut or extended, header
// counters replaced by edge values, and payload entries changed with the checksum recomputed
// (so the reader's content checks run, not only its checksum).  The reader must either refuse
// the file with SFX_EIO or SFX_EINVAL, or accept a file whose contents satisfy every property
// that loading relies on, checked here independently.  Any other outcome, or any sanitizer
// report, fails the run.
//
// usage: corpus_file_fuzz <dir> <seed> <iterations>
#include <algorithm>
#include <cinttypes>
#include <cstdio>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "../../include/sfx.h"
#include "../../suffix_match_drafter_amd/csrc/corpus_file.h"

using sfx::CorpusHeader;
using sfx::CorpusImage;

namespace {

constexpr int64_t kCap = 4096;

CorpusImage make_image(std::mt19937_64& rng) {
  // documents of 1..40 tokens (ids up to 2^31 - 1) each ending with -1, logical positions
  // starting at an arbitrary offset; the oldest ones are evicted (before tail)
  std::vector<int32_t> all;
  std::vector<int64_t> starts_all;
  const int64_t base = (int64_t)(rng() % 100000);
  const int ndocs = 20 + (int)(rng() % 60);
  for (int d = 0; d < ndocs; ++d) {
    starts_all.push_back(base + (int64_t)all.size());
    const int len = 1 + (int)(rng() % 40);
    for (int i = 0; i < len; ++i) all.push_back((int32_t)(rng() % 2147483647u));
    all.push_back(-1);
  }
  const int evicted = (int)(rng() % 5);
  CorpusImage m;
  CorpusHeader& h = m.h;
  h.capacity = kCap;
  h.tail = starts_all[evicted];
  h.head = base + (int64_t)all.size();
  h.doc_tail = 1000 + evicted;
  h.doc_head = 1000 + ndocs;
  for (int64_t q = h.tail; q < h.head; ++q) m.live.push_back(all[q - base]);
  for (int d = evicted; d < ndocs; ++d) m.starts.push_back(starts_all[d]);
  // the index covers a range that may start among the evicted documents and end before head
  const int sd = (int)(rng() % (evicted + 1));
  h.snap_start = starts_all[sd];
  h.snap_end = h.head - (int64_t)(rng() % 8 == 0 ? 0 : (rng() % (h.head - h.tail)));
  if (h.snap_end < h.snap_start) h.snap_end = h.snap_start;
  for (int64_t q = h.snap_start; q < h.snap_end; ++q) m.text.push_back(all[q - base]);
  m.sa.resize(m.text.size());
  for (size_t i = 0; i < m.sa.size(); ++i) m.sa[i] = (int32_t)i;
  std::shuffle(m.sa.begin(), m.sa.end(), rng);
  return m;
}

// What loading relies on, checked without the reader's code.
bool sound(const CorpusImage& m, std::string* why) {
  const CorpusHeader& h = m.h;
  auto no = [&](const char* w) {
    *why = w;
    return false;
  };
  if (h.capacity != kCap) return no("capacity");
  if (!(h.tail >= 0 && h.tail <= h.head && h.head - h.tail <= kCap)) return no("token range");
  if (!(h.doc_tail >= 0 && h.doc_tail <= h.doc_head && h.doc_head - h.doc_tail <= h.head - h.tail))
    return no("document range");
  if (!(h.snap_start >= 0 && h.snap_start <= h.snap_end && h.snap_end <= h.head &&
        h.snap_end - h.snap_start <= kCap))
    return no("index range");
  const size_t nl = (size_t)(h.head - h.tail), nd = (size_t)(h.doc_head - h.doc_tail),
               ni = (size_t)(h.snap_end - h.snap_start);
  if (m.live.size() != nl || m.starts.size() != nd || m.text.size() != ni || m.sa.size() != ni)
    return no("section sizes");
  if (nl > 0 && m.live.back() != -1) return no("unterminated");
  if ((nd == 0) != (nl == 0)) return no("documents vs tokens");
  for (size_t j = 0; j < nd; ++j) {
    const int64_t s = m.starts[j];
    if (s < h.tail || s >= h.head) return no("start out of range");
    if (j == 0 && s != h.tail) return no("first start");
    if (j > 0 && (s <= m.starts[j - 1] || m.live[(size_t)(s - h.tail) - 1] != -1))
      return no("start not after a separator");
  }
  for (int64_t q = std::max(h.snap_start, h.tail); q < h.snap_end; ++q)
    if (m.text[(size_t)(q - h.snap_start)] != m.live[(size_t)(q - h.tail)]) return no("text");
  std::vector<int32_t> p(m.sa);
  std::sort(p.begin(), p.end());
  for (size_t i = 0; i < ni; ++i)
    if (p[i] != (int32_t)i) return no("suffix array");
  return true;
}

std::vector<unsigned char> file_bytes(const std::string& path) {
  std::vector<unsigned char> b;
  FILE* fp = std::fopen(path.c_str(), "rb");
  if (!fp) return b;
  int c;
  while ((c = std::fgetc(fp)) != EOF) b.push_back((unsigned char)c);
  std::fclose(fp);
  return b;
}

void put_bytes(const std::string& path, const std::vector<unsigned char>& b) {
  FILE* fp = std::fopen(path.c_str(), "wb");
  if (!b.empty()) std::fwrite(b.data(), 1, b.size(), fp);
  std::fclose(fp);
}

const int64_t kEdge[] = {0, 1, -1, 2, kCap - 1, kCap, kCap + 1, INT64_MAX, INT64_MIN,
                         INT64_MAX - 1, (int64_t)1 << 62, ((int64_t)1 << 62) + 1,
                         (int64_t)1 << 31, -((int64_t)1 << 31)};

}  // namespace

int main(int argc, char** argv) {
  if (argc != 4) {
    std::fprintf(stderr, "usage: %s <dir> <seed> <iterations>\n", argv[0]);
    return 2;
  }
  const std::string dir = argv[1];
  std::mt19937_64 rng(std::strtoull(argv[2], nullptr, 10));
  const long iters = std::strtol(argv[3], nullptr, 10);
  const std::string good = dir + "/good.sfxc", path = dir + "/mutant.sfxc";
  long accepted = 0, refused = 0, by_kind[6] = {0, 0, 0, 0, 0, 0};
  for (long it = 0; it < iters; ++it) {
    if (it % 200 == 0) {  // a fresh valid image now and then
      CorpusImage m = make_image(rng);
      std::string err;
      if (sfx::write_corpus_file(good.c_str(), &m, &err) != SFX_OK) {
        std::fprintf(stderr, "write failed: %s\n", err.c_str());
        return 1;
      }
      CorpusImage back;
      if (sfx::read_corpus_file(good.c_str(), kCap, &back, &err) != SFX_OK) {
        std::fprintf(stderr, "a valid file was refused: %s\n", err.c_str());
        return 1;
      }
      std::string why;
      if (!sound(back, &why) || back.live != m.live || back.starts != m.starts ||
          back.text != m.text || back.sa != m.sa) {
        std::fprintf(stderr, "a valid file read back wrong (%s)\n", why.c_str());
        return 1;
      }
    }
    std::vector<unsigned char> b = file_bytes(good);
    const int kind = (int)(rng() % 6);
    ++by_kind[kind];
    if (kind == 0) {  // flip bytes anywhere
      const int n = 1 + (int)(rng() % 4);
      for (int i = 0; i < n; ++i) b[rng() % b.size()] ^= (unsigned char)(1 + rng() % 255);
      put_bytes(path, b);
    } else if (kind == 1) {  // cut
      b.resize(rng() % b.size());
      put_bytes(path, b);
    } else if (kind == 2) {  // extend
      const int n = 1 + (int)(rng() % 16);
      for (int i = 0; i < n; ++i) b.push_back((unsigned char)rng());
      put_bytes(path, b);
    } else if (kind == 3) {  // one header counter replaced (the checksum covers the payload only)
      const int field = 1 + (int)(rng() % 7);
      int64_t v = rng() % 2 ? kEdge[rng() % (sizeof kEdge / sizeof kEdge[0])]
                            : (int64_t)(rng() % 20000) - 100;
      std::memcpy(b.data() + 8 * field, &v, 8);
      put_bytes(path, b);
    } else {  // payload entries changed, checksum recomputed
      CorpusImage m;
      std::string err;
      if (sfx::read_corpus_file(good.c_str(), kCap, &m, &err) != SFX_OK) return 1;
      const int what = (int)(rng() % 5);
      if (what == 0 && !m.starts.empty()) {
        // a start moved a little, or to an edge of the live range or onto a neighbour
        const size_t j = rng() % m.starts.size();
        const int64_t cand[] = {m.starts[j] + (int64_t)(rng() % 7) - 3, m.h.head, m.h.head - 1,
                                m.h.head + 1, m.h.tail - 1, m.h.tail,
                                j > 0 ? m.starts[j - 1] : -1,
                                j + 1 < m.starts.size() ? m.starts[j + 1] : m.h.head + 2,
                                INT64_MAX, INT64_MIN};
        m.starts[j] = cand[rng() % (sizeof cand / sizeof cand[0])];
      }
      else if (what == 1 && !m.live.empty())
        m.live[rng() % m.live.size()] = rng() % 3 == 0 ? -1 : (int32_t)(rng() % 100);
      else if (what == 2 && m.sa.size() > 1) {
        const int32_t ni = (int32_t)m.sa.size();
        const int32_t cand[] = {m.sa[rng() % m.sa.size()], ni, ni - 1, -1, INT32_MAX, INT32_MIN,
                                (int32_t)(rng() % (2 * m.sa.size())) - 3};
        m.sa[rng() % m.sa.size()] = cand[rng() % (sizeof cand / sizeof cand[0])];
      }
      else if (what == 3 && !m.text.empty())
        m.text[rng() % m.text.size()] ^= 1;
      else if (!m.live.empty()) {  // drop the last token and move head with it
        m.live.pop_back();
        --m.h.head;
        if (m.h.snap_end > m.h.head) {
          m.h.snap_end = m.h.head;
          if (m.h.snap_start > m.h.snap_end) m.h.snap_start = m.h.snap_end;
          m.text.resize((size_t)(m.h.snap_end - m.h.snap_start));
          m.sa.resize(m.text.size());
        }
      }
      if (kind == 5) {  // and sometimes a counter beside it
        int64_t* const fields[] = {&m.h.head, &m.h.tail, &m.h.doc_head, &m.h.doc_tail,
                                   &m.h.snap_start, &m.h.snap_end};
        *fields[rng() % 6] += (int64_t)(rng() % 5) - 2;
      }
      // written raw: the image may disagree with its own counters now
      std::vector<unsigned char> out(sizeof(CorpusHeader));
      m.h.checksum = sfx::corpus_checksum(m);
      std::memcpy(out.data(), &m.h, sizeof m.h);
      auto app = [&](const void* p, size_t n) {
        const unsigned char* c = static_cast<const unsigned char*>(p);
        out.insert(out.end(), c, c + n);
      };
      app(m.live.data(), 4 * m.live.size());
      app(m.starts.data(), 8 * m.starts.size());
      app(m.text.data(), 4 * m.text.size());
      app(m.sa.data(), 4 * m.sa.size());
      put_bytes(path, out);
    }
    CorpusImage got;
    std::string err;
    const int rc = sfx::read_corpus_file(path.c_str(), kCap, &got, &err);
    if (rc == SFX_OK) {
      std::string why;
      if (!sound(got, &why)) {
        std::fprintf(stderr, "iteration %ld (kind %d): accepted an unsound file: %s\n", it, kind,
                     why.c_str());
        return 1;
      }
      ++accepted;
    } else if (rc == SFX_EIO || rc == SFX_EINVAL) {
      ++refused;
    } else {
      std::fprintf(stderr, "iteration %ld: unexpected code %d (%s)\n", it, rc, err.c_str());
      return 1;
    }
  }
  std::printf("iterations %ld accepted %ld refused %ld kinds %ld %ld %ld %ld %ld %ld\n", iters,
              accepted, refused, by_kind[0], by_kind[1], by_kind[2], by_kind[3], by_kind[4],
              by_kind[5]);
  return 0;
}
