// sfx_api.cpp -- host side of libsfx: the C-ABI declared in include/sfx.h.
//
// Host code only validates, allocates at creation, and enqueues kernels.  The propose and ingest
// paths never read device memory from the host.  The index rebuild is enqueued by the host,
// which follows the device's count of suffixes left to sort two doubling rounds late through
// pinned memory (no wait per round), either inline on the caller's stream (sfx_rebuild) or on
// a library-owned worker thread and side stream (sfx_rebuild_async + sfx_poll).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "../../include/sfx.h"
#include "accept.h"
#include "corpus.h"
#include "corpus_file.h"
#include "call_forms.h"
#include "checks.h"
#include "delta_index.h"
#include "noalloc.h"
#include "propose.h"
#include "sa_build.h"

using namespace sfx;

namespace {

thread_local std::string g_err = "no error";

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SFX_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_OR_RETURN(expr, what)                  \
  do {                                             \
    hipError_t e_ = (expr);                        \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

constexpr int kIngestChunk = 65536;  // documents per ingest launch

uint32_t next_pow2_u32(uint64_t v) {
  uint64_t p = 1;
  while (p < v) p <<= 1;
  return p > 0x80000000ull ? 0x80000000u : (uint32_t)p;
}

}  // namespace

struct sfx_ctx {
  sfx_config cfg{};
  int device = 0;
  int32_t* pick = nullptr;                 // [max_batch] winner of each row's last propose
  int32_t* masked = nullptr;               // [2 * max_batch] prefix lengths, sampled ids
  int32_t* counted = nullptr;              // [max_batch * max_sampled] cut sampled ids
  unsigned long long* accept = nullptr;    // acceptance counts (accept.h layout)
  uint32_t* err = nullptr;                 // sticky SFX_ERR_* word (SFX_FLAG_CHECK_INPUTS)
  // corpus (absent when corpus_capacity == 0)
  Ctl* ctl = nullptr;
  int32_t* ring = nullptr;
  int64_t cap = 0;
  int64_t* doc_start = nullptr;
  int64_t dcap = 0;
  int64_t* doc_off = nullptr;
  int32_t* doc_idx = nullptr;
  int32_t* inflight = nullptr;   // [2 * max_batch] cursor and claim of every batch row, then
                                 // [2 * kIngestChunk] segment starts and lengths
  int64_t* range_dev = nullptr;  // [2] snapshot range read back by the rebuild driver
  IndexBuf idx[2]{};
  uint32_t ht_slots = 0;
  void* sa_ws = nullptr;
  size_t sa_ws_bytes = 0;
  SaWork saw{};
  SaPoll poll{};  // pinned round counts and events of the rebuild's suffix-array rounds
  int64_t last_index_tokens = 0;  // snapshot tokens of the last index build
  hipStream_t side = nullptr;
  hipEvent_t ev_snap = nullptr;
  hipEvent_t ev_done = nullptr;
  int active_host = -1;  // host mirror of the live buffer
  // per-call pair index of the delta (delta_index.h); absent above kPairMaxBatch rows
  int32_t* pair_group = nullptr;
  PairSeg* pair_seg = nullptr;
  uint32_t* pair_list = nullptr;
  uint32_t pair_slots = 0;
  // Ingest calls so far, and how many of them the live index covers (that of the snapshot
  // being built, for an asynchronous rebuild).  While they differ the corpus may hold a delta,
  // and the step builds the pair index first.
  uint64_t ingest_epoch = 0;
  uint64_t live_epoch = 0;
  uint64_t snap_epoch = 0;
  // asynchronous rebuild
  std::thread worker;
  std::atomic<int> async_state{0};  // 0 idle, 1 running, 2 finished
  std::atomic<int> fail_next{0};    // test hook: the next rebuild fails before its swap
  int async_buf = -1;
  uint32_t async_mask = 0;
  int async_err = SFX_OK;
  std::string async_msg;
};

namespace {

int validate(const sfx_config* c) {
  if (!c) return fail(SFX_EINVAL, "config is NULL");
  if (c->k < 1 || c->k > kMaxK) return fail(SFX_EINVAL, "k=%d outside [1,%d]", c->k, kMaxK);
  if (c->max_tree_depth < 1 || c->max_tree_depth > kMaxD)
    return fail(SFX_EINVAL, "max_tree_depth=%d outside [1,%d]", c->max_tree_depth, kMaxD);
  if (c->num_backoff < 1 || c->num_backoff > kMaxNB)
    return fail(SFX_EINVAL, "num_backoff=%d outside [1,%d]", c->num_backoff, kMaxNB);
  if (c->max_occurrences < 1 || c->max_occurrences > kMaxM)
    return fail(SFX_EINVAL, "max_occurrences=%d outside [1,%d]", c->max_occurrences, kMaxM);
  if (c->mode != SFX_MODE_LONGEST_FILL && c->mode != SFX_MODE_SCORED)
    return fail(SFX_EINVAL, "mode=%d unknown", c->mode);
  if (c->mode == SFX_MODE_LONGEST_FILL && c->num_backoff != 1)
    return fail(SFX_EINVAL, "LONGEST_FILL mode takes num_backoff == 1 (got %d)", c->num_backoff);
  if (c->min_self_match < 1) return fail(SFX_EINVAL, "min_self_match must be >= 1");
  if (c->max_batch < 0) return fail(SFX_EINVAL, "max_batch must be >= 0");
  if (c->max_seq < 0 || c->max_seq > kMaxSeq)
    return fail(SFX_EINVAL, "max_seq=%d outside [0,%d]", c->max_seq, kMaxSeq);
  if (c->max_sampled < 0 || c->max_sampled > kMaxT)
    return fail(SFX_EINVAL, "max_sampled=%d outside [0,%d]", c->max_sampled, kMaxT);
  if (c->spec_factor_ppm < 0) return fail(SFX_EINVAL, "max_spec_factor must be >= 0");
  if (c->spec_offset_ppm < 0) return fail(SFX_EINVAL, "max_spec_offset must be >= 0");
  if (c->spec_factor_ppm > (int64_t)1e15 || c->spec_offset_ppm > (int64_t)1e15)
    return fail(SFX_EINVAL, "spec factor/offset too large");
  if (c->min_token_prob_ppm < 0 || c->min_token_prob_ppm > 1000000)
    return fail(SFX_EINVAL, "min_token_prob must be in [0,1]");
  if (c->corpus_capacity < 0 || c->corpus_capacity > (int64_t(1) << 30))
    return fail(SFX_EINVAL, "corpus_capacity outside [0, 2^30]");
  if (c->corpus_capacity > 0) {
    if (c->max_tree_depth < 2)
      return fail(SFX_EINVAL, "a corpus needs max_tree_depth >= 2 (last-2 probe)");
    if (c->min_corpus_match < 2 || c->min_corpus_match > c->max_tree_depth)
      return fail(SFX_EINVAL, "min_corpus_match=%d outside [2, max_tree_depth]",
                  c->min_corpus_match);
  }
  if (c->flags & ~(SFX_FLAG_STREAM_CONTEXT | SFX_FLAG_CHECK_INPUTS | SFX_FLAG_TREE_DEPTH_CAP))
    return fail(SFX_EINVAL, "unknown flags 0x%x", c->flags);
  if (c->reserved != 0) return fail(SFX_EINVAL, "reserved must be 0");
  return SFX_OK;
}

// Host side of the suffix-array round counts: pinned counts and events.
bool alloc_poll(SaPoll* p) {
  *p = SaPoll{};
  if (hipHostMalloc((void**)&p->counts, sizeof(int32_t) * kPollRounds, hipHostMallocDefault) !=
      hipSuccess) {
    p->counts = nullptr;
    return false;
  }
  for (int i = 0; i < kPollRounds; ++i)
    if (hipEventCreateWithFlags(&p->ev[i], hipEventDisableTiming) != hipSuccess) {
      p->ev[i] = nullptr;
      return false;
    }
  return true;
}

void free_poll(SaPoll* p) {
  for (int i = 0; i < kPollRounds; ++i)
    if (p->ev[i]) (void)hipEventDestroy(p->ev[i]);
  if (p->counts) (void)hipHostFree(p->counts);
  *p = SaPoll{};
}

void free_ctx(sfx_ctx* c) {
  auto f = [](void* p) {
    if (p) (void)hipFree(p);
  };
  f(c->pick);
  f(c->masked);
  f(c->counted);
  f(c->accept);
  f(c->err);
  f(c->ctl);
  f(c->ring);
  f(c->doc_start);
  f(c->doc_off);
  f(c->doc_idx);
  f(c->inflight);
  f(c->range_dev);
  for (auto& b : c->idx) {
    f(b.text);
    f(b.sa);
    for (int g = 0; g < kNG; ++g) {
      f(b.pl[g]);
      f(b.ht[g]);
    }
  }
  f(c->sa_ws);
  f(c->pair_group);
  f(c->pair_seg);
  f(c->pair_list);
  free_poll(&c->poll);
  if (c->side) (void)hipStreamDestroy(c->side);
  if (c->ev_snap) (void)hipEventDestroy(c->ev_snap);
  if (c->ev_done) (void)hipEventDestroy(c->ev_done);
  delete c;
}

// Table size for n snapshot tokens: a power of two at least twice any possible group count.
uint32_t slots_for(const sfx_ctx* c, int64_t n) {
  uint32_t s = next_pow2_u32((uint64_t)(n < 1 ? 1 : n) * 2);
  return s > c->ht_slots ? c->ht_slots : s;
}

// Suffix array and probe tables of buffer `buf`, whose snapshot range was recorded on `st`.
int build_index(sfx_ctx* c, int buf, hipStream_t st, uint32_t* mask_out) {
  int64_t range[2] = {0, 0};
  HIP_OR_RETURN(hipMemcpyAsync(range, c->range_dev, sizeof range, hipMemcpyDeviceToHost, st),
                "snapshot range read");
  HIP_OR_RETURN(hipStreamSynchronize(st), "snapshot wait");
  const int64_t n = range[1] - range[0];
  if (n < 0 || n > c->cap) return fail(SFX_EHIP, "corrupt snapshot range");
  IndexBuf& b = c->idx[buf];
  c->last_index_tokens = n;
  HIP_OR_RETURN(sa_build(b.text, n, b.sa, c->saw, st, &c->poll, nullptr), "suffix array build");
  const uint32_t slots = slots_for(c, n);
  HIP_OR_RETURN(ngram_tables_build(b.text, b.sa, n, b.pl, b.ht, slots, c->saw, st),
                "probe table build");
  *mask_out = slots - 1;
  return SFX_OK;
}

int check_ctx(sfx_ctx* c) {
  if (!c) return fail(SFX_EINVAL, "context is NULL");
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess && dev != c->device)
    return fail(SFX_EINVAL, "context was created on device %d, current device is %d", c->device,
                dev);
  return SFX_OK;
}

bool checking(const sfx_ctx* c) { return (c->cfg.flags & SFX_FLAG_CHECK_INPUTS) != 0; }

void finish_async(sfx_ctx* c) {
  if (c->worker.joinable()) c->worker.join();
}

// ------------------------------------------------------------------ corpus files
// Copies n elements of a device ring of `size` elements starting at logical index `from`
// (slot from % size) into host memory, in at most two pieces.
template <typename T>
hipError_t ring_to_host(T* dst, const T* ring, int64_t size, int64_t from, int64_t n,
                        hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t s0 = from % size;
  const int64_t first = n < size - s0 ? n : size - s0;
  hipError_t e = hipMemcpyAsync(dst, ring + s0, sizeof(T) * first, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess && n > first)
    e = hipMemcpyAsync(dst + first, ring, sizeof(T) * (n - first), hipMemcpyDeviceToHost, st);
  return e;
}

template <typename T>
hipError_t host_to_ring(T* ring, int64_t size, int64_t from, const T* src, int64_t n,
                        hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t s0 = from % size;
  const int64_t first = n < size - s0 ? n : size - s0;
  hipError_t e = hipMemcpyAsync(ring + s0, src, sizeof(T) * first, hipMemcpyHostToDevice, st);
  if (e == hipSuccess && n > first)
    e = hipMemcpyAsync(ring, src + first, sizeof(T) * (n - first), hipMemcpyHostToDevice, st);
  return e;
}

int swap_in(sfx_ctx* c, hipStream_t st) {
  HIP_OR_RETURN(hipStreamWaitEvent(st, c->ev_done, 0), "wait for rebuild");
  HIP_OR_RETURN(launch_swap(c->ctl, c->async_buf, c->async_mask, st), "swap launch");
  c->active_host = c->async_buf;
  c->live_epoch = c->snap_epoch;
  c->async_state.store(0);
  return SFX_OK;
}

}  // namespace

extern "C" {

const char* sfx_last_error(void) { return g_err.c_str(); }

int sfx_create(const sfx_config* cfg, sfx_ctx** out) {
  if (!out) return fail(SFX_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = validate(cfg);
  if (rc) return rc;
  sfx_ctx* c = new sfx_ctx();
  c->cfg = *cfg;
  if (hipGetDevice(&c->device) != hipSuccess) {
    delete c;
    return fail(SFX_EHIP, "no HIP device");
  }
  hipError_t e = propose_prepare();
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, "propose kernel attributes");
  }
  {
    const bool corpus = cfg->corpus_capacity > 0;
    const bool staged = propose_staged(cfg->max_seq, cfg->max_sampled,
                                       (cfg->flags & SFX_FLAG_STREAM_CONTEXT) != 0, corpus,
                                       cfg->num_backoff);
    const size_t lds =
        propose_dynamic_lds(staged, cfg->max_seq, cfg->max_sampled, corpus, cfg->num_backoff);
    if (lds + propose_static_lds() > kLdsBytes) {
      delete c;
      return fail(SFX_EINVAL, "max_seq=%d with max_sampled=%d needs %zu bytes of LDS per request, "
                  "more than the %zu a workgroup has", cfg->max_seq, cfg->max_sampled,
                  lds + propose_static_lds(), kLdsBytes);
    }
  }
  {
    const int rows = cfg->max_batch > 0 ? cfg->max_batch : 1;
    if (hipMalloc((void**)&c->pick, 4 * (size_t)rows) != hipSuccess ||
        hipMalloc((void**)&c->masked, 8 * (size_t)rows) != hipSuccess ||
        hipMalloc((void**)&c->counted,
                  4 * (size_t)rows * (cfg->max_sampled > 0 ? cfg->max_sampled : 1)) !=
            hipSuccess ||
        hipMalloc((void**)&c->accept, sizeof(unsigned long long) * kAcceptEntries) != hipSuccess ||
        hipMalloc((void**)&c->err, sizeof(uint32_t)) != hipSuccess) {
      free_ctx(c);
      return fail(SFX_ENOMEM, "device allocation failed for the acceptance table");
    }
    if ((e = launch_accept_reset(c->accept, c->pick, rows, nullptr)) != hipSuccess ||
        (e = launch_clear_word(c->err, nullptr)) != hipSuccess ||
        (e = hipStreamSynchronize(nullptr)) != hipSuccess) {
      free_ctx(c);
      return hip_fail(e, "acceptance table init");
    }
  }
  if (cfg->corpus_capacity > 0) {
    c->cap = cfg->corpus_capacity;
    c->dcap = c->cap + 1;
    c->ht_slots = next_pow2_u32((uint64_t)c->cap * 2);
    auto al = [&](void** p, size_t bytes) { return hipMalloc(p, bytes) == hipSuccess; };
    bool ok = al((void**)&c->ctl, sizeof(Ctl)) && al((void**)&c->ring, 4 * c->cap) &&
              al((void**)&c->doc_start, 8 * c->dcap) &&
              al((void**)&c->doc_off, 8 * (kIngestChunk + 1)) &&
              al((void**)&c->doc_idx, 4 * (kIngestChunk + 1)) &&
              al((void**)&c->inflight, 4 * (2 * (size_t)cfg->max_batch + 2 * kIngestChunk)) &&
              al((void**)&c->range_dev, 32);
    for (int bi = 0; bi < 2 && ok; ++bi) {
      IndexBuf& b = c->idx[bi];
      ok = al((void**)&b.text, 4 * (c->cap + kTextSlack)) && al((void**)&b.sa, 4 * c->cap);
      for (int g = 0; g < kNG && ok; ++g)
        ok = al((void**)&b.pl[g], 4 * c->cap) &&
             al((void**)&b.ht[g], sizeof(NgramSlot) * (size_t)c->ht_slots);
    }
    c->sa_ws_bytes = sa_workspace_bytes(c->cap);
    ok = ok && al(&c->sa_ws, c->sa_ws_bytes);
    if (ok && cfg->max_batch >= 1 && cfg->max_batch <= kPairMaxBatch) {
      const int mb = cfg->max_batch;
      c->pair_slots = pair_slots(mb);
      ok = al((void**)&c->pair_group, 4 * (size_t)mb) &&
           al((void**)&c->pair_seg, sizeof(PairSeg) * (size_t)(mb + 1) * kPairSlices) &&
           al((void**)&c->pair_list, 4 * pair_list_entries(c->cap));
    }
    if (!ok) {
      free_ctx(c);
      return fail(SFX_ENOMEM, "device allocation failed for a corpus of %lld tokens",
                  (long long)cfg->corpus_capacity);
    }
    c->saw = sa_carve(c->sa_ws, c->cap);
    if (!alloc_poll(&c->poll) ||
        hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&c->ev_snap, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c->ev_done, hipEventDisableTiming) != hipSuccess) {
      free_ctx(c);
      return fail(SFX_EHIP, "stream/event creation failed");
    }
    if ((e = launch_ctl_init(c->ctl, c->side)) != hipSuccess ||
        (e = hipMemsetAsync(c->inflight, 0, 4 * (size_t)cfg->max_batch, c->side)) !=
            hipSuccess ||
        (e = launch_claims_init(c->inflight + cfg->max_batch, cfg->max_batch, c->side)) !=
            hipSuccess ||
        (e = hipStreamSynchronize(c->side)) != hipSuccess) {
      free_ctx(c);
      return hip_fail(e, "control block init");
    }
  }
  *out = c;
  return SFX_OK;
}

void sfx_destroy(sfx_ctx* c) {
  if (!c) return;
  finish_async(c);
  if (c->side) (void)hipStreamSynchronize(c->side);
  free_ctx(c);
}

}  // extern "C"

// The per-length draft cap and the per-c0 stop count of the drafter step (suffix-gpu page, How it
// works step 3 and Quickstart; gitcode blog section 4): in SCORED mode a candidate of match
// length l drafts at most floor((factor * l + offset) / 1e6) tokens, and the chain stops at a
// vote count c with c * 1e6 < min_token_prob * c0.  Both are exact integer ratios, taken here
// once per call.  With SFX_FLAG_TREE_DEPTH_CAP the match length plus the draft length stays
// within max_tree_depth.
static void fill_tables(const sfx_config& g, int32_t k, ProposeArgs* a) {
  const bool scored = g.mode == SFX_MODE_SCORED;
  for (int l = 0; l <= kMaxD; ++l) {
    int64_t cap = k;
    if (scored) {
      const int64_t c = (g.spec_factor_ppm * l + g.spec_offset_ppm) / 1000000;
      if (c < cap) cap = c < 0 ? 0 : c;
    }
    if (g.flags & SFX_FLAG_TREE_DEPTH_CAP) {
      const int64_t room = (int64_t)g.max_tree_depth - l;
      if (room < cap) cap = room < 0 ? 0 : room;
    }
    a->cap_of_len[l] = (uint8_t)cap;
  }
  for (int c0 = 0; c0 <= kMaxM; ++c0)
    a->min_count[c0] =
        scored ? (uint8_t)((g.min_token_prob_ppm * c0 + 999999) / 1000000) : (uint8_t)0;
}

#ifndef SFX_PHASE_TRACE
#define SFX_PHASE_TRACE 0
#endif
#if SFX_PHASE_TRACE
// Phase-trace builds only: the device buffer that every propose launch stamps its wavefronts'
// phase times into ([B][16][kTracePhases] uint64), or nullptr.
static uint64_t* g_phase_trace = nullptr;
extern "C" void sfx_debug_phase_trace(void* buf) { g_phase_trace = (uint64_t*)buf; }
#endif

// The drafter step with draft width k (at most the configured one), after argument checks.
// With force_pairs the delta grouping passes run even when no ingest is pending (a captured
// chain meant for engines that ingest every step).  A call with no ingest pending (nothing
// ingested since the live snapshot was taken, so no delta) launches the kernel without the
// general path; a replayable one (a chain captured into a graph, here or by the caller on a
// capturing stream, run later against whatever corpus is then live) always takes the one
// with it.
static int propose_k(sfx_ctx* c, int32_t k, int32_t B, int32_t S, int32_t T,
                     const int32_t* ntns, const int32_t* tok, const int32_t* samp,
                     int32_t* draft, int32_t* nvalid, void* stream, bool force_pairs = false,
                     bool replayable = false) {
  const sfx_config& g = c->cfg;
  if (B < 0 || S < 0 || T < 0) return fail(SFX_EINVAL, "negative shape B=%d S=%d T=%d", B, S, T);
  if (B > g.max_batch || S > g.max_seq || T > g.max_sampled)
    return fail(SFX_ECAPACITY, "shape B=%d S=%d T=%d above max_batch=%d max_seq=%d max_sampled=%d",
                B, S, T, g.max_batch, g.max_seq, g.max_sampled);
  if (B == 0) return SFX_OK;
  if (!ntns || !draft || !nvalid || (S > 0 && !tok) || (T > 0 && !samp))
    return fail(SFX_EINVAL, "NULL array argument");
  ProposeArgs a{};
  a.B = B;
  a.S = S;
  a.T = T;
  a.ntns = ntns;
  a.tok = tok;
  a.samp = samp;
  a.draft = draft;
  a.nvalid = nvalid;
  a.k = k;
  a.D = g.max_tree_depth;
  a.nb = g.num_backoff;
  a.M = g.max_occurrences;
  a.mode = g.mode;
  a.min_self = g.min_self_match;
  a.min_corpus = g.min_corpus_match;
  fill_tables(g, k, &a);
  a.ctl = c->ctl;
  a.idx[0] = c->idx[0];
  a.idx[1] = c->idx[1];
  a.ring = c->ring;
  a.ring_cap = c->cap > 0 ? c->cap : 1;
  a.stream_ctx = (g.flags & SFX_FLAG_STREAM_CONTEXT) != 0;
  a.pick = c->pick;
  a.err = c->err;
#if SFX_PHASE_TRACE
  a.trace = g_phase_trace;
#endif
  if (c->pair_list && B <= kPairMaxBatch && (force_pairs || c->ingest_epoch != c->live_epoch)) {
    PairIndexArgs p{};
    p.B = B;
    p.S = S;
    p.T = T;
    p.D = g.max_tree_depth;
    p.ntns = ntns;
    p.tok = tok;
    p.samp = samp;
    p.ctl = c->ctl;
    p.ring = c->ring;
    p.ring_cap = c->cap;
    p.slots = c->pair_slots;
    p.group = c->pair_group;
    p.seg = c->pair_seg;
    p.list = c->pair_list;
    HIP_OR_RETURN(launch_pair_index(p, (hipStream_t)stream), "pair index launch");
    a.pair_group = c->pair_group;
    a.pair_seg = c->pair_seg;
    a.pair_list = c->pair_list;
  }
  bool general = replayable || force_pairs || c->ingest_epoch != c->live_epoch;
  if (!general) {
    // a launch captured into a graph (by the caller) is replayed later, whatever the corpus is
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    HIP_OR_RETURN(hipStreamIsCapturing((hipStream_t)stream, &cs), "capture status");
    general = cs != hipStreamCaptureStatusNone;
  }
  HIP_OR_RETURN(launch_propose(a, general, (hipStream_t)stream), "propose launch");
  return SFX_OK;
}

extern "C" {

int sfx_propose(sfx_ctx* c, int32_t B, int32_t S, int32_t T, const int32_t* ntns,
                const int32_t* tok, const int32_t* samp, int32_t* draft, int32_t* nvalid,
                void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  rc = propose_k(c, c->cfg.k, B, S, T, ntns, tok, samp, draft, nvalid, stream);
  if (rc || !checking(c)) return rc;
  HIP_OR_RETURN(launch_check_propose(B, S, T, ntns, tok, samp, nullptr, c->err,
                                     (hipStream_t)stream), "input check launch");
  return SFX_OK;
}

int sfx_propose_masked(sfx_ctx* c, int32_t B, int32_t S, const int32_t* ntns,
                       const int32_t* tok, const int32_t* mask, int32_t* draft,
                       int32_t* nvalid, void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  const sfx_config& g = c->cfg;
  if (B < 0 || S < 0) return fail(SFX_EINVAL, "negative shape B=%d S=%d", B, S);
  if (B > g.max_batch || S > g.max_seq || g.max_sampled < 1)
    return fail(SFX_ECAPACITY, "shape B=%d S=%d above max_batch=%d max_seq=%d (or max_sampled 0)",
                B, S, g.max_batch, g.max_seq);
  if (B == 0) return SFX_OK;
  if (!ntns || !mask || !draft || !nvalid || (S > 0 && !tok))
    return fail(SFX_EINVAL, "NULL array argument");
  hipStream_t st = (hipStream_t)stream;
  int32_t* n2 = c->masked;
  int32_t* s2 = c->masked + g.max_batch;
  HIP_OR_RETURN(launch_masked_prep(B, S, ntns, tok, mask, n2, s2, st), "masked prep launch");
  rc = propose_k(c, g.k, B, S, 1, n2, tok, s2, draft, nvalid, stream);
  if (rc || !checking(c)) return rc;
  HIP_OR_RETURN(launch_check_propose(B, S, 0, ntns, tok, nullptr, nullptr, c->err, st),
                "input check launch");
  return SFX_OK;
}

int sfx_propose_counts(sfx_ctx* c, int32_t k, int32_t B, int32_t S, int32_t T,
                       const int32_t* ntns, const int32_t* tok, const int32_t* sampled,
                       const int32_t* counts, int32_t* draft, int32_t* nvalid, void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (k < 1) return fail(SFX_EINVAL, "k=%d below 1", k);
  if (k > c->cfg.k) return fail(SFX_ECAPACITY, "k=%d above the configured k=%d", k, c->cfg.k);
  if (B < 0 || T < 0) return fail(SFX_EINVAL, "negative shape B=%d T=%d", B, T);
  if (B > c->cfg.max_batch || T > c->cfg.max_sampled)
    return fail(SFX_ECAPACITY, "shape B=%d T=%d above max_batch=%d max_sampled=%d", B, T,
                c->cfg.max_batch, c->cfg.max_sampled);
  if (B == 0) return SFX_OK;
  if (!counts || (T > 0 && !sampled)) return fail(SFX_EINVAL, "NULL array argument");
  HIP_OR_RETURN(launch_counts_prep(B, T, sampled, counts, c->counted, (hipStream_t)stream),
                "counts prep launch");
  rc = propose_k(c, k, B, S, T, ntns, tok, c->counted, draft, nvalid, stream);
  if (rc || !checking(c)) return rc;
  HIP_OR_RETURN(launch_check_propose(B, S, T, ntns, tok, sampled, counts, c->err,
                                     (hipStream_t)stream), "input check launch");
  return SFX_OK;
}

int sfx_update_state(int32_t B, int32_t S, int32_t T, int32_t* tok, const int32_t* ntns,
                     const int32_t* samp, int32_t* nout, void* stream) {
  if (B < 0 || S < 0 || T < 0) return fail(SFX_EINVAL, "negative shape");
  if (B == 0) return SFX_OK;
  if (!ntns || !nout || (S > 0 && !tok) || (T > 0 && !samp))
    return fail(SFX_EINVAL, "NULL array argument");
  HIP_OR_RETURN(launch_update_state(B, S, T, tok, ntns, samp, nout, (hipStream_t)stream),
                "update_state launch");
  return SFX_OK;
}

static int ingest_common(sfx_ctx* c, IngestArgs a, int hint, hipStream_t st) {
  a.ctl = c->ctl;
  a.ring = c->ring;
  a.cap = c->cap;
  a.doc_start = c->doc_start;
  a.dcap = c->dcap;
  a.doc_off = c->doc_off;
  a.doc_idx = c->doc_idx;
  const int R = a.R;
  ++c->ingest_epoch;
  for (int r0 = 0; r0 < R; r0 += kIngestChunk) {
    IngestArgs ch = a;
    ch.R = R - r0 < kIngestChunk ? R - r0 : kIngestChunk;
    if (ch.doc_offsets) ch.doc_offsets += r0;
    else {
      ch.row_indices += r0;
      ch.lengths += r0;
    }
    HIP_OR_RETURN(launch_ingest(ch, hint, st), "ingest launch");
  }
  return SFX_OK;
}

int sfx_harvest_finished(sfx_ctx* c, int32_t R, const int32_t* rows, const int32_t* lengths,
                         const int32_t* tok, int32_t num_rows, int32_t S, void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!c->ctl) return fail(SFX_ESTATE, "context has no corpus (corpus_capacity == 0)");
  if (R < 0 || S < 0 || num_rows < 0) return fail(SFX_EINVAL, "negative shape");
  if (R == 0) return SFX_OK;
  if (!rows || !lengths || (S > 0 && num_rows > 0 && !tok))
    return fail(SFX_EINVAL, "NULL array argument");
  IngestArgs a{};
  a.R = R;
  a.row_indices = rows;
  a.lengths = lengths;
  a.num_rows = num_rows;
  a.S = S;
  a.tokens = tok;
  if (checking(c))
    HIP_OR_RETURN(launch_check_ingest(R, rows, lengths, num_rows, S, nullptr, tok, c->err,
                                      (hipStream_t)stream), "input check launch");
  return ingest_common(c, a, S, (hipStream_t)stream);
}

int sfx_ingest(sfx_ctx* c, int32_t num_docs, const int64_t* offs, const int32_t* tokens,
               void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!c->ctl) return fail(SFX_ESTATE, "context has no corpus (corpus_capacity == 0)");
  if (num_docs < 0) return fail(SFX_EINVAL, "negative num_docs");
  if (num_docs == 0) return SFX_OK;
  if (!offs || !tokens) return fail(SFX_EINVAL, "NULL array argument");
  IngestArgs a{};
  a.R = num_docs;
  a.doc_offsets = offs;
  a.tokens = tokens;
  if (checking(c))
    HIP_OR_RETURN(launch_check_ingest(num_docs, nullptr, nullptr, 0, 0, offs, tokens, c->err,
                                      (hipStream_t)stream), "input check launch");
  return ingest_common(c, a, 1 << 16, (hipStream_t)stream);
}

int sfx_ingest_inflight(sfx_ctx* c, int32_t R, const int32_t* rows, const int32_t* lengths,
                        const int32_t* final_flags, const int32_t* tok, int32_t num_rows,
                        int32_t S, int32_t min_chunk, void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!c->ctl) return fail(SFX_ESTATE, "context has no corpus (corpus_capacity == 0)");
  if (R < 0 || S < 0 || num_rows < 0 || min_chunk < 0)
    return fail(SFX_EINVAL, "negative shape or min_chunk");
  if (R == 0) return SFX_OK;
  if (R > kIngestChunk)
    return fail(SFX_ECAPACITY, "R=%d above %d entries per in-flight ingest", R, kIngestChunk);
  if (!rows || !lengths || (S > 0 && num_rows > 0 && !tok))
    return fail(SFX_EINVAL, "NULL array argument");
  hipStream_t st = (hipStream_t)stream;
  const int mb = c->cfg.max_batch;
  if (checking(c))
    HIP_OR_RETURN(launch_check_ingest(R, rows, lengths, num_rows < mb ? num_rows : mb, S, nullptr,
                                      tok, c->err, st), "input check launch");
  InflightArgs f{};
  f.R = R;
  f.row_indices = rows;
  f.lengths = lengths;
  f.final_flags = final_flags;
  f.num_rows = num_rows;
  f.S = S;
  f.min_chunk = min_chunk;
  f.max_rows = mb;
  f.cursor = c->inflight;
  f.claim = c->inflight + mb;
  f.seg_start = c->inflight + 2 * (size_t)mb;
  f.seg_len = f.seg_start + kIngestChunk;
  HIP_OR_RETURN(launch_inflight_prepare(f, st), "in-flight prepare launch");
  IngestArgs a{};
  a.R = R;
  a.row_indices = rows;
  a.lengths = lengths;
  a.num_rows = num_rows;
  a.S = S;
  a.tokens = tok;
  a.seg_start = f.seg_start;
  a.seg_len = f.seg_len;
  return ingest_common(c, a, S, st);
}

static int pick_buffer(sfx_ctx* c) { return c->active_host == 0 ? 1 : 0; }

int sfx_rebuild(sfx_ctx* c, void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!c->ctl) return fail(SFX_ESTATE, "context has no corpus (corpus_capacity == 0)");
  if (c->async_state.load() != 0) return fail(SFX_ESTATE, "an asynchronous rebuild is in flight");
  hipStream_t st = (hipStream_t)stream;
  const int buf = pick_buffer(c);
  const uint64_t epoch = c->ingest_epoch;
  HIP_OR_RETURN(launch_snapshot(c->ctl, c->ring, c->cap, c->idx[buf].text, buf, c->range_dev, st),
                "snapshot launch");
  uint32_t mask = 0;
  if ((rc = build_index(c, buf, st, &mask)) != SFX_OK) return rc;
  if (c->fail_next.exchange(0)) return fail(SFX_EHIP, "injected rebuild failure");
  HIP_OR_RETURN(launch_swap(c->ctl, buf, mask, st), "swap launch");
  c->active_host = buf;
  c->live_epoch = epoch;
  return SFX_OK;
}

int sfx_rebuild_async(sfx_ctx* c, void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!c->ctl) return fail(SFX_ESTATE, "context has no corpus (corpus_capacity == 0)");
  if (c->async_state.load() != 0) return fail(SFX_ESTATE, "an asynchronous rebuild is in flight");
  finish_async(c);
  hipStream_t st = (hipStream_t)stream;
  const int buf = pick_buffer(c);
  HIP_OR_RETURN(launch_snapshot(c->ctl, c->ring, c->cap, c->idx[buf].text, buf, c->range_dev, st),
                "snapshot launch");
  HIP_OR_RETURN(hipEventRecord(c->ev_snap, st), "snapshot event");
  c->async_buf = buf;
  c->snap_epoch = c->ingest_epoch;
  c->async_err = SFX_OK;
  c->async_state.store(1);
  c->worker = std::thread([c, buf]() {
    (void)hipSetDevice(c->device);
    int r = SFX_OK;
    uint32_t mask = 0;
    if (hipStreamWaitEvent(c->side, c->ev_snap, 0) != hipSuccess) r = fail(SFX_EHIP, "wait");
    if (r == SFX_OK) r = build_index(c, buf, c->side, &mask);
    if (r == SFX_OK && hipEventRecord(c->ev_done, c->side) != hipSuccess)
      r = fail(SFX_EHIP, "rebuild event");
    if (r == SFX_OK && hipStreamSynchronize(c->side) != hipSuccess)
      r = fail(SFX_EHIP, "rebuild wait");
    if (r == SFX_OK && c->fail_next.exchange(0)) r = fail(SFX_EHIP, "injected rebuild failure");
    c->async_mask = mask;
    c->async_err = r;
    if (r != SFX_OK) c->async_msg = g_err;
    c->async_state.store(2);
  });
  return SFX_OK;
}

int sfx_poll(sfx_ctx* c, int32_t* swapped, void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (swapped) *swapped = 0;
  if (!c->ctl || c->async_state.load() != 2) return SFX_OK;
  finish_async(c);
  if (c->async_err != SFX_OK) {
    c->async_state.store(0);
    return fail(c->async_err, "asynchronous rebuild failed: %s", c->async_msg.c_str());
  }
  if ((rc = swap_in(c, (hipStream_t)stream)) != SFX_OK) return rc;
  if (swapped) *swapped = 1;
  return SFX_OK;
}

int sfx_wait_rebuild(sfx_ctx* c, void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!c->ctl || c->async_state.load() == 0) return SFX_OK;
  finish_async(c);
  if (c->async_err != SFX_OK) {
    c->async_state.store(0);
    return fail(c->async_err, "asynchronous rebuild failed: %s", c->async_msg.c_str());
  }
  return swap_in(c, (hipStream_t)stream);
}

int sfx_corpus_snapshot(sfx_ctx* c, int32_t* text_out, int64_t cap, int64_t* n_out,
                        void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!n_out) return fail(SFX_EINVAL, "n_out is NULL");
  *n_out = 0;
  if (!c->ctl) return SFX_OK;
  hipStream_t st = (hipStream_t)stream;
  HIP_OR_RETURN(launch_live_range(c->ctl, c->range_dev + 2, st), "range launch");
  int64_t range[2];
  HIP_OR_RETURN(hipMemcpyAsync(range, c->range_dev + 2, sizeof range, hipMemcpyDeviceToHost, st),
                "range read");
  HIP_OR_RETURN(hipStreamSynchronize(st), "range wait");
  const int64_t n = range[1] - range[0];
  *n_out = n;
  if (n > cap) return fail(SFX_ECAPACITY, "live corpus has %lld tokens, buffer %lld",
                           (long long)n, (long long)cap);
  if (n > 0 && !text_out) return fail(SFX_EINVAL, "text_out is NULL");
  HIP_OR_RETURN(launch_ring_copy(c->ctl, c->ring, c->cap, text_out, cap, st), "copy launch");
  HIP_OR_RETURN(hipStreamSynchronize(st), "copy wait");
  return SFX_OK;
}

int sfx_rebuild_stats(sfx_ctx* c, int32_t* rounds_out, int64_t* tokens_out) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!rounds_out || !tokens_out) return fail(SFX_EINVAL, "NULL output argument");
  if (!c->ctl) return fail(SFX_ESTATE, "context has no corpus (corpus_capacity == 0)");
  if (c->async_state.load() == 1) return fail(SFX_ESTATE, "an asynchronous rebuild is in flight");
  const int e = c->poll.enqueued;
  if (e > 0) HIP_OR_RETURN(hipEventSynchronize(c->poll.ev[e - 1]), "last round wait");
  int rounds = c->last_index_tokens > 0 ? 1 : 0;
  for (int i = 0; i < e && c->poll.counts[i] > 0; ++i) ++rounds;
  *rounds_out = rounds;
  *tokens_out = c->last_index_tokens;
  return SFX_OK;
}

int sfx_debug_index(sfx_ctx* c, int32_t* text_out, int32_t* sa_out, int64_t cap, int64_t* n_out,
                    void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!n_out) return fail(SFX_EINVAL, "n_out is NULL");
  *n_out = 0;
  if (!c->ctl) return fail(SFX_ESTATE, "context has no corpus (corpus_capacity == 0)");
  hipStream_t st = (hipStream_t)stream;
  Ctl h;
  HIP_OR_RETURN(hipMemcpyAsync(&h, c->ctl, sizeof h, hipMemcpyDeviceToHost, st), "control read");
  HIP_OR_RETURN(hipStreamSynchronize(st), "control wait");
  if (h.active < 0) return SFX_OK;  // no live index
  const int64_t n = h.snap_end[h.active] - h.snap_start[h.active];
  *n_out = n;
  if (n > cap) return fail(SFX_ECAPACITY, "live index has %lld tokens, buffers %lld",
                           (long long)n, (long long)cap);
  if (n > 0 && (!text_out || !sa_out)) return fail(SFX_EINVAL, "NULL array argument");
  const IndexBuf& b = c->idx[h.active];
  HIP_OR_RETURN(hipMemcpyAsync(text_out, b.text, 4 * (size_t)n, hipMemcpyDeviceToDevice, st),
                "text copy");
  HIP_OR_RETURN(hipMemcpyAsync(sa_out, b.sa, 4 * (size_t)n, hipMemcpyDeviceToDevice, st),
                "suffix array copy");
  HIP_OR_RETURN(hipStreamSynchronize(st), "copy wait");
  return SFX_OK;
}

int sfx_accept_estimate(sfx_ctx* c, int32_t B, int32_t* est_ppm, void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (B < 0) return fail(SFX_EINVAL, "negative B");
  if (B > c->cfg.max_batch) return fail(SFX_ECAPACITY, "B=%d above max_batch=%d", B,
                                        c->cfg.max_batch);
  if (B == 0) return SFX_OK;
  if (!est_ppm) return fail(SFX_EINVAL, "NULL array argument");
  HIP_OR_RETURN(launch_accept_estimate(B, c->cfg.k, c->pick, c->accept, est_ppm,
                                       (hipStream_t)stream), "estimate launch");
  return SFX_OK;
}

int sfx_accept_feedback(sfx_ctx* c, int32_t B, const int32_t* num_accepted, void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (B < 0) return fail(SFX_EINVAL, "negative B");
  if (B > c->cfg.max_batch) return fail(SFX_ECAPACITY, "B=%d above max_batch=%d", B,
                                        c->cfg.max_batch);
  if (B == 0) return SFX_OK;
  if (!num_accepted) return fail(SFX_EINVAL, "NULL array argument");
  HIP_OR_RETURN(launch_accept_feedback(B, c->pick, num_accepted, c->accept, (hipStream_t)stream),
                "feedback launch");
  return SFX_OK;
}

int sfx_accept_reset(sfx_ctx* c, void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  const int rows = c->cfg.max_batch > 0 ? c->cfg.max_batch : 1;
  HIP_OR_RETURN(launch_accept_reset(c->accept, c->pick, rows, (hipStream_t)stream),
                "reset launch");
  return SFX_OK;
}

int sfx_accept_counts(sfx_ctx* c, uint64_t* counts, void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!counts) return fail(SFX_EINVAL, "NULL array argument");
  HIP_OR_RETURN(hipMemcpyAsync(counts, c->accept, sizeof(unsigned long long) * kAcceptEntries,
                               hipMemcpyDeviceToDevice, (hipStream_t)stream),
                "counts copy");
  return SFX_OK;
}

int sfx_save(sfx_ctx* c, const char* path, void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!path) return fail(SFX_EINVAL, "path is NULL");
  if (!c->ctl) return fail(SFX_ESTATE, "context has no corpus (corpus_capacity == 0)");
  hipStream_t st = (hipStream_t)stream;
  Ctl k{};
  HIP_OR_RETURN(hipMemcpyAsync(&k, c->ctl, sizeof k, hipMemcpyDeviceToHost, st), "control read");
  HIP_OR_RETURN(hipStreamSynchronize(st), "control wait");
  CorpusImage m;
  CorpusHeader& h = m.h;
  h.capacity = c->cap;
  h.head = k.head;
  h.tail = k.tail;
  h.doc_head = k.doc_head;
  h.doc_tail = k.doc_tail;
  const int a = k.active;
  h.snap_start = a >= 0 ? k.snap_start[a] : 0;
  h.snap_end = a >= 0 ? k.snap_end[a] : 0;
  const int64_t nl = h.head - h.tail, nd = h.doc_head - h.doc_tail, ni = h.snap_end - h.snap_start;
  if (nl < 0 || nl > c->cap || nd < 0 || nd >= c->dcap || ni < 0 || ni > c->cap)
    return fail(SFX_EHIP, "corrupt control block");
  m.live.resize(nl);
  m.starts.resize(nd);
  m.text.resize(ni);
  m.sa.resize(ni);
  HIP_OR_RETURN(ring_to_host(m.live.data(), c->ring, c->cap, h.tail, nl, st), "ring read");
  HIP_OR_RETURN(ring_to_host(m.starts.data(), c->doc_start, c->dcap, h.doc_tail, nd, st),
                "document read");
  if (ni > 0) {
    HIP_OR_RETURN(hipMemcpyAsync(m.text.data(), c->idx[a].text, 4 * ni, hipMemcpyDeviceToHost, st),
                  "index text read");
    HIP_OR_RETURN(hipMemcpyAsync(m.sa.data(), c->idx[a].sa, 4 * ni, hipMemcpyDeviceToHost, st),
                  "suffix array read");
  }
  HIP_OR_RETURN(hipStreamSynchronize(st), "read wait");
  std::string why;
  if ((rc = write_corpus_file(path, &m, &why)) != SFX_OK) return fail(rc, "%s", why.c_str());
  return SFX_OK;
}

int sfx_load(sfx_ctx* c, const char* path, void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!path) return fail(SFX_EINVAL, "path is NULL");
  if (!c->ctl) return fail(SFX_ESTATE, "context has no corpus (corpus_capacity == 0)");
  if (c->async_state.load() != 0) return fail(SFX_ESTATE, "an asynchronous rebuild is in flight");
  CorpusImage m;
  std::string why;
  if ((rc = read_corpus_file(path, c->cap, &m, &why)) != SFX_OK) return fail(rc, "%s", why.c_str());
  const CorpusHeader& h = m.h;
  const int64_t nl = h.head - h.tail, nd = h.doc_head - h.doc_tail, ni = h.snap_end - h.snap_start;
  hipStream_t st = (hipStream_t)stream;
  HIP_OR_RETURN(host_to_ring(c->ring, c->cap, h.tail, m.live.data(), nl, st), "ring write");
  HIP_OR_RETURN(host_to_ring(c->doc_start, c->dcap, h.doc_tail, m.starts.data(), nd, st),
                "document write");
  uint32_t mask = 0;
  IndexBuf& b = c->idx[0];
  if (ni > 0) {
    HIP_OR_RETURN(hipMemcpyAsync(b.text, m.text.data(), 4 * ni, hipMemcpyHostToDevice, st),
                  "index text write");
    HIP_OR_RETURN(hipMemcpyAsync(b.sa, m.sa.data(), 4 * ni, hipMemcpyHostToDevice, st),
                  "suffix array write");
    const uint32_t slots = slots_for(c, ni);
    HIP_OR_RETURN(ngram_tables_build(b.text, b.sa, ni, b.pl, b.ht, slots, c->saw, st),
                  "probe table build");
    mask = slots - 1;
  }
  Ctl k{};
  k.head = h.head;
  k.tail = h.tail;
  k.doc_head = h.doc_head;
  k.doc_tail = h.doc_tail;
  k.snap_start[0] = ni > 0 ? h.snap_start : 0;
  k.snap_end[0] = ni > 0 ? h.snap_end : 0;
  k.ingest_base = h.head;
  k.ht_mask[0] = mask;
  k.active = ni > 0 ? 0 : -1;
  k.pending = -1;
  HIP_OR_RETURN(hipMemcpyAsync(c->ctl, &k, sizeof k, hipMemcpyHostToDevice, st), "control write");
  HIP_OR_RETURN(hipStreamSynchronize(st), "load wait");
  c->active_host = k.active;
  ++c->ingest_epoch;  // the file's documents past its snapshot form a delta
  return SFX_OK;
}

size_t sfx_suffix_array_workspace_bytes(int64_t n) { return sa_workspace_bytes(n); }

int sfx_build_suffix_array(const int32_t* text, int64_t n, int32_t* sa, void* ws, size_t ws_bytes,
                           void* stream) {
  if (n < 0 || n > (int64_t(1) << 30)) return fail(SFX_EINVAL, "n=%lld outside [0,2^30]",
                                                   (long long)n);
  if (n == 0) return SFX_OK;
  if (!text || !sa || !ws) return fail(SFX_EINVAL, "NULL array argument");
  if (ws_bytes < sa_workspace_bytes(n))
    return fail(SFX_ECAPACITY, "workspace of %zu bytes, %zu needed", ws_bytes,
                sa_workspace_bytes(n));
  SaWork w = sa_carve(ws, n);
  SaPoll poll{};
  if (!alloc_poll(&poll)) {
    free_poll(&poll);
    return fail(SFX_ENOMEM, "pinned round-count buffer");
  }
  const hipError_t e = sa_build(text, n, sa, w, (hipStream_t)stream, &poll, nullptr);
  // the events and the pinned counts are freed only after the last enqueued round has read
  // them: wait for the stream first
  const hipError_t e2 = e == hipSuccess ? hipStreamSynchronize((hipStream_t)stream) : e;
  free_poll(&poll);
  HIP_OR_RETURN(e2, "suffix array build");
  return SFX_OK;
}

int sfx_build_suffix_array_noalloc(const int32_t* text, int64_t n, int32_t* sa, void* stream) {
  if (n < 0 || n > kNoAllocMaxTokens)
    return fail(SFX_ECAPACITY, "n=%lld outside [0, %lld], the allocation-free maximum",
                (long long)n, (long long)kNoAllocMaxTokens);
  if (n == 0) return SFX_OK;
  if (!text || !sa) return fail(SFX_EINVAL, "NULL array argument");
  void* ws = nullptr;
  size_t bytes = 0;
  HIP_OR_RETURN(noalloc_workspace(&ws, &bytes), "workspace lookup");
  if (bytes < sa_workspace_bytes(n)) return fail(SFX_ECAPACITY, "workspace too small");
  // no poll: every doubling round is enqueued (rounds after convergence do nothing), with no
  // host memory, event or wait
  HIP_OR_RETURN(sa_build(text, n, sa, sa_carve(ws, n), (hipStream_t)stream, nullptr, nullptr),
                "suffix array build");
  return SFX_OK;
}

int sfx_debug_errors(sfx_ctx* c, uint32_t* bits_out, void* stream) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!bits_out) return fail(SFX_EINVAL, "bits_out is NULL");
  hipStream_t st = (hipStream_t)stream;
  uint32_t v = 0;
  HIP_OR_RETURN(hipMemcpyAsync(&v, c->err, sizeof v, hipMemcpyDeviceToHost, st),
                "error word read");
  HIP_OR_RETURN(launch_clear_word(c->err, st), "error word clear");
  HIP_OR_RETURN(hipStreamSynchronize(st), "error word sync");
  *bits_out = v;
  return SFX_OK;
}

// ------------------------------------------------------------------ batch-bucketed graphs
// RFC page "[RFC]: Suffix decoding on GPU (suffix_gpu)", Design, Proposer bullet: the draft
// chain is captured per batch-size bucket at warm-up, with an eager fallback.  Each bucket keeps
// an exact graph (B == Bp) and a padded one whose first node empties rows B .. Bp-1; only that
// node's arguments change between replays.  Both are captured from the stream (a node added to
// a captured graph by hand measured slower to launch).
constexpr int kMaxGraphBuckets = 64;

}  // extern "C"

struct sfx_graphs {
  sfx_ctx* ctx = nullptr;
  int32_t S = 0, T = 0, flags = 0;
  int32_t* ntns = nullptr;
  int32_t* tok = nullptr;
  int32_t* samp = nullptr;
  int32_t* draft = nullptr;
  int32_t* nvalid = nullptr;
  int32_t* nout = nullptr;
  int nb = 0;
  int32_t bucket[kMaxGraphBuckets]{};
  hipGraph_t graph[kMaxGraphBuckets]{};  // the padded graph (its padding node lives there)
  hipGraphExec_t exact[kMaxGraphBuckets]{};
  hipGraphExec_t padded[kMaxGraphBuckets]{};
  hipGraphNode_t pad[kMaxGraphBuckets]{};
  int32_t pad_from[kMaxGraphBuckets]{};
  int64_t replays = 0, eager = 0;
};

namespace {

// The chain of one step over B rows of the graph set's buffers.
int graph_chain(sfx_graphs* g, int32_t B, hipStream_t st) {
  int rc = check_ctx(g->ctx);
  if (rc) return rc;
  rc = propose_k(g->ctx, g->ctx->cfg.k, B, g->S, g->T, g->ntns, g->tok, g->samp, g->draft,
                 g->nvalid, st, (g->flags & SFX_GRAPHS_DELTA_INDEX) != 0, true);
  if (rc) return rc;
  if (checking(g->ctx))
    HIP_OR_RETURN(launch_check_propose(B, g->S, g->T, g->ntns, g->tok, g->samp, nullptr,
                                       g->ctx->err, st), "input check launch");
  if (g->flags & SFX_GRAPHS_UPDATE_STATE)
    return sfx_update_state(B, g->S, g->T, g->tok, g->ntns, g->samp, g->nout, st);
  return SFX_OK;
}

// Captures bucket i's chain on a stream of its own (thread-local mode: the context's rebuild
// worker may use the runtime meanwhile), once as it is and once behind the padding node (found
// as the capture's only dependency right after it is launched).  Any failure ends the capture,
// drops what was captured, discards that stream and clears the runtime's last error; a graph
// that is missing runs eagerly.
hipGraphExec_t capture_chain(sfx_graphs* g, int i, bool padded, hipGraphNode_t* pad_node,
                             hipGraph_t* graph_out) {
  const int bp = g->bucket[i];
  hipStream_t cap = nullptr;
  if (hipStreamCreateWithFlags(&cap, hipStreamNonBlocking) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    (void)hipStreamDestroy(cap);
    (void)hipGetLastError();
    return nullptr;
  }
  int rc = SFX_OK;
  if (padded) {
    hipStreamCaptureStatus cs;
    const hipGraphNode_t* deps = nullptr;
    size_t ndeps = 0;
    if (launch_pad_rows(g->ntns, g->samp, g->T, bp, bp, cap) != hipSuccess ||
        hipStreamGetCaptureInfo_v2(cap, &cs, nullptr, nullptr, &deps, &ndeps) != hipSuccess ||
        ndeps != 1)
      rc = SFX_EHIP;
    else
      *pad_node = deps[0];
  }
  if (rc == SFX_OK) rc = graph_chain(g, bp, cap);
  if (rc == SFX_OK && (g->flags & SFX_GRAPHS_DEBUG_BREAK_ODD) && (i & 1))
    rc = hipStreamSynchronize(cap) == hipSuccess ? SFX_OK : SFX_EHIP;  // not allowed here
  hipGraph_t gr = nullptr;
  const hipError_t e = hipStreamEndCapture(cap, &gr);
  (void)hipStreamDestroy(cap);
  hipGraphExec_t ex = nullptr;
  if (rc != SFX_OK || e != hipSuccess || !gr ||
      hipGraphInstantiate(&ex, gr, nullptr, nullptr, 0) != hipSuccess) {
    ex = nullptr;
    if (gr) (void)hipGraphDestroy(gr);
    gr = nullptr;
  }
  (void)hipGetLastError();
  if (padded)
    *graph_out = gr;  // the node handle stays valid while its graph lives
  else if (gr)
    (void)hipGraphDestroy(gr);
  return ex;
}

void capture_bucket(sfx_graphs* g, int i, hipStream_t upload) {
  g->exact[i] = capture_chain(g, i, false, nullptr, nullptr);
  if (g->exact[i]) (void)hipGraphUpload(g->exact[i], upload);
  if (g->bucket[i] > 1) {
    g->padded[i] = capture_chain(g, i, true, &g->pad[i], &g->graph[i]);
    g->pad_from[i] = g->bucket[i];
    if (g->padded[i]) (void)hipGraphUpload(g->padded[i], upload);
  }
  (void)hipGetLastError();
}

void free_graphs(sfx_graphs* g) {
  for (int i = 0; i < g->nb; ++i) {
    if (g->exact[i]) (void)hipGraphExecDestroy(g->exact[i]);
    if (g->padded[i]) (void)hipGraphExecDestroy(g->padded[i]);
    if (g->graph[i]) (void)hipGraphDestroy(g->graph[i]);
  }
  delete g;
}

}  // namespace

extern "C" {

int sfx_graphs_create(sfx_ctx* c, int32_t nbuckets, const int32_t* buckets, int32_t S,
                      int32_t T, int32_t* ntns, int32_t* tok, int32_t* samp, int32_t* draft,
                      int32_t* nvalid, int32_t* nout, int32_t flags, void* stream,
                      sfx_graphs** out) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!out) return fail(SFX_EINVAL, "out is NULL");
  *out = nullptr;
  if (nbuckets < 1 || nbuckets > kMaxGraphBuckets || !buckets)
    return fail(SFX_EINVAL, "nbuckets=%d outside [1,%d] (or buckets NULL)", nbuckets,
                kMaxGraphBuckets);
  if (flags & ~(SFX_GRAPHS_EAGER | SFX_GRAPHS_UPDATE_STATE | SFX_GRAPHS_DELTA_INDEX |
                SFX_GRAPHS_DEBUG_BREAK_ODD))
    return fail(SFX_EINVAL, "unknown graph flags 0x%x", flags);
  for (int i = 0; i < nbuckets; ++i) {
    if (buckets[i] < 1 || (i > 0 && buckets[i] <= buckets[i - 1]))
      return fail(SFX_EINVAL, "buckets must be >= 1 and strictly ascending (bucket %d = %d)", i,
                  buckets[i]);
  }
  if (buckets[nbuckets - 1] > c->cfg.max_batch)
    return fail(SFX_ECAPACITY, "bucket %d above max_batch=%d", buckets[nbuckets - 1],
                c->cfg.max_batch);
  if (S < 0 || T < 0) return fail(SFX_EINVAL, "negative shape S=%d T=%d", S, T);
  if (S > c->cfg.max_seq || T > c->cfg.max_sampled)
    return fail(SFX_ECAPACITY, "S=%d T=%d above max_seq=%d max_sampled=%d", S, T,
                c->cfg.max_seq, c->cfg.max_sampled);
  const bool update = (flags & SFX_GRAPHS_UPDATE_STATE) != 0;
  if (!ntns || !draft || !nvalid || (S > 0 && !tok) || (T > 0 && !samp) || (update && !nout))
    return fail(SFX_EINVAL, "NULL buffer argument");
  if (!update && nout) return fail(SFX_EINVAL, "num_tokens_out given without the update flag");
  sfx_graphs* g = new sfx_graphs;
  g->ctx = c;
  g->S = S;
  g->T = T;
  g->flags = flags;
  g->ntns = ntns;
  g->tok = tok;
  g->samp = samp;
  g->draft = draft;
  g->nvalid = nvalid;
  g->nout = nout;
  g->nb = nbuckets;
  for (int i = 0; i < nbuckets; ++i) g->bucket[i] = buckets[i];
  if (!(flags & SFX_GRAPHS_EAGER))
    for (int i = 0; i < nbuckets; ++i) capture_bucket(g, i, (hipStream_t)stream);
  *out = g;
  return SFX_OK;
}

int sfx_graphs_propose(sfx_graphs* g, int32_t B, void* stream) {
  if (!g) return fail(SFX_EINVAL, "graph set is NULL");
  if (B < 0) return fail(SFX_EINVAL, "negative B=%d", B);
  if (B == 0) return SFX_OK;
  hipStream_t st = (hipStream_t)stream;
  int i = 0;
  while (i < g->nb && g->bucket[i] < B) ++i;
  if (i < g->nb) {
    if (B == g->bucket[i] && g->exact[i]) {
      HIP_OR_RETURN(hipGraphLaunch(g->exact[i], st), "graph launch");
      ++g->replays;
      return SFX_OK;
    }
    if (B < g->bucket[i] && g->padded[i]) {
      if (g->pad_from[i] != B) {
        HIP_OR_RETURN(set_pad_rows(g->padded[i], g->pad[i], g->ntns, g->samp, g->T, B,
                                   g->bucket[i]), "pad node update");
        g->pad_from[i] = B;
      }
      HIP_OR_RETURN(hipGraphLaunch(g->padded[i], st), "graph launch");
      ++g->replays;
      return SFX_OK;
    }
  }
  const int rc = graph_chain(g, B, st);
  if (rc == SFX_OK) ++g->eager;
  return rc;
}

int sfx_graphs_stats(sfx_graphs* g, int32_t* nbuckets, uint64_t* exact_mask,
                     uint64_t* padded_mask, int64_t* replays, int64_t* eager_calls) {
  if (!g) return fail(SFX_EINVAL, "graph set is NULL");
  uint64_t em = 0, pm = 0;
  for (int i = 0; i < g->nb; ++i) {
    if (g->exact[i]) em |= 1ull << i;
    if (g->padded[i]) pm |= 1ull << i;
  }
  if (nbuckets) *nbuckets = g->nb;
  if (exact_mask) *exact_mask = em;
  if (padded_mask) *padded_mask = pm;
  if (replays) *replays = g->replays;
  if (eager_calls) *eager_calls = g->eager;
  return SFX_OK;
}

void sfx_graphs_destroy(sfx_graphs* g) {
  if (g) free_graphs(g);
}

int sfx_debug_fail_next_rebuild(sfx_ctx* c) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!c->ctl) return fail(SFX_ESTATE, "context has no corpus (corpus_capacity == 0)");
  c->fail_next.store(1);
  return SFX_OK;
}

}  // extern "C"
