// propose.hip -- the drafter step on gfx950: one workgroup (16 wavefronts) per request.
//
// Steps, in the order of the suffix-gpu page, How it works:
//   1. local match (step 1): each worker wavefront owns a contiguous chunk of end positions; it
//      streams the chunk with coalesced bounds-checked loads (staging it in LDS when the row
//      fits there) and keeps one ballot word per 64 positions marking the positions whose
//      token is the last context token.  The marked positions are listed in order and their
//      backward match lengths against the tail computed, into a per-wavefront histogram.  The
//      histograms give the ladder (t-th largest length) and, per wavefront, the offsets of its
//      earliest continuation sites, so one ordered pass writes the sites of every level;
//   2. global match (step 2; vLLM docs, Model Runner V2: probe by the last 2 and last 4 tokens,
//      extend to the longest match): 2-, 3- and 4-gram probes into hash tables over the
//      suffix-array groups of the live snapshot and backward extension of the 4-gram
//      occurrences.  With a live snapshot, a dedicated wavefront does it while the other
//      fifteen work through the local match, which synchronise among themselves only; without
//      a delta it also derives the corpus ladder and sites.  With a delta (documents appended
//      since the snapshot) the whole workgroup then finds the delta's occurrences -- from the
//      per-call pair index, or by a brute-force scan -- and merges;
//   3. expansion (step 3): one wavefront per candidate votes depth by depth over its sites
//      (one ballot pair when every alive site agrees or one token holds a majority, ballots
//      per token when few sites are alive, an LDS hash otherwise); stop rule and score use
//      integer cross-multiplication; selection and the [k] output row follow.
#include <type_traits>

#include "delta_index.h"
#include "propose.h"

namespace sfx {

namespace {

constexpr int NT = 1024;
constexpr int NW = NT / 64;
constexpr int GW = NW - 1;          // the corpus wavefront of the fast path
constexpr int kVoteSlots = 256;
constexpr int kSmallVote = 24;      // alive sites at or below this vote with ballots

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// DPP controls (GFX9 encoding): cross-lane moves inside the VALU, no LDS round trip.
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i inside a row of 16
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside a half row of 8
constexpr int kDppRowBcast15 = 0x142; // lane 15 of each row to the next row
constexpr int kDppRowBcast31 = 0x143; // lane 31 to rows 2 and 3

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_incl_add(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr1, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr2, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr4, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr8, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xC, 0xF, false);
  return v;
}

// Maximum / minimum over the 64 lanes (every lane takes part).
__device__ __forceinline__ int wave_max(int v) {
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppQuadXor1, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppQuadXor2, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppHalfMirror, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppMirror, 0xF, 0xF, false));
  const int a0 = __builtin_amdgcn_readlane(v, 0), a1 = __builtin_amdgcn_readlane(v, 16);
  const int a2 = __builtin_amdgcn_readlane(v, 32), a3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(a0, a1), max(a2, a3));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppQuadXor1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppQuadXor2, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppHalfMirror, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppMirror, 0xF, 0xF, false));
  const uint32_t a0 = __builtin_amdgcn_readlane((int)v, 0), a1 = __builtin_amdgcn_readlane((int)v, 16);
  const uint32_t a2 = __builtin_amdgcn_readlane((int)v, 32), a3 = __builtin_amdgcn_readlane((int)v, 48);
  return max(max(a0, a1), max(a2, a3));
}

__device__ __forceinline__ int wave_min(int v) {
  v = min(v, __builtin_amdgcn_mov_dpp(v, kDppQuadXor1, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_mov_dpp(v, kDppQuadXor2, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_mov_dpp(v, kDppHalfMirror, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_mov_dpp(v, kDppMirror, 0xF, 0xF, false));
  const int a0 = __builtin_amdgcn_readlane(v, 0), a1 = __builtin_amdgcn_readlane(v, 16);
  const int a2 = __builtin_amdgcn_readlane(v, 32), a3 = __builtin_amdgcn_readlane(v, 48);
  return min(min(a0, a1), min(a2, a3));
}

__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Exclusive prefix sum of one int per thread over the workgroup; *total gets the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int s = lane < NW ? wsum[lane] : 0;
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) {
      int y = __shfl_up(s, o, 64);
      if (lane >= o) s += y;
    }
    if (lane < NW) wsum[lane] = s;
  }
  __syncthreads();
  int base = wid ? wsum[wid - 1] : 0;
  *total = wsum[NW - 1];
  __syncthreads();
  return base + x - v;
}

// Barrier over the worker wavefronts only, so that the corpus wavefront of the fast path keeps
// working through the local phases: an LDS arrival count.  Every worker wavefront passes each
// such barrier exactly once, so the count reaches k * (workers) at the k-th one; the spin is
// bounded as a guard.
__device__ __forceinline__ void worker_barrier(int* ctr, int target, int lane) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  for (int spin = 0; spin < (1 << 24); ++spin) {
    if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ int ctx_at(const int32_t* row, const int32_t* smp, int n, int x) {
  return x < n ? row[x] : smp[x - n];
}

// Count one vote for `tok` in a wavefront's LDS table; returns the slot used.
__device__ __forceinline__ int vote_insert(int* hk, int* hc, int tok) {
  uint32_t h = ((uint32_t)tok * 0x9E3779B1u) >> 24;
  for (;;) {
    int prev = atomicCAS(&hk[h], -1, tok);
    if (prev == -1 || prev == tok) {
      atomicAdd(&hc[h], 1);
      return (int)h;
    }
    h = (h + 1) & (kVoteSlots - 1);
  }
}

struct Smem {
  int tail[kMaxD];
  int gtail[kMaxD];
  int whist[NW][kMaxD + 1];
  int wsuf[NW][kMaxD + 2];
  int ghist[kMaxD + 1];
  int dhist[kMaxD + 1];
  int g_off[kNG], g_live[kNG];
  int cand_len[2 * kMaxNB], cand_sup[2 * kMaxNB], cand_c0[2 * kMaxNB], cand_valid[2 * kMaxNB];
  int cand_src[2 * kMaxNB], cand_n[2 * kMaxNB];
  int cand_snum[2 * kMaxNB];  // at most k * M = 4096
  int cand_out[2 * kMaxNB][kMaxK];
  int lsites[kMaxNB][kMaxM];
  long long gsites[kMaxNB][kMaxM];
  int gpl[kNG][kMaxM];  // heads of the live 2-, 3- and 4-gram groups
  int gm4[kMaxM];       // extension lengths of the first 4-gram occurrences
  const int32_t* plp[kNG];
  int wsum[NW + 1];
  int wbar;  // arrivals at the worker-only barriers
};

// Shape of one request and the corpus state it sees.  Every thread derives it from the same
// uniform loads, so no thread waits for another before the staging starts.
struct Req {
  int n, t, L, J, Lcap;
  int act;
  bool has, fast, delta;
  long long snap_start, snap_n, tail_w, delta_lo, delta_hi;
  uint32_t ht_mask;
};

// Flat view of one index buffer.  Separate scalar fields (no arrays) and constant-index
// selects keep the kernel arguments out of scratch memory.
struct View {
  const int32_t* text;
  const int32_t* pl0;
  const int32_t* pl1;
  const int32_t* pl2;
  const NgramSlot* ht0;
  const NgramSlot* ht1;
  const NgramSlot* ht2;
  uint32_t mask;
};
__device__ __forceinline__ View view_of(const ProposeArgs& a, int act, uint32_t mask) {
  const bool z = act == 0;
  View v;
  v.mask = mask;
  v.text = z ? a.idx[0].text : a.idx[1].text;
  v.pl0 = z ? a.idx[0].pl[0] : a.idx[1].pl[0];
  v.pl1 = z ? a.idx[0].pl[1] : a.idx[1].pl[1];
  v.pl2 = z ? a.idx[0].pl[2] : a.idx[1].pl[2];
  v.ht0 = z ? a.idx[0].ht[0] : a.idx[1].ht[0];
  v.ht1 = z ? a.idx[0].ht[1] : a.idx[1].ht[1];
  v.ht2 = z ? a.idx[0].ht[2] : a.idx[1].ht[2];
  return v;
}

// Probe of the (G+2)-gram that ends the context: its group in the position list, minus the
// prefix of occurrences in documents evicted since the snapshot.
template <int G>
__device__ void probe_ngram(const View ib, const int* tail, int Lcap, long long dead_below,
                            int* off_out, int* live_out) {
  constexpr int ng = G + 2;
  int off = 0, live = 0;
  if (ng <= Lcap) {
    int key[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) key[x] = x < ng ? tail[ng - 1 - x] : -1;
    const NgramSlot* ht = G == 0 ? ib.ht0 : (G == 1 ? ib.ht1 : ib.ht2);
    const int32_t* plist = G == 0 ? ib.pl0 : (G == 1 ? ib.pl1 : ib.pl2);
    uint32_t h = ngram_hash4(key, ng) & ib.mask;
    int cnt = 0;
    for (;;) {
      const NgramSlot s = ht[h];
      if (s.owner == 0) break;
      bool eq = true;
#pragma unroll
      for (int x = 0; x < ng; ++x) eq = eq && s.key[x] == key[x];
      if (eq) {
        off = s.off;
        cnt = s.cnt;
        break;
      }
      h = (h + 1) & ib.mask;
    }
    int skip = 0;
    if (cnt > 0 && dead_below > 0) {
      const int32_t* pl = plist + off;
      int lo = 0, hi = cnt;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((long long)pl[mid] < dead_below) lo = mid + 1;
        else hi = mid;
      }
      skip = lo;
    }
    off += skip;
    live = cnt - skip;
  }
  *off_out = off;
  *live_out = live;
}

// Backward extension of a 4-gram occurrence starting at snapshot position i: the match length
// (>= 4) against the tail, at most `cap`.  The preceding tokens are fetched eight at a time, all
// eight loads in flight, so a match of length l costs about (l - 4) / 8 + 1 round trips.
__device__ __forceinline__ int extend4(const int32_t* text, const int* tail, int i, int cap) {
  int m = 4;
  for (int base = 0; base < cap - 4; base += 8) {
    int c[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int o = base + q;
      c[q] = (o < cap - 4 && i - 1 - o >= 0) ? text[i - 1 - o] : -2;
    }
    bool stop = false;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (!stop) {
        const int ti = 4 + base + q < kMaxD ? 4 + base + q : kMaxD - 1;
        if (c[q] >= 0 && c[q] == tail[ti]) ++m;
        else stop = true;
      }
    }
    if (stop) break;
  }
  return m;
}

// Address of the corpus token at logical position q: snapshot text below snap_end, else ring slot
// `slot` (q mod ring capacity, which the caller steps along instead of dividing each time).  A
// choice of pointer, so that the load itself is unconditional.
__device__ __forceinline__ const int32_t* corpus_ptr(const ProposeArgs& a, const int32_t* text,
                                                     long long snap_start, long long snap_n,
                                                     long long q, int slot) {
  const long long s = q - snap_start;
  return (s >= 0 && s < snap_n) ? text + s : a.ring + slot;
}

__device__ __forceinline__ int ring_next(int r, int cap) { return r + 1 == cap ? 0 : r + 1; }
__device__ __forceinline__ int ring_prev(int r, int cap) { return r == 0 ? cap - 1 : r - 1; }

constexpr int kDeltaLoads = 8;  // 64-position chunks per round of the delta scan

template <int U>
__device__ __forceinline__ uint64_t pick_mask(const uint64_t (&h)[U], int u) {
  uint64_t x = h[0];
#pragma unroll
  for (int i = 1; i < U; ++i) x = u == i ? h[i] : x;
  return x;
}

// One wavefront scans the delta end positions [x0, x1), x1 < delta end (so every position has a
// next token inside the delta), in position order.  Lanes read consecutive ring slots.  A
// position is an occurrence of the tail's last two tokens when its own token is tail[0] and the
// one before it (not before dlo) is tail[1]: two compares per chunk, whose ballots are combined
// with a one-bit shift, select them.  Only those lanes extend backwards, and an occurrence
// followed by a separator is dropped.  For every chunk that holds a candidate, f(x, x, m) gets
// each lane's position (twice: as the record coordinate and as the position) and match length
// (0 where none); f returns false to stop the scan.
template <typename F>
__device__ __forceinline__ void delta_scan_wave(const ProposeArgs& a, long long dlo, long long x0,
                                                long long x1, int Lcap, const int* tail,
                                                int lane, F&& f) {
  const int t0 = tail[0], t1 = tail[1];
  if (t1 < 0 || x0 >= x1) return;  // a negative tail token matches no corpus token
  const int cap = (int)a.ring_cap;
  long long x = x0;
  int r = (int)(x0 % a.ring_cap);
  while (x < x1) {
    // a run of ring slots without wrap-around: positions x .. x+len-1 in slots r .. r+len-1
    const long long room = (long long)(cap - r);
    const int len = (int)(x1 - x < room ? x1 - x : room);
    uint64_t carry = 0;  // position x - 1 holds tail[1]
    if (x - 1 >= dlo) carry = a.ring[ring_prev(r, cap)] == t1 ? 1ull : 0ull;
    const int32_t* p = a.ring + r;
    for (int o = 0; o < len; o += 64 * kDeltaLoads) {
      int v[kDeltaLoads];
      if (o + 64 * kDeltaLoads <= len) {
#pragma unroll
        for (int u = 0; u < kDeltaLoads; ++u) v[u] = p[o + 64 * u + lane];
      } else {
#pragma unroll
        for (int u = 0; u < kDeltaLoads; ++u) {
          const int i = o + 64 * u + lane;
          v[u] = i < len ? p[i] : -1;
        }
      }
      uint64_t hit[kDeltaLoads];
      uint64_t any = 0;
#pragma unroll
      for (int u = 0; u < kDeltaLoads; ++u) {
        const uint64_t b0 = __ballot(v[u] == t0), b1 = __ballot(v[u] == t1);
        hit[u] = b0 & ((b1 << 1) | carry);
        carry = b1 >> 63;
        any |= hit[u];
      }
      if (!any) continue;
      for (int u = 0; u < kDeltaLoads; ++u) {
        const uint64_t hm = pick_mask(hit, u);
        if (!hm) continue;
        const int i = o + 64 * u + lane;  // this lane's offset in the run
        const long long xp = x + i;
        int m = 0;
        if ((hm >> lane) & 1) {
          const int s = r + i;
          if (a.ring[ring_next(s, cap)] >= 0) {
            m = 2;
            int rb = ring_prev(s, cap);
            while (m < Lcap && xp - m >= dlo) {
              rb = ring_prev(rb, cap);
              const int c = a.ring[rb];
              if (c < 0 || c != tail[m]) break;
              ++m;
            }
          }
        }
        if (!f(xp, xp, m)) return;
      }
    }
    x += len;
    r = 0;  // a run ends at x1 or at the last slot
  }
}

constexpr int kListRound = 4;    // tokens compared per round trip when extending listed entries
constexpr int kListBatches = 4;  // 64-entry batches whose first loads are issued together

// The same occurrences from the per-call pair index: entries [i0, i1) of the request's group
// list hold, in position order, the offsets from dlo of the delta positions that end with the
// tail's last two tokens and are followed by a real token.  All 64 lanes extend an entry each:
// the next token (where most occurrences of a frequent pair end), then kListRound tokens per
// round trip.  The list entries and next tokens of kListBatches batches are loaded together,
// so a wavefront waits for two round trips per kListBatches batches plus the rounds of its
// longest matches.  f(i, x, m) gets, batch by batch in order, each lane's entry index,
// position and match length (0 past i1).
template <typename F>
__device__ __forceinline__ void delta_list_wave(const ProposeArgs& a, long long dlo, long long i0,
                                                long long i1, int Lcap, const int* tail,
                                                int lane, F&& f) {
  const int cap = (int)a.ring_cap;
  const int dslot = (int)(dlo % a.ring_cap);
  for (long long e0 = i0; e0 < i1; e0 += 64 * kListBatches) {
    uint32_t o[kListBatches];
#pragma unroll
    for (int u = 0; u < kListBatches; ++u) {
      const long long i = e0 + 64 * u + lane;
      o[u] = i < i1 ? a.pair_list[i] : 0u;
    }
    int sl[kListBatches], lim[kListBatches], nxt[kListBatches];
#pragma unroll
    for (int u = 0; u < kListBatches; ++u) {
      const long long i = e0 + 64 * u + lane;
      const long long x = dlo + (long long)o[u];
      int sx = dslot + (int)o[u];
      if (sx >= cap) sx -= cap;
      sl[u] = sx;
      // length m extends while m < Lcap and position x - m is still in the delta
      lim[u] = i >= i1 ? 0 : ((long long)Lcap <= x - dlo ? Lcap : (int)(x - dlo) + 1);
      int q = sx - 2;
      if (q < 0) q += cap;
      nxt[u] = 2 < lim[u] ? a.ring[q] : -1;
    }
#pragma unroll
    for (int u = 0; u < kListBatches; ++u) {
      if (e0 + 64 * u >= i1) return;  // uniform: no entry left
      const long long i = e0 + 64 * u + lane;
      int m = 0;
      if (i < i1) {
        m = nxt[u] >= 0 && nxt[u] == tail[2] ? 3 : 2;
        while (m > 2 && m < lim[u]) {
          int v[kListRound];
#pragma unroll
          for (int j = 0; j < kListRound; ++j) {
            int q = sl[u] - m - j;  // m + j < lim <= the delta's length <= cap: one wrap at most
            if (q < 0) q += cap;
            v[j] = m + j < lim[u] ? a.ring[q] : -2;
          }
          int run = 0;
          bool stop = false;
#pragma unroll
          for (int j = 0; j < kListRound; ++j) {
            const int tj = m + j < kMaxD ? m + j : kMaxD - 1;
            stop = stop || v[j] < 0 || v[j] != tail[tj];
            run += stop ? 0 : 1;
          }
          m += run;
          if (stop) break;
        }
      }
      if (!f(i, dlo + (long long)o[u], m)) return;
    }
  }
}

// Depth-wise vote of one candidate held by one wavefront: lane l owns sites l and l+64, whose
// continuation windows are w0 / w1 (-1 past the end of a continuation).  Writes the tokens to
// out[] and returns the count and the sum of per-depth counts.  cmin is the smallest
// count the stop rule keeps (0 when there is no stop rule).
// State of one candidate's depth-wise vote, kept by its wavefront.
struct VoteState {
  bool al0, al1;  // this lane's two sites still on the voted path
  bool done;
  bool site0;     // site 0 (lane 0, first half) is still on the voted path
  int nout;       // tokens voted so far
  int snum;       // their counts summed: at most k * M, so every product below fits 32 bits
  int tokv;       // lane i collects the i-th voted token
};

// One depth of the vote: x0 and x1 are this lane's two sites' tokens at this depth.
__device__ __forceinline__ void vote_depth(VoteState& v, int x0, int x1, int cmin, int* hk, int* hc,
                                           int lane) {
  bool& al0 = v.al0;
  bool& al1 = v.al1;
  bool& done = v.done;
  bool& site0 = v.site0;
  int& nout = v.nout;
  int& snum = v.snum;
  int& tokv = v.tokv;
  const int tk0 = al0 ? x0 : -1, tk1 = al1 ? x1 : -1;
  const uint64_t v0 = __ballot(tk0 >= 0), v1 = __ballot(tk1 >= 0);
  // site 0's token at this depth does not depend on the votes so far
  const int s0tok = __builtin_amdgcn_readfirstlane(x0);
  int c = 0, w = -1;
  if ((v0 | v1) == 0) {
    done = true;
  } else {
    // the reference is an alive site's token: site 0's while it stays on the voted path,
    // else the first alive site's; when every alive site agrees with it the token wins
    // with all their votes
    int first;
    if (site0 && s0tok >= 0) {
      first = s0tok;
    } else {
      const int fl = v0 ? __builtin_ctzll(v0) : __builtin_ctzll(v1);
      first = v0 ? __builtin_amdgcn_readlane(tk0, fl) : __builtin_amdgcn_readlane(tk1, fl);
    }
    const uint64_t f0 = __ballot(tk0 == first), f1 = __ballot(tk1 == first);
    const int nalive = __popcll(v0) + __popcll(v1);
    const int cf = __popcll(f0) + __popcll(f1);
    if (cf == nalive) {
      c = nalive;
      w = first;
    } else if (2 * cf > nalive) {
      // a strict majority: no other token can reach its count
      c = cf;
      w = first;
    } else if (nalive <= kSmallVote) {
      // few alive sites: one ballot pair per distinct token, until the best count exceeds
      // every vote not yet counted
      uint64_t key = ((uint64_t)cf << 32) | (uint32_t)(0x7FFFFFFF - first);
      uint64_t r0 = v0 & ~f0, rr1 = v1 & ~f1;
      int rest = nalive - cf;
      while ((r0 | rr1) && (int)(key >> 32) <= rest) {
        const int tok = r0 ? __builtin_amdgcn_readlane(tk0, __builtin_ctzll(r0))
                           : __builtin_amdgcn_readlane(tk1, __builtin_ctzll(rr1));
        const uint64_t e0 = __ballot(tk0 == tok), e1 = __ballot(tk1 == tok);
        const uint64_t k = ((uint64_t)(__popcll(e0) + __popcll(e1)) << 32) |
                           (uint32_t)(0x7FFFFFFF - tok);
        key = k > key ? k : key;
        r0 &= ~e0;
        rr1 &= ~e1;
        rest -= __popcll(e0) + __popcll(e1);
      }
      c = (int)(key >> 32);
      w = 0x7FFFFFFF - (int)(uint32_t)(key & 0xFFFFFFFFu);
    } else {
      // many alive sites: counts in an LDS hash, then max count and smallest token
      for (int x = lane; x < kVoteSlots; x += 64) {
        hk[x] = -1;
        hc[x] = 0;
      }
      wave_sync();
      int sl0 = -1, sl1 = -1;
      if (tk0 >= 0) sl0 = vote_insert(hk, hc, tk0);
      if (tk1 >= 0) sl1 = vote_insert(hk, hc, tk1);
      wave_sync();
      const int cnt0 = sl0 >= 0 ? hc[sl0] : 0, cnt1 = sl1 >= 0 ? hc[sl1] : 0;
      if (__ballot(tk0 >= (1 << 24) || tk1 >= (1 << 24)) == 0) {
        // tokens below 2^24: count and token packed in one key, one reduction
        const uint32_t k0 = sl0 >= 0 ? ((uint32_t)cnt0 << 24) | (uint32_t)(0xFFFFFF - tk0) : 0u;
        const uint32_t k1 = sl1 >= 0 ? ((uint32_t)cnt1 << 24) | (uint32_t)(0xFFFFFF - tk1) : 0u;
        const uint32_t key = wave_max_u32(k0 > k1 ? k0 : k1);
        c = (int)(key >> 24);
        w = 0xFFFFFF - (int)(key & 0xFFFFFFu);
      } else {
        c = wave_max(cnt0 > cnt1 ? cnt0 : cnt1);
        int tmin = 0x7FFFFFFF;
        if (sl0 >= 0 && cnt0 == c) tmin = tk0;
        if (sl1 >= 0 && cnt1 == c && tk1 < tmin) tmin = tk1;
        w = wave_min(tmin);
      }
      wave_sync();
    }
    if (c < cmin) {
      done = true;
    } else {
      tokv = lane == nout ? w : tokv;
      ++nout;
      snum += c;
      site0 = site0 && s0tok == w;
      al0 = tk0 == w;
      al1 = tk1 == w;
    }
  }
}

template <int KMAX>
__device__ __forceinline__ void vote_run(const int (&w0)[KMAX], const int (&w1)[KMAX], int c0,
                                         int cap, int cmin, int* hk, int* hc, int lane, int* out,
                                         int* n_out, int* snum_out) {
  VoteState v{lane < c0, lane + 64 < c0, false, true, 0, 0, -1};
#pragma unroll
  for (int d = 0; d < KMAX; ++d) {
    if (!v.done && d < cap) vote_depth(v, w0[d], w1[d], cmin, hk, hc, lane);
  }
  if (lane < v.nout) out[lane] = v.tokv;
  *n_out = v.nout;
  *snum_out = v.snum;
}


// The corpus wavefront of the fast path (live snapshot, no delta), first part, run while the
// other wavefronts stage the context: tail from global memory, the three n-gram probes, the
// heads of the three position-ordered groups into LDS, and the backward extension of the live
// 4-gram occurrences into a length histogram (lengths of the first kMaxM kept in LDS).
__device__ __forceinline__ void corpus_wave_probe(const ProposeArgs& a, const Req& r, Smem& sm,
                                                  const int32_t* row, const int32_t* smp,
                                                  int lane) {
  const int n = r.n, L = r.L, Lcap = r.Lcap, M = a.M;
  if (lane < Lcap) sm.gtail[lane] = ctx_at(row, smp, n, L - 1 - lane);
  for (int i = lane; i <= kMaxD; i += 64) sm.ghist[i] = 0;
  wave_sync();
  const View ib = view_of(a, r.act, r.ht_mask);
  const long long dead_below = r.tail_w - r.snap_start;
  if (lane == 0) probe_ngram<0>(ib, sm.gtail, Lcap, dead_below, &sm.g_off[0], &sm.g_live[0]);
  if (lane == 1) probe_ngram<1>(ib, sm.gtail, Lcap, dead_below, &sm.g_off[1], &sm.g_live[1]);
  if (lane == 2) probe_ngram<2>(ib, sm.gtail, Lcap, dead_below, &sm.g_off[2], &sm.g_live[2]);
  wave_sync();
#pragma unroll
  for (int g = 0; g < kNG; ++g) {
    const int32_t* pl = (g == 0 ? ib.pl0 : (g == 1 ? ib.pl1 : ib.pl2)) + sm.g_off[g];
    const int ns = sm.g_live[g] < M ? sm.g_live[g] : M;
    for (int x = lane; x < ns; x += 64) sm.gpl[g][x] = pl[x];
  }
  const int live4 = sm.g_live[2];
  if (Lcap >= 5 && live4 > 0) {
    const int32_t* pl4 = ib.pl2 + sm.g_off[2];
    for (int x = lane; x < live4; x += 64) {
      const int i = pl4[x];
      const int m = extend4(ib.text, sm.gtail, i, Lcap);
      if (x < kMaxM) {
        sm.gm4[x] = m;
        sm.gpl[2][x] = i;
      }
      if (m >= 5) atomicAdd(&sm.ghist[m], 1);
    }
  }
}

// Second part, run while the other wavefronts compute the match lengths of the context: the
// corpus ladder (lane l - 1 holds the support of length l) and the earliest sites of each level.
__device__ __forceinline__ void corpus_wave_sites(const ProposeArgs& a, const Req& r, Smem& sm,
                                                  int lane) {
  const int Lcap = r.Lcap, nb = a.nb, M = a.M;
  const long long snap_start = r.snap_start;
  wave_sync();
  // support of length v = lane + 1 (lengths up to 64 on 64 lanes): the live v-gram group for
  // v <= 4, else the extensions reaching v
  const int v = lane + 1;
  const int gh = (v >= 5 && v <= Lcap) ? sm.ghist[v] : 0;
  const int gin = wave_incl_add(gh);
  const int gsuf = __builtin_amdgcn_readlane(gin, 63) - gin + gh;
  const int sup_l = v >= 2 && v <= 4 ? sm.g_live[v - 2] : gsuf;
  const int minc = a.min_corpus > 2 ? a.min_corpus : 2;
  int prev_l = -1, prev_src = -1;
  for (int ti = 0; ti < nb; ++ti) {
    const uint64_t ok = __ballot(v >= 2 && v <= Lcap && sup_l >= ti + 1);
    const int l = ok ? 64 - __builtin_clzll(ok) : 0;
    const int sup = l ? __builtin_amdgcn_readlane(sup_l, l - 1) : 0;
    const int ci = nb + ti;
    const int src = (ti > 0 && l == prev_l) ? prev_src : ci;
    prev_l = l;
    prev_src = src;
    if (lane == 0) {
      sm.cand_len[ci] = l;
      sm.cand_sup[ci] = sup;
      sm.cand_valid[ci] = l >= minc;
      sm.cand_c0[ci] = sup < M ? sup : M;
      sm.cand_src[ci] = src;
    }
    if (l < minc || src != ci) continue;
    long long* gs = sm.gsites[ti];
    if (l <= 4) {
      const int g = l - 2;
      const int ns = sup < M ? sup : M;
      for (int x = lane; x < ns; x += 64) gs[x] = (long long)sm.gpl[g][x] + l + snap_start;
    } else {
      // the first M live 4-gram occurrences (position order) whose extension reaches l
      const int live4 = sm.g_live[2];
      const uint64_t below = lanes_below(lane);
      const View ib = view_of(a, r.act, r.ht_mask);
      const int32_t* pl4 = ib.pl2 + sm.g_off[2];
      int run = 0;
      for (int base = 0; base < live4 && run < M; base += 64) {
        const int x = base + lane;
        bool q = false;
        int i = 0;
        if (x < live4) {
          if (x < kMaxM) {
            i = sm.gpl[2][x];
            q = sm.gm4[x] >= l;
          } else {
            i = pl4[x];
            q = extend4(ib.text, sm.gtail, i, l) >= l;
          }
        }
        const uint64_t bal = __ballot(q);
        const int rk = run + __popcll(bal & below);
        if (q && rk < M) gs[rk] = (long long)i + 4 + snap_start;
        run += __popcll(bal);
      }
    }
  }
}

// Dynamic LDS of one request.  Staged: [context ints | hit positions (u16) | hit lengths (u8) |
// hit bit words]; streaming (the context stays in HBM): the same without the context.  The vote
// tables of the expansion alias the start of the region once those are dead.
constexpr int kVoteBytes = NW * 2 * kVoteSlots * 4;
// context ints, then 64 spare slots that absorb the staging stores of lanes past the row end
__host__ __device__ inline int ctx_ints(int S, int T) { return ((S + T + 4 + 3) & ~3) + 64; }
__host__ __device__ inline int ctx_spare(int S, int T) { return ctx_ints(S, T) - 64; }
// Hit-list entries: wavefront w owns the entries of its end positions [cbeg, cend), from entry
// cbeg on; J <= S + T - 1, so S + T + 64 * NW entries always suffice.
__host__ __device__ inline int hit_cap(int S, int T) { return (S + T + 64 * NW + 63) & ~63; }
__host__ __device__ inline size_t hpos_offset(bool staged, int S, int T) {
  return staged ? (size_t)4 * ctx_ints(S, T) : 0;
}
__host__ __device__ inline size_t hmb_offset(bool staged, int S, int T) {
  return hpos_offset(staged, S, T) + (size_t)2 * hit_cap(S, T);
}
// one 64-bit word of hit bits per 64 end positions
__host__ __device__ inline size_t bits_offset(bool staged, int S, int T) {
  return (hmb_offset(staged, S, T) + hit_cap(S, T) + 15) & ~(size_t)15;
}
// With a corpus, the region from hpos_offset on also holds the delta scan's occurrence records
// (after the local phase), at least kDeltaMinRecs per wavefront.
constexpr int kDeltaMinRecs = 256;
__host__ __device__ inline size_t dyn_bytes(bool staged, int S, int T, bool corpus) {
  size_t b = bits_offset(staged, S, T) + (size_t)8 * (hit_cap(S, T) / 64);
  if (b < (size_t)kVoteBytes) b = kVoteBytes;
  if (corpus) {
    const size_t need = hpos_offset(staged, S, T) + (size_t)4 * NW * kDeltaMinRecs;
    if (b < need) b = need;
  }
  return b;
}

constexpr int kScreenLoads = 16;  // 64-position words per screening group (1024 positions)

// Share of the end positions per wavefront age rank on a SIMD (oldest first), and the total share
// of wavefronts 0 .. w-1.
constexpr int kAgeWeight[4] = {22, 18, 14, 12};
__host__ __device__ constexpr int age_prefix(int w) {
  int p = 0;
  for (int r = 0; r < 4; ++r) {
    const int in_rank = w > 4 * r ? (w - 4 * r < 4 ? w - 4 * r : 4) : 0;
    p += kAgeWeight[r] * in_rank;
  }
  return p;
}
// First 64-position run of wavefront w out of nch runs shared by NWW workers (the division is by
// a compile-time total).
template <int NWW>
__device__ __forceinline__ int first_run(int nch, int w) {
  constexpr int pt = age_prefix(NWW);
  return nch * age_prefix(w) / pt;
}
constexpr uint32_t kBufferWord3 = 0x00020000;  // raw buffer resource, gfx9 format bits

__device__ __forceinline__ int lanes_before(uint64_t bal) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

// Lanes L and L+1 of acc := the low and high halves of a 64-bit ballot; L is an immediate.
// The ballot is an SGPR pair written by a VALU compare just before, and the compiler does not
// look inside inline assembly for hazards, so five wait states come first.
template <int L>
__device__ __forceinline__ uint32_t put_ballot(uint32_t acc, uint64_t v) {
  asm volatile("s_nop 4\n\tv_writelane_b32 %0, %1, %3\n\tv_writelane_b32 %0, %2, %4"
               : "+v"(acc)
               : "s"((uint32_t)v), "s"((uint32_t)(v >> 32)), "i"(L), "i"(L + 1));
  return acc;
}

// f(integral_constant<int, I>) for I = I0 .. N-1, unrolled at compile time (so that lane and
// register indices are immediates).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Local step 1 for one wavefront's chunk [cbeg, cend) of end positions.  The row part is read
// with bounds-checked buffer loads (every load of a lane in flight; lanes on consecutive
// positions, so each load instruction is one coalesced 256-byte run) and staged in LDS when
// STAGED.  For every 64 positions one ballot is kept as a bit word: the end positions whose
// token is the last context token t0 (match length >= 1).  Word i covers positions
// cbeg + 64 i ...; the end positions among the sampled ids (at most T - 1, after every row
// position) go to *s1, based at max(cbeg, n).  Returns the number of row words.
template <bool STAGED>
__device__ __forceinline__ int stage_screen(int* ctxs, int spare, uint64_t* b1w,
                                            const int32_t* row, const int32_t* smp, int n,
                                            int cbeg, int cend, int t0, int lane, uint64_t* s1) {
  const int rend = __builtin_amdgcn_readfirstlane(cend < n ? cend : n);
  // t0 arrives by a scalar load, which shares a counter with the LDS stores below: settle it
  // once here so that no store in the loop has to drain that counter
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  int nw = 0;
  if (rend > cbeg) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)row, (short)0, rend * 4, kBufferWord3);
    for (int g0 = cbeg; g0 < rend; g0 += 64 * kScreenLoads) {
      int v[kScreenLoads];
      const int vo = (g0 + lane) * 4;
#pragma unroll
      for (int i = 0; i < kScreenLoads; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, vo + 256 * i, 0, 0);
      const int ne = (rend - g0 + 63) >> 6 < kScreenLoads ? (rend - g0 + 63) >> 6 : kScreenLoads;
      const int nfull = (rend - g0) >> 6;  // elements whose 64 positions all lie below rend
      uint32_t a1 = 0;
      static_for<0, kScreenLoads>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if (i < ne) {
          const int x = g0 + 64 * i + lane;
          uint64_t w1;
          if (i < nfull) {
            if (STAGED) ctxs[x] = v[i];
            w1 = __ballot(v[i] == t0);
          } else {
            const int rem = rend - g0 - 64 * i;  // 1..63
            if (STAGED) ctxs[x < rend ? x : spare + lane] = v[i];
            w1 = __ballot(v[i] == t0) & ((1ull << rem) - 1ull);
          }
          a1 = put_ballot<(2 * i) & 62>(a1, w1);
        }
      });
      if (lane < 2 * ne) reinterpret_cast<uint32_t*>(b1w + nw)[lane] = a1;
      nw += ne;
    }
  }
  *s1 = 0;
  if (cend > n) {
    const int x = (cbeg > n ? cbeg : n) + lane;
    const bool in = x < cend;
    const int v = in ? smp[x - n] : -1;
    *s1 = __ballot(in && v == t0);
  }
  return nw;
}

// Positions of the set bits of nw words (word i based at base0 + 64 i) followed by one extra
// word `extra` based at xbase, in order, into out[]; returns their number.  Every lane of the
// wavefront takes part, on a 16-bit quarter of a word each, so that a lane walks at most 16 bits.
__device__ __forceinline__ int bits_to_list(const uint64_t* w, int nw, uint64_t extra, int xbase,
                                            int base0, uint16_t* out, int lane) {
  int cnt = 0;
  const int nq = 4 * (nw + 1);
  for (int q0 = 0; q0 < nq; q0 += 64) {
    const int q = q0 + lane;
    const int wi = q >> 2, part = q & 3;
    const uint64_t wd = wi < nw ? w[wi] : (wi == nw ? extra : 0ull);
    uint32_t piece = (uint32_t)(wd >> (16 * part)) & 0xFFFFu;
    const int base = (wi < nw ? base0 + 64 * wi : xbase) + 16 * part;
    const int c = __popc(piece);
    const int incl = wave_incl_add(c);
    int at = cnt + incl - c;
    while (piece) {
      out[at++] = (uint16_t)(base + __builtin_ctz(piece));
      piece &= piece - 1;
    }
    cnt += __builtin_amdgcn_readlane(incl, 63);
  }
  return cnt;
}

// Local step 2: the backward match length of every listed hit (its last token already matches,
// so the length is at least 1), one hit per lane: the previous token decides whether the match
// goes on; if it does, the tail is compared four offsets per round.  Lengths go to hmb[] and
// the wavefront's histogram.
constexpr int kTailRegs = 24;  // tail offsets 2 .. 25 held in registers during the extension
template <bool STAGED>
__device__ __forceinline__ void extend_hits(const int* ctxs, const uint16_t* hpos, uint8_t* hmb,
                                            int nhit, const int* tail, int D, int* whist,
                                            const int32_t* row, const int32_t* smp, int n,
                                            int lane) {
  const int t1 = D >= 2 ? tail[1] : -1;
  const bool short_d = D <= 2 + kTailRegs;
  int tq[kTailRegs];
#pragma unroll
  for (int x = 0; x < kTailRegs; ++x) tq[x] = (short_d && 2 + x < D) ? tail[2 + x] : -1;
  for (int e0 = 0; e0 < nhit; e0 += 64) {
    const int e = e0 + lane;
    const bool ok = e < nhit;
    const int j = ok ? hpos[e] : 0;
    const int lim = D < j + 1 ? D : j + 1;
    int m = 1;
    if (ok && lim >= 2) {
      const int c1 = STAGED ? ctxs[j - 1] : ctx_at(row, smp, n, j - 1);
      if (c1 == t1 && short_d) {
        // offsets 2 .. 25 in six rounds of four, compared with tail values held in registers
        m = 2;
        bool go = true;
#pragma unroll
        for (int r = 0; r < kTailRegs / 4; ++r) {
          if (go && 2 + 4 * r < lim) {
            int c[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int o = 2 + 4 * r + q;
              c[q] = STAGED ? ctxs[o < lim ? j - o : 0] : ctx_at(row, smp, n, o < lim ? j - o : 0);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              go = go && 2 + 4 * r + q < lim && c[q] == tq[4 * r + q];
              m += go ? 1 : 0;
            }
          }
        }
      } else if (c1 == t1) {
        m = 2;
        for (int o0 = 2; o0 < lim; o0 += 4) {
          int c[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int at = o0 + q < lim ? j - o0 - q : 0;
            c[q] = STAGED ? ctxs[at] : ctx_at(row, smp, n, at);
          }
          bool stop = false;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (!stop) {
              if (o0 + q < lim && c[q] == tail[o0 + q]) ++m;
              else stop = true;
            }
          }
          if (stop) break;
        }
      }
    }
    if (ok) hmb[e] = (uint8_t)m;
    const uint64_t one = __ballot(ok && m == 1);
    if (ok && m > 1) atomicAdd(&whist[m], 1);
    if (lane == 0 && one) atomicAdd(&whist[1], __popcll(one));
  }
}

template <int KMAX, bool STAGED>
__global__ __launch_bounds__(NT) void propose_kernel(ProposeArgs a) {
  extern __shared__ int4 dyn4[];
  unsigned char* dyn = reinterpret_cast<unsigned char*>(dyn4);
  int* ctxs = reinterpret_cast<int*>(dyn);  // the context (STAGED only)
  uint16_t* hpos_all = reinterpret_cast<uint16_t*>(dyn + hpos_offset(STAGED, a.S, a.T));
  uint8_t* hmb_all = dyn + hmb_offset(STAGED, a.S, a.T);
  uint64_t* bits_all = reinterpret_cast<uint64_t*>(dyn + bits_offset(STAGED, a.S, a.T));
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform (SGPR)
  const int b = blockIdx.x;
  const int32_t* row = a.tok + (int64_t)b * a.S;
  const int32_t* smp = a.samp + (int64_t)b * a.T;
  const int D = a.D, nb = a.nb, M = a.M;

  Req r;
  {
    int n = a.ntns[b];
    n = n < 0 ? 0 : (n > a.S ? a.S : n);
    int t = 0;
    while (t < a.T && smp[t] >= 0) ++t;
    r.n = n;
    r.t = t;
    r.L = n + t;
    r.J = r.L > 0 ? r.L - 1 : 0;
    r.Lcap = D < r.L ? D : r.L;
    r.has = a.ctl != nullptr;
    r.act = -1;
    r.fast = false;
    r.delta = false;
    r.snap_start = r.snap_n = r.tail_w = r.delta_lo = r.delta_hi = 0;
    r.ht_mask = 0;
    bool delta = false;
    if (r.has) {
      const Ctl c = *a.ctl;  // one round of loads for the whole control block
      r.act = c.active;
      r.tail_w = c.tail;
      r.delta_hi = c.head;
      if (r.act >= 0) {
        r.ht_mask = r.act == 0 ? c.ht_mask[0] : c.ht_mask[1];
        r.snap_start = r.act == 0 ? c.snap_start[0] : c.snap_start[1];
        const long long se = r.act == 0 ? c.snap_end[0] : c.snap_end[1];
        r.snap_n = se - r.snap_start;
        r.delta_lo = se > r.tail_w ? se : r.tail_w;
      } else {
        r.delta_lo = r.tail_w;
      }
      delta = r.delta_hi - r.delta_lo > 1;
      r.delta = delta;
      r.fast = r.act >= 0 && r.snap_n > 0 && r.Lcap >= 2;
    }
  }
  const int n = r.n, t = r.t, L = r.L, Lcap = r.Lcap, J = r.J;
  int32_t* drow = a.draft + (int64_t)b * a.k;
  if (t == 0) {
    for (int i = tid; i < a.k; i += NT) drow[i] = -1;
    if (tid == 0) {
      a.nvalid[b] = 0;
      a.pick[b] = -1;
    }
    return;
  }
  const bool fast = r.fast;
  for (int i = tid; i < NW * (kMaxD + 1); i += NT) (&sm.whist[0][0])[i] = 0;
  if (!fast && tid < 2 * kMaxNB) sm.cand_valid[tid] = 0;
  if (tid == 0) sm.wbar = 0;
  __syncthreads();
  // the tail (read from the extension on) and the sampled ids of the staged context: loaded now,
  // stored to LDS once wavefront 0 has screened its positions, so that the round trip overlaps
  // its screen
  const int tailv = tid < Lcap ? ctx_at(row, smp, n, L - 1 - tid) : 0;
  const int sampv = (STAGED && tid < t) ? smp[tid] : 0;

  // ---------------------------------------------------------------- 1. local match
  // Wavefront w < NWW owns end positions [cbeg, cend): it stages them (STAGED) and marks the
  // ones whose token equals the last context token.  The ranges are runs of 64 positions in
  // wavefront order, sized by the wavefront's age on its SIMD (wavefront w is the (w / 4)-th
  // on SIMD w % 4): a SIMD issues for its oldest ready wavefront first, so its younger ones
  // get fewer positions and every worker reaches the barriers at about the same time.  In the
  // fast path the corpus wavefront probes the corpus and derives its ladder and sites
  // meanwhile, through every local phase (the workers synchronise among themselves only).
  const int NWW = fast ? NW - 1 : NW;
  const bool worker = wid < NWW;
  int cbeg = J, cend = J;
  if (worker) {
    const int nch = (J + 63) >> 6;
    cbeg = 64 * (fast ? first_run<NW - 1>(nch, wid) : first_run<NW>(nch, wid));
    cend = wid + 1 == NWW ? J
                          : 64 * (fast ? first_run<NW - 1>(nch, wid + 1) : first_run<NW>(nch, wid + 1));
    cbeg = cbeg < J ? cbeg : J;
    cend = cend < J ? cend : J;
  }
  if (fast && wid == GW) {
    corpus_wave_probe(a, r, sm, row, smp, lane);
    if (!r.delta) corpus_wave_sites(a, r, sm, lane);
  } else {
    uint16_t* hpos = hpos_all + cbeg;
    uint8_t* hmb = hmb_all + cbeg;
    uint64_t* b1w = bits_all + (cbeg >> 6);
    uint64_t s1 = 0;
    const int sbase = cbeg > n ? cbeg : n;
    const int nw = stage_screen<STAGED>(ctxs, ctx_spare(a.S, a.T), b1w, row, smp, n, cbeg, cend,
                                        smp[t - 1], lane, &s1);
    if (tid < Lcap) sm.tail[tid] = tailv;
    if (STAGED && tid < t) ctxs[n + tid] = sampv;
    if (fast) worker_barrier(&sm.wbar, NWW, lane);
    else __syncthreads();

    // match lengths of the hits, listed in order
    const int nhit = bits_to_list(b1w, nw, s1, sbase, cbeg, hpos, lane);
    wave_sync();
    extend_hits<STAGED>(ctxs, hpos, hmb, nhit, sm.tail, D, sm.whist[wid], row, smp, n, lane);
    wave_sync();
    {
      // this wavefront's suffix sums: wsuf[w][v] = its positions with length >= v, for
      // v = lane + 1 (lengths 1 .. 64 on 64 lanes)
      const int h = lane + 1 <= D ? sm.whist[wid][lane + 1] : 0;
      const int incl = wave_incl_add(h);
      sm.wsuf[wid][lane + 1] = __builtin_amdgcn_readlane(incl, 63) - incl + h;
    }
    if (fast) worker_barrier(&sm.wbar, 2 * NWW, lane);
    else __syncthreads();

    // ladder and this wavefront's site offsets: every worker wavefront derives them from the
    // per-wavefront suffix sums (lane v - 1 of cg = positions with length >= v); wavefront 0 also
    // records the candidates.  Then the earliest sites of every distinct local level, in one
    // ordered pass over the hit list.
    int cg = 0;
    for (int w = 0; w < NWW; ++w) cg += sm.wsuf[w][lane + 1];
    const int maxl = D < J ? D : J;
    const int mins = a.min_self > 1 ? a.min_self : 1;
    int lv[kMaxNB], pre[kMaxNB], run[kMaxNB];
    bool act[kMaxNB];
    bool any = false;
    int prev_l = -1, prev_src = -1;
#pragma unroll
    for (int ti = 0; ti < kMaxNB; ++ti) {
      act[ti] = false;
      lv[ti] = 0;
      pre[ti] = 0;
      run[ti] = 0;
      if (ti < nb) {
        const uint64_t ok = __ballot(lane + 1 <= maxl && cg >= ti + 1);
        const int l = ok ? 64 - __builtin_clzll(ok) : 0;
        const int sup = l ? __builtin_amdgcn_readlane(cg, l - 1) : 0;
        const int src = (ti > 0 && l == prev_l) ? prev_src : ti;
        prev_l = l;
        prev_src = src;
        if (wid == 0 && lane == 0) {
          sm.cand_len[ti] = l;
          sm.cand_sup[ti] = sup;
          sm.cand_valid[ti] = l >= mins;
          sm.cand_c0[ti] = sup < M ? sup : M;
          sm.cand_src[ti] = src;
        }
        const int c = (l >= 1 && lane < NWW) ? sm.wsuf[lane][l] : 0;
        const int x = wave_incl_add(c);
        const int mypre = __builtin_amdgcn_readlane(x - c, wid);
        act[ti] = l >= mins && src == ti && mypre < M;
        lv[ti] = l;
        pre[ti] = mypre;
        any = any || act[ti];
      }
    }
    for (int e0 = 0; any && e0 < nhit; e0 += 64) {
      const int e = e0 + lane;
      const int j = e < nhit ? hpos[e] : 0;
      const int m = e < nhit ? hmb[e] : 0;
      any = false;
#pragma unroll
      for (int ti = 0; ti < kMaxNB; ++ti) {
        if (act[ti]) {
          const bool q = m >= lv[ti];
          const uint64_t bal = __ballot(q);
          const int rk = pre[ti] + run[ti] + lanes_before(bal);
          if (q && rk < M) sm.lsites[ti][rk] = j + 1;
          run[ti] += __popcll(bal);
          act[ti] = pre[ti] + run[ti] < M;
          any = any || act[ti];
        }
      }
    }
  }

  // ---------------------------------------------------------------- 2. global (general path)
  if (r.has && (!fast || r.delta) && Lcap >= 2) {
    // With a live snapshot and a delta, the corpus wavefront has probed the snapshot beside the
    // local phase (its results stand); the workers may use their histograms until here.
    if (fast) __syncthreads();
    if (tid <= kMaxD) {
      if (!fast) sm.ghist[tid] = 0;
      sm.dhist[tid] = 0;
    }
    for (int i = tid; i < NW * (kMaxD + 1); i += NT) (&sm.whist[0][0])[i] = 0;
    __syncthreads();
    const int act = r.act;
    const long long snap_start = r.snap_start;
    const long long dead_below = r.tail_w - snap_start;
    const View ib = view_of(a, act >= 0 ? act : 0, r.ht_mask);
    if (tid == 0) {
      sm.plp[0] = ib.pl0;
      sm.plp[1] = ib.pl1;
      sm.plp[2] = ib.pl2;
    }
    if (fast) {
      // probed already
    } else if (act >= 0 && r.snap_n > 0) {
      if (tid == 0) probe_ngram<0>(ib, sm.tail, Lcap, dead_below, &sm.g_off[0], &sm.g_live[0]);
      if (tid == 1) probe_ngram<1>(ib, sm.tail, Lcap, dead_below, &sm.g_off[1], &sm.g_live[1]);
      if (tid == 2) probe_ngram<2>(ib, sm.tail, Lcap, dead_below, &sm.g_off[2], &sm.g_live[2]);
    } else if (tid < kNG) {
      sm.g_off[tid] = 0;
      sm.g_live[tid] = 0;
    }
    __syncthreads();
    const int live4 = sm.g_live[2];
    if (!fast && act >= 0 && Lcap >= 5 && live4 > 0) {
      const int32_t* pl4 = ib.pl2 + sm.g_off[2];
      for (int x = tid; x < live4; x += NT) {
        const int m = extend4(ib.text, sm.tail, pl4[x], Lcap);
        if (m >= 5) atomicAdd(&sm.ghist[m], 1);
      }
    }
    // delta: documents appended since the live snapshot.  With the per-call pair index,
    // wavefront w owns entries [sb, se) of the request's group list; without it, the end
    // positions [sb, se), scanned by brute force.  It keeps its occurrences of length >= 2 in
    // LDS, in position order (coordinate offset from sb << 6 | length - 2; the context hit
    // lists are dead by now), at most H of them, plus a length histogram.
    const long long dlo = r.delta_lo, dhi = r.delta_hi;
    const bool has_delta = dhi - dlo > 1;
    const bool listed = has_delta && a.pair_group != nullptr;
    long long sb, se;
    if (listed) {
      const int g = a.pair_group[b];
      const long long i0 = g >= 0 ? a.pair_base[g] : 0;
      const long long i1 = g >= 0 ? i0 + a.pair_tot[g] : 0;
      const long long per = ((i1 - i0 + NW - 1) / NW + 63) / 64 * 64;
      sb = i0 + (long long)wid * per < i1 ? i0 + (long long)wid * per : i1;
      se = sb + per < i1 ? sb + per : i1;
    } else {
      const long long dseg = has_delta ? ((dhi - 1 - dlo + NW - 1) / NW + 63) / 64 * 64 : 0;
      sb = dlo + (long long)wid * dseg;
      se = has_delta ? (sb + dseg < dhi - 1 ? sb + dseg : dhi - 1) : sb;
    }
    const size_t dbase = hpos_offset(STAGED, a.S, a.T);
    const int H = (int)((dyn_bytes(STAGED, a.S, a.T, true) - dbase) / (4 * NW));
    uint32_t* recs = reinterpret_cast<uint32_t*>(dyn + dbase) + wid * H;
    int nrec = 0;
    if (has_delta) {
      int* wh = sm.whist[wid];
      auto keep = [&](long long u, long long, int m) {
        const bool q = m >= 2;
        const uint64_t bal = __ballot(q);
        if (bal) {
          const int rk = nrec + lanes_before(bal);
          if (q && rk < H) recs[rk] = ((uint32_t)(u - sb) << 6) | (uint32_t)(m - 2);
          // length 2 (most occurrences of a frequent pair) counted from one ballot, not with
          // one conflicting LDS atomic per lane
          const uint64_t two = __ballot(m == 2);
          if (m > 2) atomicAdd(&wh[m], 1);
          if (lane == 0 && two) atomicAdd(&wh[2], __popcll(two));
          nrec += __popcll(bal);
        }
        return true;
      };
      if (listed) delta_list_wave(a, dlo, sb, se, Lcap, sm.tail, lane, keep);
      else delta_scan_wave(a, dlo, sb, se, Lcap, sm.tail, lane, keep);
      wave_sync();
      // this wavefront's suffix sums: wsuf[w][v] = its occurrences of length >= v, v = lane + 1
      const int h = lane + 1 <= Lcap ? wh[lane + 1] : 0;
      const int incl = wave_incl_add(h);
      sm.wsuf[wid][lane + 1] = __builtin_amdgcn_readlane(incl, 63) - incl + h;
    }
    __syncthreads();
    if (has_delta && wid == 0) {
      int sum = 0;
      for (int w = 0; w < NW; ++w) sum += sm.wsuf[w][lane + 1];
      sm.dhist[lane + 1] = sum;  // delta occurrences of length >= lane + 1
      wave_sync();
    }
    if (wid == 0) {
      // the corpus ladder on one wavefront: lane v - 1 holds the support of length v, the live
      // snapshot's (the v-gram group for v <= 4, else the 4-gram occurrences extending to v)
      // plus the delta's; it does not grow with v, so candidate ti takes the largest length
      // whose support is at least ti + 1
      const int v = lane + 1;
      const int gh = (v >= 5 && v <= Lcap) ? sm.ghist[v] : 0;
      const int gin = wave_incl_add(gh);
      const int gsuf = __builtin_amdgcn_readlane(gin, 63) - gin + gh;
      int snap = v >= 2 && v <= 4 ? sm.g_live[v - 2] : gsuf;
      if (act < 0) snap = 0;
      const int cnt = snap + (v <= Lcap ? sm.dhist[v] : 0);
      const int minc = a.min_corpus > 2 ? a.min_corpus : 2;
      int prev_l = -1, prev_src = -1;
      for (int ti = 0; ti < nb; ++ti) {
        const uint64_t ok = __ballot(v >= 2 && v <= Lcap && cnt >= ti + 1);
        const int l = ok ? 64 - __builtin_clzll(ok) : 0;
        const int sup = l ? __builtin_amdgcn_readlane(cnt, l - 1) : 0;
        const int ci = nb + ti;
        const int src = (ti > 0 && l == prev_l) ? prev_src : ci;
        prev_l = l;
        prev_src = src;
        if (lane == 0) {
          sm.cand_len[ci] = l;
          sm.cand_sup[ci] = sup;
          sm.cand_valid[ci] = l >= minc;
          sm.cand_c0[ci] = sup < M ? sup : M;
          sm.cand_src[ci] = src;
        }
      }
    }
    __syncthreads();
    // earliest sites: live snapshot occurrences in position order, then delta occurrences
    for (int ti = 0; ti < nb; ++ti) {
      const int ci = nb + ti;
      if (!sm.cand_valid[ci] || sm.cand_src[ci] != ci) continue;  // uniform
      const int l = sm.cand_len[ci];
      long long* gs = sm.gsites[ti];
      int nsnap = 0;
      if (act >= 0) {
        if (l <= 4) {
          const int g = l - 2;
          const int live = sm.g_live[g];
          const int32_t* pl = sm.plp[g] + sm.g_off[g];
          nsnap = live < M ? live : M;
          for (int x = tid; x < nsnap; x += NT) gs[x] = (long long)pl[x] + l + snap_start;
        } else {
          const int32_t* pl4 = ib.pl2 + sm.g_off[2];
          const int seg = (live4 + NT - 1) / NT;
          const int lo = tid * seg < live4 ? tid * seg : live4;
          const int hi = lo + seg < live4 ? lo + seg : live4;
          int c = 0;
          for (int x = lo; x < hi; ++x) c += extend4(ib.text, sm.tail, pl4[x], l) >= l;
          int total;
          int rk = block_exclusive_scan(c, sm.wsum, &total);
          if (c && rk < M) {
            for (int x = lo; x < hi && rk < M; ++x) {
              const int i = pl4[x];
              if (extend4(ib.text, sm.tail, i, l) >= l) gs[rk++] = (long long)i + 4 + snap_start;
            }
          }
          nsnap = total < M ? total : M;
        }
      }
      // delta occurrences follow every snapshot occurrence in logical order, and this
      // wavefront's follow those of the wavefronts before it: from its records, then, if it
      // found more than it kept, from a rescan past the last one kept
      if (nsnap < M && has_delta) {
        const int c = lane < NW ? sm.wsuf[lane][l] : 0;
        const int incl = wave_incl_add(c);
        int off = nsnap + __builtin_amdgcn_readlane(incl - c, wid);
        const int kept = nrec < H ? nrec : H;
        for (int base = 0; base < kept && off < M; base += 64) {
          const int e = base + lane;
          const uint32_t rc = e < kept ? recs[e] : 0u;
          const bool q = e < kept && (int)(rc & 63u) + 2 >= l;
          const uint64_t bal = __ballot(q);
          const int rk = off + lanes_before(bal);
          if (q && rk < M) {
            const long long u = sb + (long long)(rc >> 6);
            gs[rk] = (listed ? dlo + (long long)a.pair_list[u] : u) + 1;
          }
          off += __popcll(bal);
        }
        if (nrec > H && off < M) {
          const long long from = sb + (long long)(recs[H - 1] >> 6) + 1;
          auto site = [&](long long, long long x, int m) {
            const bool q = m >= l;
            const uint64_t bal = __ballot(q);
            const int rk = off + lanes_before(bal);
            if (q && rk < M) gs[rk] = x + 1;
            off += __popcll(bal);
            return off < M;
          };
          if (listed) delta_list_wave(a, dlo, from, se, Lcap, sm.tail, lane, site);
          else delta_scan_wave(a, dlo, from, se, Lcap, sm.tail, lane, site);
        }
      }
      // no barrier per candidate: each writes only its own site array, and the workgroup scan
      // of the next one ends with its own barriers
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- 3. expansion and vote
  const bool voter = wid < 2 * nb && sm.cand_valid[wid] && sm.cand_src[wid] == wid;
  int w0[KMAX], w1[KMAX];
  int c0 = 0, cap = 0;
  if (voter) {
    const int ci = wid;
    const int src = sm.cand_src[ci];
    c0 = sm.cand_c0[ci];
    cap = a.cap_of_len[sm.cand_len[ci]];
    const int s0 = lane, s1 = lane + 64;
    if (ci < nb) {
      const int* ls = sm.lsites[src];
      const int p0 = s0 < c0 ? ls[s0] : 0, p1 = s1 < c0 ? ls[s1] : 0;
#pragma unroll
      for (int d = 0; d < KMAX; ++d) {
        const bool q0 = s0 < c0 && d < cap && p0 + d < L, q1 = s1 < c0 && d < cap && p1 + d < L;
        if (STAGED) {
          w0[d] = q0 ? ctxs[p0 + d] : -1;
          w1[d] = q1 ? ctxs[p1 + d] : -1;
        } else {
          w0[d] = q0 ? ctx_at(row, smp, n, p0 + d) : -1;
          w1[d] = q1 ? ctx_at(row, smp, n, p1 + d) : -1;
        }
      }
    } else {
      const long long* gs = sm.gsites[src - nb];
      const int act = r.act;
      const int32_t* text = act == 0 ? a.idx[0].text : (act == 1 ? a.idx[1].text : nullptr);
      const long long ss = r.snap_start, sn = r.snap_n;
      const long long q0 = s0 < c0 ? gs[s0] : 0, q1 = s1 < c0 ? gs[s1] : 0;
      bool live0 = s0 < c0, live1 = s1 < c0;
      const int rcap = (int)a.ring_cap;
      int r0 = (int)(q0 % a.ring_cap), r1 = (int)(q1 % a.ring_cap);
      // every window token is loaded at once (each address is a live snapshot position or a
      // ring slot, so always in bounds); a site's window then ends at its first separator
#pragma unroll
      for (int d = 0; d < KMAX; ++d) {
        w0[d] = *corpus_ptr(a, text, ss, sn, q0 + d, r0);
        w1[d] = *corpus_ptr(a, text, ss, sn, q1 + d, r1);
        r0 = ring_next(r0, rcap);
        r1 = ring_next(r1, rcap);
      }
#pragma unroll
      for (int d = 0; d < KMAX; ++d) {
        live0 = live0 && d < cap && w0[d] >= 0;
        live1 = live1 && d < cap && w1[d] >= 0;
        w0[d] = live0 ? w0[d] : -1;
        w1[d] = live1 ? w1[d] : -1;
      }
    }
  }
  __syncthreads();  // the context and the hit lists are dead from here on: vote tables
  if (voter) {
    int nout = 0, snum = 0;
    int* hk = reinterpret_cast<int*>(dyn) + wid * (2 * kVoteSlots);
    vote_run<KMAX>(w0, w1, c0, cap, a.min_count[c0], hk, hk + kVoteSlots, lane,
                   sm.cand_out[wid], &nout, &snum);
    if (lane == 0) {
      sm.cand_n[wid] = nout;
      sm.cand_snum[wid] = snum;
    }
  }
  __syncthreads();

  // selection and output row, by wavefront 0 from registers (a candidate with the same length
  // as an earlier one of its source shares that one's sites and vote)
  if (wid != 0) return;
  const bool cv = lane < 2 * nb && sm.cand_valid[lane];
  const int csrc = cv ? sm.cand_src[lane] : 0;
  const int csn = cv ? sm.cand_snum[csrc] : 0;
  const int cc0 = cv ? sm.cand_c0[lane] : 1;
  const int clen = cv ? sm.cand_len[lane] : 0;
  const int cn = cv ? sm.cand_n[csrc] : 0;
  const uint64_t vmask = __ballot(cv);
  int win = -1;
  if (a.mode == 0) {
    const bool lv = (vmask >> 0) & 1, gv = (vmask >> nb) & 1;
    const int l0 = __builtin_amdgcn_readlane(clen, 0), g0 = __builtin_amdgcn_readlane(clen, nb);
    if (lv && (!gv || l0 >= g0)) win = 0;
    else if (gv) win = nb;
  } else {
    // scores snum / c0 compared by cross products (snum <= k * M = 4096, c0 <= M = 128)
    int bsn = 0, bc0 = 1;
    for (int i = 0; i < 2 * nb; ++i) {
      if (!((vmask >> i) & 1)) continue;
      const int sn = __builtin_amdgcn_readlane(csn, i);
      const int c0i = __builtin_amdgcn_readlane(cc0, i);
      if (win < 0 || sn * bc0 > bsn * c0i) {
        win = i;
        bsn = sn;
        bc0 = c0i;
      }
    }
  }
  const int ws = win >= 0 ? __builtin_amdgcn_readlane(csrc, win) : -1;
  const int nv = win >= 0 ? __builtin_amdgcn_readlane(cn, win) : 0;
  const int fill = a.mode == 0 ? sm.tail[0] : -1;
  const int wlen = win >= 0 ? __builtin_amdgcn_readlane(clen, win) : 0;
  for (int i = lane; i < a.k; i += 64) drow[i] = i < nv ? sm.cand_out[ws][i] : fill;
  if (lane == 0) {
    a.nvalid[b] = nv;
    a.pick[b] = win >= 0 ? (nv << 16) | ((win >= nb ? 1 : 0) << 8) | wlen : -1;
  }
}

__global__ void update_state_kernel(int B, int S, int T, int32_t* tok, const int32_t* ntns,
                                    const int32_t* samp, int32_t* nout) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int n = ntns[b];
  n = n < 0 ? 0 : (n > S ? S : n);
  int i = 0;
  while (i < T && samp[(int64_t)b * T + i] >= 0 && n + i < S) {
    tok[(int64_t)b * S + n + i] = samp[(int64_t)b * T + i];
    ++i;
  }
  nout[b] = n + i;
}

template <int KMAX>
hipError_t launch_k(const ProposeArgs& a, bool staged, size_t dyn, hipStream_t st) {
  if (staged)
    hipLaunchKernelGGL((propose_kernel<KMAX, true>), dim3(a.B), dim3(NT), dyn, st, a);
  else
    hipLaunchKernelGGL((propose_kernel<KMAX, false>), dim3(a.B), dim3(NT), dyn, st, a);
  return hipGetLastError();
}

}  // namespace

size_t propose_dynamic_lds(bool staged, int S, int T, bool corpus) {
  return dyn_bytes(staged, S, T, corpus);
}

namespace {
size_t g_static_lds = 0;  // largest static LDS over the propose instantiations (queried)
}

size_t propose_static_lds() { return g_static_lds ? g_static_lds : sizeof(Smem); }

bool propose_staged(int S, int T, bool stream_ctx, bool corpus) {
  return !stream_ctx && dyn_bytes(true, S, T, corpus) + propose_static_lds() <= kLdsBytes;
}

hipError_t propose_prepare() {
  const void* fns[] = {
      (const void*)propose_kernel<8, true>,  (const void*)propose_kernel<8, false>,
      (const void*)propose_kernel<16, true>, (const void*)propose_kernel<16, false>,
      (const void*)propose_kernel<32, true>, (const void*)propose_kernel<32, false>};
  size_t st = sizeof(Smem);
  for (const void* f : fns) {
    hipFuncAttributes fa;
    hipError_t e = hipFuncGetAttributes(&fa, f);
    if (e != hipSuccess) return e;
    if (fa.sharedSizeBytes > st) st = fa.sharedSizeBytes;
  }
  if (st >= kLdsBytes) return hipErrorInvalidValue;
  for (const void* f : fns) {
    hipError_t e =
        hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kLdsBytes - st));
    if (e != hipSuccess) return e;
  }
  g_static_lds = st;
  return hipSuccess;
}

hipError_t launch_propose(const ProposeArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const bool corpus = a.ctl != nullptr;
  const bool staged = propose_staged(a.S, a.T, a.stream_ctx != 0, corpus);
  const size_t dyn = dyn_bytes(staged, a.S, a.T, corpus);
  if (dyn + propose_static_lds() > kLdsBytes) return hipErrorInvalidValue;
  if (a.k <= 8) return launch_k<8>(a, staged, dyn, st);
  if (a.k <= 16) return launch_k<16>(a, staged, dyn, st);
  return launch_k<32>(a, staged, dyn, st);
}

hipError_t launch_update_state(int B, int S, int T, int32_t* tok, const int32_t* ntns,
                               const int32_t* samp, int32_t* nout, hipStream_t st) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(update_state_kernel, dim3((B + 255) / 256), dim3(256), 0, st, B, S, T, tok,
                     ntns, samp, nout);
  return hipGetLastError();
}

}  // namespace sfx
