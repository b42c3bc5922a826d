// propose.hip -- the drafter step on gfx950: one workgroup (16 wavefronts) per request.
//
// Steps, in the order of the suffix-gpu page, How it works:
//   1. local match (step 1): each worker wavefront owns a contiguous chunk of end positions.  It
//      streams the chunk with coalesced bounds-checked loads (staging it, plus the 64 positions
//      before it, in LDS when the row fits there) and keeps one ballot word per 64 positions:
//      the end positions whose token is the last context token.  Without waiting for the other
//      wavefronts it then narrows those words to the positions whose previous token is the
//      second-to-last context token, computes their backward match lengths against the tail and
//      publishes per-length counts.  After one barrier among the workers, wavefront t derives
//      the t-th rung of the ladder (the t-th largest match length), gathers its earliest
//      continuation sites from the published lists and votes;
//   2. global match (step 2; vLLM docs, Model Runner V2: probe by the last 2 and last 4 tokens,
//      extend to the longest match): 2-, 3- and 4-gram probes into hash tables over the
//      suffix-array groups of the live snapshot and backward extension of the 4-gram
//      occurrences.  With a live snapshot and no delta a dedicated wavefront does all of it --
//      probes, ladder, earliest sites and the votes of the corpus candidates -- while the others
//      work through the local match.  With a delta (documents appended since the snapshot) the
//      whole workgroup then finds the delta's occurrences -- from the per-call pair index, or by
//      a brute-force scan -- and merges;
//   3. expansion (step 3): one wavefront per candidate votes depth by depth over its sites, with
//      the alive sites as wavefront masks (one ballot pair settles a depth whose alive sites
//      agree or hold a strict majority; ballots per token when few sites are alive, an LDS hash
//      otherwise); stop rule and score use integer cross-multiplication; selection and the [k]
//      output row follow.
#include <type_traits>

#include "delta_index.h"
#include "propose.h"

#ifndef SFX_PHASE_TRACE
#define SFX_PHASE_TRACE 0
#endif

namespace sfx {

namespace {

constexpr int NT = 1024;
constexpr int NW = NT / 64;
constexpr int GW = NW - 1;          // the corpus wavefront of the fast path
constexpr int kVoteSlots = 256;     // LDS hash slots of one voter (keys and counts)
constexpr int kSmallVote = 24;      // alive sites at or below this vote with ballots
constexpr int kColSites = 8;        // candidates with at most this many sites vote by columns
constexpr int kPrefetchTokens = 2048;  // row tokens fetched during the set-up round trip

// f(integral_constant<int, I>) for I = I0 .. N-1, unrolled at compile time (so that lane and
// register indices are immediates).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

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
// whole-wavefront lane moves: lane i takes lane i - 1 (lane 0 keeps the old value), and lane i
// takes lane i - 1 mod 64
constexpr int kDppWaveShr1 = 0x138;
constexpr int kDppWaveRor1 = 0x13C;

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

// Maximum over lanes 0 .. 15 (every lane takes part; the others hold their own row's).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppQuadXor1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppQuadXor2, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppHalfMirror, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppMirror, 0xF, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
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

__device__ __forceinline__ int lanes_before(uint64_t bal) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
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
// working through the local phase: an LDS arrival count.  Every worker wavefront passes it
// exactly once, so the count reaches the number of workers.  The wait is bounded so that every
// wavefront ends even if the count never arrives; running out of the bound raises
// kErrSyncTimeout in the context's error word (the call's results are then unreliable).
constexpr int kSpinBound = 1 << 24;
__device__ __forceinline__ void worker_barrier(int* ctr, int target, int lane, uint32_t* err) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  bool ok = false;
  for (int spin = 0; spin < kSpinBound; ++spin) {
    if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) {
      ok = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (!ok && lane == 0 && err)
    __hip_atomic_fetch_or(err, (uint32_t)kErrSyncTimeout, __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Bounded wait for an LDS flag set by another wavefront of the workgroup (same timeout
// convention as worker_barrier).
__device__ __forceinline__ void wait_flag(int* flag, int lane, uint32_t* err) {
  bool ok = false;
  for (int spin = 0; spin < kSpinBound; ++spin) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0) {
      ok = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (!ok && lane == 0 && err)
    __hip_atomic_fetch_or(err, (uint32_t)kErrSyncTimeout, __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ int ctx_at(const int32_t* row, const int32_t* smp, int n, int x) {
  return x < n ? row[x] : smp[x - n];
}

// An int in LDS, typed as such: a function that is not inlined sees a generic pointer
// otherwise, and reaches LDS through flat instructions (slower, and every one waits on the
// vector memory counter too).
typedef __attribute__((address_space(3))) int lds_int;
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i lds_v4i;

// Count this lane's votes for t0 (when p0) and t1 (when p1) in a wavefront's LDS table, by
// open addressing; *s0 / *s1 get the slots used (-1 for no vote).  The two inserts of a lane
// run side by side, so that their exchanges share one LDS round trip.
__device__ __forceinline__ void vote_insert2(lds_int* hk, lds_int* hc, bool p0, int t0, bool p1,
                                             int t1, int* s0, int* s1) {
  uint32_t h0 = ((uint32_t)t0 * 0x9E3779B1u) >> 24, h1 = ((uint32_t)t1 * 0x9E3779B1u) >> 24;
  *s0 = -1;
  *s1 = -1;
  while (p0 || p1) {
    int q0 = -1, q1 = -1;  // on return: the slot's key before the exchange
    if (p0)
      __hip_atomic_compare_exchange_strong(&hk[h0], &q0, t0, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
    if (p1)
      __hip_atomic_compare_exchange_strong(&hk[h1], &q1, t1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
    if (p0) {
      if (q0 == -1 || q0 == t0) {
        __hip_atomic_fetch_add(&hc[h0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        *s0 = (int)h0;
        p0 = false;
      } else {
        h0 = (h0 + 1) & (kVoteSlots - 1);
      }
    }
    if (p1) {
      if (q1 == -1 || q1 == t1) {
        __hip_atomic_fetch_add(&hc[h1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        *s1 = (int)h1;
        p1 = false;
      } else {
        h1 = (h1 + 1) & (kVoteSlots - 1);
      }
    }
  }
}

struct Smem {
  int tail[kMaxD];
  int gtail[kMaxD];
  // per worker wavefront w: wsuf[w][v] = its end positions with match length >= v (v >= 1);
  // while they are computed, wsuf[w][m] counts its lengths m >= 3 (converted in place)
  int wsuf[NW][kMaxD + 2];
  int wbeg[NW];          // first end position of each worker wavefront (its list base)
  int vex[kMaxNB][NW];   // per local voter: exclusive prefix of the scanned lists
  int ghist[kMaxD + 1];
  int dhist[kMaxD + 1];
  int g_off[kNG], g_live[kNG];
  int cand_len[2 * kMaxNB], cand_sup[2 * kMaxNB], cand_c0[2 * kMaxNB], cand_valid[2 * kMaxNB];
  int cand_src[2 * kMaxNB], cand_n[2 * kMaxNB];
  int cand_snum[2 * kMaxNB];  // at most k * M = 4096
  // 1 once candidate i's vote is final (its cand_n / cand_snum written before): the scored mode
  // drops a vote as soon as a final score beats every score it could still reach
  int cand_done[2 * kMaxNB];  // 0, or a final vote's 1 << 30 | snum << 8 | c0
  int cand_out[2 * kMaxNB][kMaxK];
  int lsites[kMaxNB][kMaxM];
  int gsites[kMaxNB][kMaxM];  // logical corpus positions minus the oldest live one (Ctl tail)
  int gpl[kNG][kMaxM];  // heads of the live 2-, 3- and 4-gram groups
  int gm4[kMaxM];       // extension lengths of the first 4-gram occurrences
  // hot 4-gram groups: per length l >= 5, the support and the first suffix-array index of the
  // suffixes that start with the length-l tail pattern and continue with a real token
  int hsup[kMaxD + 1], hlo[kMaxD + 1];
  int hoff[kMaxD + 1], hcnt[kMaxD + 1];  // position-list group of P_l's first 4-gram
  int ghot;  // 1 when the snapshot part of lengths >= 5 comes from them
  int sink[NW];   // the set-up prefetch's values (kept only so that the loads are made)
  int hrad[256];  // digit histogram of the hot site selection
  int hn;    // snapshot sites found by the general path's hot site pass
  const int32_t* plp[kNG];
  int wsum[NW + 1];
  int wbar;    // arrivals at the worker-only barrier
  int gready;  // the corpus wavefront has published its candidates and sites (fast path)
  int lready;  // local candidate 0's length and validity are written (fast path)
  uint8_t cap_tab[kMaxD + 1];  // the per-call draft cap and stop-count tables, staged
  uint8_t min_tab[kMaxM + 1];
#if SFX_PHASE_TRACE
  unsigned long long ts[NW][kTracePhases];
#endif
};

// Shape of one request and the corpus state it sees.  Every thread derives it from the same
// uniform loads, so no thread waits for another before the staging starts.
struct Req {
  int n, t, L, J, Lcap;
  int t0;  // the last context token (the last sampled id)
  int act;
  bool has, fast, delta;
  long long snap_start, snap_n, tail_w, delta_lo, delta_hi;
  uint32_t ht_mask;
};

// Flat view of one index buffer.  Separate scalar fields (no arrays) and constant-index
// selects keep the kernel arguments out of scratch memory.
struct View {
  const int32_t* text;
  const int32_t* sa;
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
  v.sa = z ? a.idx[0].sa : a.idx[1].sa;
  v.pl0 = z ? a.idx[0].pl[0] : a.idx[1].pl[0];
  v.pl1 = z ? a.idx[0].pl[1] : a.idx[1].pl[1];
  v.pl2 = z ? a.idx[0].pl[2] : a.idx[1].pl[2];
  v.ht0 = z ? a.idx[0].ht[0] : a.idx[1].ht[0];
  v.ht1 = z ? a.idx[0].ht[1] : a.idx[1].ht[1];
  v.ht2 = z ? a.idx[0].ht[2] : a.idx[1].ht[2];
  return v;
}

// Probe of the (g+2)-gram that ends the context: its group in the position list, minus the
// prefix of occurrences in documents evicted since the snapshot.  The n-gram is chosen at run
// time (g = lane), so that the three probes of one wavefront run side by side, not one branch
// after another.
__device__ __forceinline__ void probe_lane(const View ib, const int* tail, int Lcap,
                                           long long dead_below, int g, int* off_out,
                                           int* live_out) {
  const int ng = g + 2;
  int off = 0, live = 0;
  if (ng <= Lcap) {
    int key[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) key[x] = x < ng ? tail[x < ng ? ng - 1 - x : 0] : -1;
    const NgramSlot* ht = g == 0 ? ib.ht0 : (g == 1 ? ib.ht1 : ib.ht2);
    const int32_t* plist = g == 0 ? ib.pl0 : (g == 1 ? ib.pl1 : ib.pl2);
    uint32_t h = ngram_hash4(key, ng) & ib.mask;
    int cnt = 0;
    for (;;) {
      const NgramSlot s = ht[h];
      if (s.owner == 0) break;
      if (s.key[0] == key[0] && s.key[1] == key[1] && s.key[2] == key[2] &&
          s.key[3] == key[3]) {
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
// (>= 4) against the tail, at most `cap`, given that the `start` tokens before it match already.
// The preceding tokens are fetched kExtRound at a time, all of them in flight together, so a
// match of up to kExtRound + 4 tokens costs one round trip.
constexpr int kExtRound = 20;
__device__ __noinline__ int extend4(const int32_t* text, const int* tail, int i, int cap,
                                    int start = 0) {
  int m = 4 + start;
  for (int base = start; base < cap - 4; base += kExtRound) {
    int c[kExtRound];
#pragma unroll
    for (int q = 0; q < kExtRound; ++q) {
      const int o = base + q;
      c[q] = (o < cap - 4 && i - 1 - o >= 0) ? text[i - 1 - o] : -2;
    }
    bool stop = false;
    int run = 0;
#pragma unroll
    for (int q = 0; q < kExtRound; ++q) {
      const int ti = 4 + base + q < kMaxD ? 4 + base + q : kMaxD - 1;
      stop = stop || c[q] < 0 || c[q] != tail[ti];
      run += stop ? 0 : 1;
    }
    m += run;
    if (stop) break;
  }
  return m;
}

// Hot 4-gram groups (suffix-gpu page, How it works step 2: a fixed-iteration binary search of the
// suffix array for every pattern length).  Extending each live occurrence of the tail's 4-gram
// costs one round trip per 64 occurrences, so above kHotGroup of them the snapshot part of
// lengths >= 5 comes from the suffix array instead.  The suffixes that start with the length-l
// tail pattern P_l and continue with a real token form one range of it, inside the group of
// the 4-gram that starts P_l (whose range the probe table holds): two bound searches per length,
// all lengths at once, give every support.  A candidate's earliest sites are then the smallest
// positions of its range, selected from the range itself, or found by a position-ordered scan of
// a 4-gram group that stops after M of them (about M * group / support entries), whichever
// costs fewer round trips.  This needs every snapshot position live, so it
// is not used while documents evicted since the snapshot still lie in it.
constexpr int kHotGroup = 1024;
constexpr int kHotSelect = 2048;  // range entries read per selection chunk
constexpr int kHotCmp = 16;  // suffix tokens compared per round trip

// Bounds of lengths l = 5 .. Lcap: lane pair (2 (l - 5), 2 (l - 5) + 1) finds the first index of
// the range whose suffix is >= P_l followed by token 0 (lower bound), and the first whose suffix
// is above every suffix with prefix P_l (upper bound).  tl[x] is the context token x places
// before the last one.  Writes sup[l] and lo[l] for 5 <= l <= Lcap, and the 4-gram group's
// position-list offset and size in goff[l], gcnt[l].
//
// A function of its own (so is hot_sites): only a hot group runs it, and inlined its code sits
// in every request's path and instruction cache.  Its arrays are in LDS, typed as such inside,
// so that it reaches them with ds instructions rather than flat ones.
__device__ __noinline__ void hot_bounds(const View ib, const int* tl_g, int Lcap, int snap_n,
                                        int lane, int* sup_g, int* lo_g, int* goff_g, int* gcnt_g) {
  const lds_int* tl = (const lds_int*)tl_g;
  lds_int* sup = (lds_int*)sup_g;
  lds_int* lo_out = (lds_int*)lo_g;
  lds_int* goff = (lds_int*)goff_g;
  lds_int* gcnt = (lds_int*)gcnt_g;
  for (int pass = 0; pass < 2; ++pass) {
    const int idx = lane + 64 * pass;
    const int l = 5 + (idx >> 1), side = idx & 1;
    int lo = 0;
    if (l <= Lcap) {
      // the group of Q_l = P_l[0..3] = tl[l-1], tl[l-2], tl[l-3], tl[l-4]
      int key[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) key[x] = tl[l - 1 - x];
      uint32_t h = ngram_hash4(key, 4) & ib.mask;
      int beg = 0, cnt = 0, off = 0;
      for (;;) {
        const NgramSlot s = ib.ht2[h];
        if (s.owner == 0) break;
        if (s.key[0] == key[0] && s.key[1] == key[1] && s.key[2] == key[2] &&
            s.key[3] == key[3]) {
          beg = s.sa_lo;
          cnt = s.cnt;
          off = s.off;
          break;
        }
        h = (h + 1) & ib.mask;
      }
      if (side == 0) {
        goff[l] = off;
        gcnt[l] = cnt;
      }
      lo = beg;
      int hi = beg + cnt;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const int pos = ib.sa[mid];
        // compare the suffix at pos from offset 4 on with P_l (then, for the lower bound, with
        // token 0 at offset l); every suffix of the group matches offsets 0..3
        int cmp = 0;  // -1 suffix below, +1 above, 0 equal so far
        for (int o0 = 4; o0 <= l && cmp == 0; o0 += kHotCmp) {
          int c[kHotCmp];
#pragma unroll
          for (int q = 0; q < kHotCmp; ++q) {
            // the text ends with a separator, which decides before any clamped read matters
            const int at = pos + o0 + q < snap_n ? pos + o0 + q : snap_n - 1;
            c[q] = ib.text[at];
          }
#pragma unroll
          for (int q = 0; q < kHotCmp; ++q) {
            const int o = o0 + q;
            if (cmp == 0 && o <= l) {
              if (o < l) {
                const int p = tl[l - 1 - o];
                cmp = c[q] < p ? -1 : (c[q] > p ? 1 : 0);
              } else if (side == 0) {
                cmp = c[q] < 0 ? -1 : 1;  // continues with a separator: below P_l, 0
              }
            }
          }
        }
        const bool right = side == 0 ? cmp < 0 : cmp <= 0;
        if (right) lo = mid + 1;
        else hi = mid;
      }
    }
    const int up = __builtin_amdgcn_ds_bpermute(4 * ((lane + 1) & 63), lo);
    if (l <= Lcap && side == 0) {
      sup[l] = up - lo;
      lo_out[l] = lo;
    }
  }
}

// Earliest sites of a hot candidate of length l from its range [lo, lo + sup): the m =
// min(M, sup) smallest suffix positions, put in order by rank; gs[r] = position + l + sbase.
// The range is read kHotSelect entries at a time; the m smallest of a chunk and of the best so
// far (two per lane) are those up to the m-th smallest, found digit by digit (8 bits at a time)
// from a histogram in LDS (positions are distinct).  Returns m.
__device__ __forceinline__ int hot_select(const View ib, int* hist, int lo, int sup, int l, int M,
                                       int snap_n, int sbase, int* gs, int lane) {
  constexpr int Q = kHotSelect / 64;
  constexpr int kNone = 0x7fffffff;
  const int top = 32 - __builtin_clz((unsigned)(snap_n > 1 ? snap_n - 1 : 1));
  const int shift0 = ((top + 7) / 8 - 1) * 8;  // lowest bit of the highest digit
  int b0 = kNone, b1 = kNone, nb = 0;
  for (int c0 = 0; c0 < sup; c0 += kHotSelect) {
    int v[Q + 2];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = c0 + lane + 64 * q;
      v[q] = e < sup ? ib.sa[lo + e] : kNone;
    }
    v[Q] = b0;
    v[Q + 1] = b1;
    const int cn = sup - c0 < kHotSelect ? sup - c0 : kHotSelect;
    const int m = nb + cn < M ? nb + cn : M;
    // the m-th smallest of the chunk and the best so far
    int prefix = 0, need = m;
    for (int sh = shift0; sh >= 0; sh -= 8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) hist[4 * lane + q] = 0;
      wave_sync();
      const unsigned hi_mask = sh + 8 >= 32 ? 0u : ~((1u << (sh + 8)) - 1u);
#pragma unroll
      for (int q = 0; q < Q + 2; ++q) {
        const unsigned x = (unsigned)v[q];
        if (v[q] != kNone && (x & hi_mask) == (unsigned)prefix)
          atomicAdd(&hist[(x >> sh) & 255u], 1);
      }
      wave_sync();
      const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                h3 = hist[4 * lane + 3];
      const int tot = h0 + h1 + h2 + h3;
      const int incl = wave_incl_add(tot);
      const int excl = incl - tot;
      // the lane whose four digits hold the need-th value, then the digit inside it
      const uint64_t past = __ballot(incl >= need);
      const int owner = __builtin_ctzll(past);
      int d = 4 * lane, below = excl;
      if (below + h0 < need) {
        below += h0;
        d += 1;
        if (below + h1 < need) {
          below += h1;
          d += 1;
          if (below + h2 < need) {
            below += h2;
            d += 1;
          }
        }
      }
      const int dd = __builtin_amdgcn_readlane(d, owner);
      const int bb = __builtin_amdgcn_readlane(below, owner);
      prefix |= dd << sh;
      need -= bb;
      wave_sync();
    }
    // keep the m values <= prefix, in any order
    int n = 0;
#pragma unroll
    for (int q = 0; q < Q + 2; ++q) {
      const bool k = v[q] != kNone && v[q] <= prefix;
      const uint64_t bal = __ballot(k);
      if (k) gs[n + lanes_before(bal)] = v[q];
      n += __popcll(bal);
    }
    wave_sync();
    b0 = lane < m ? gs[lane] : kNone;
    b1 = lane + 64 < m ? gs[lane + 64] : kNone;
    nb = m;
    wave_sync();
  }
  const int m = nb;
  int r0 = 0, r1 = 0;
  for (int j = 0; j < m; ++j) {
    const int x = gs[j];
    r0 += x < b0 ? 1 : 0;
    r1 += x < b1 ? 1 : 0;
  }
  wave_sync();
  if (lane < m) gs[r0] = b0 + l + sbase;
  if (lane + 64 < m) gs[r1] = b1 + l + sbase;
  wave_sync();
  return m;
}

// Earliest sites of a hot candidate of length l with a larger range, from the position list of
// the 4-gram that starts P_l (pl, cnt entries, each the start of a continuing occurrence of it):
// in position order, the entries whose suffix goes on with the rest of P_l and then a real token,
// until M are found.  Returns how many.
__device__ __forceinline__ int hot_scan_head(const View ib, const int32_t* pl, int cnt,
                                          const int* tl, int l, int M, int snap_n, int sbase,
                                          int* gs, int lane) {
  const uint64_t below = lanes_below(lane);
  int run = 0;
  for (int base = 0; base < cnt && run < M; base += 64) {
    const int x = base + lane;
    const int pos = x < cnt ? pl[x] : 0;
    bool live = x < cnt, ok = live;
    for (int o0 = 4; o0 <= l && __ballot(live); o0 += kHotCmp) {
      int c[kHotCmp];
#pragma unroll
      for (int q = 0; q < kHotCmp; ++q) {
        const int at = pos + o0 + q < snap_n ? pos + o0 + q : snap_n - 1;
        c[q] = ib.text[at];
      }
#pragma unroll
      for (int q = 0; q < kHotCmp; ++q) {
        const int o = o0 + q;
        if (live && o <= l) {
          const bool eq = o < l ? c[q] == tl[l - 1 - o] : c[q] >= 0;
          ok = ok && eq;
          live = eq && o < l;
        }
      }
    }
    const uint64_t bal = __ballot(ok);
    const int rk = run + __popcll(bal & below);
    if (ok && rk < M) gs[rk] = pos + l + sbase;
    run += __popcll(bal);
  }
  return run < M ? run : M;
}

// Earliest sites of a hot candidate of length l with a larger range: the live 4-gram
// occurrences in position order whose extension reaches l, until M are found.  Returns how many.
__device__ __forceinline__ int hot_scan(const View ib, const int32_t* pl4, int live4,
                                        const int* tl, int l, int M, int sbase, int* gs,
                                        int lane) {
  const uint64_t below = lanes_below(lane);
  int run = 0;
  for (int base = 0; base < live4 && run < M; base += 64) {
    const int x = base + lane;
    const int i = x < live4 ? pl4[x] : 0;
    const bool q = x < live4 && extend4(ib.text, tl, i, l) >= l;
    const uint64_t bal = __ballot(q);
    const int rk = run + __popcll(bal & below);
    if (q && rk < M) gs[rk] = i + 4 + sbase;
    run += __popcll(bal);
  }
  return run < M ? run : M;
}

// Earliest sites of hot candidate length l: selection from its range when it is small, else the
// position-ordered scan of whichever 4-gram group is smaller (the one that starts P_l, or the
// tail's).  Returns how many were written to gs.
__device__ __noinline__ int hot_sites(const View ib, Smem& sm_g, const int* tl_g, int l, int M,
                                      int snap_n, int sbase, const int32_t* pl4, int live4,
                                      int* gs_g, int lane) {
  // (sm, the tail and the sites are in LDS: cast through LDS pointers, the inlined helpers reach
  // them with ds instructions)
  Smem& sm = *(Smem*)(lds_int*)(int*)&sm_g;
  const int* tl = (const int*)(const lds_int*)tl_g;
  int* gs = (int*)(lds_int*)gs_g;
  const int sup = sm.hsup[l];
  const int hcnt = sm.hcnt[l];
  // costs in round trips: a selection chunk is one plus about as much arithmetic; a scan takes
  // about two and a half per 64 entries, and reaches M sites after about M * group / sup of them
  const long long sel = 2ll * ((sup + kHotSelect - 1) / kHotSelect);
  const bool head = hcnt <= live4;
  const long long grp = head ? hcnt : live4;
  const long long scan = 5ll * ((long long)M * grp / sup / 64 + 1) / 2;
  if (sel <= scan) return hot_select(ib, sm.hrad, sm.hlo[l], sup, l, M, snap_n, sbase, gs, lane);
  if (head) return hot_scan_head(ib, ib.pl2 + sm.hoff[l], hcnt, tl, l, M, snap_n, sbase, gs, lane);
  return hot_scan(ib, pl4, live4, tl, l, M, sbase, gs, lane);
}

// Backward extension of two 4-gram occurrences at once (q0, q1: whether each exists): the four
// tokens before each are fetched together (unconditionally, at clamped positions), and only a
// match that runs through all four goes on with extend4.
__device__ __forceinline__ void extend4_pair(const int32_t* text, const int* tail, int i0,
                                             bool q0, int i1, bool q1, int cap, int* m0,
                                             int* m1) {
  int c[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    c[q] = text[i0 - 1 - q >= 0 ? i0 - 1 - q : 0];
    c[4 + q] = text[i1 - 1 - q >= 0 ? i1 - 1 - q : 0];
  }
  bool s0 = !q0, s1 = !q1;
  int r0 = 0, r1 = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = tail[4 + q];
    const bool in = q < cap - 4;
    s0 = s0 | !in | (i0 - 1 - q < 0) | (c[q] < 0) | (c[q] != t);
    s1 = s1 | !in | (i1 - 1 - q < 0) | (c[4 + q] < 0) | (c[4 + q] != t);
    r0 += s0 ? 0 : 1;
    r1 += s1 ? 0 : 1;
  }
  *m0 = 4 + r0;
  *m1 = 4 + r1;
  if (!s0 && cap > 8) *m0 = extend4(text, tail, i0, cap, 4);
  if (!s1 && cap > 8) *m1 = extend4(text, tail, i1, cap, 4);
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

// Listed delta entries: wavefront w of a request walks the request's group in slices
// w * kListSlices .. (w + 1) * kListSlices - 1, one running entry number v over them.  Lane j <
// kListSlices holds slice j's first entry number (non-decreasing in j) in `first` and the
// difference between its list index and its entry number in `shift`; entry v is in the last
// slice whose first entry number is at most v.  Every lane of the wavefront must take part.
constexpr int kListSlices = kPairSlices / NW;
__device__ __forceinline__ int list_index(int v, int first, int shift) {
  int j = 0;
#pragma unroll
  for (int q = 1; q < kListSlices; ++q) j += v >= __builtin_amdgcn_readlane(first, q) ? 1 : 0;
  return v + __builtin_amdgcn_ds_bpermute(4 * j, shift);
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
                                                int lane, int lfirst, int lshift, F&& f) {
  const int cap = (int)a.ring_cap;
  const int dslot = (int)(dlo % a.ring_cap);
  for (long long e0 = i0; e0 < i1; e0 += 64 * kListBatches) {
    uint32_t o[kListBatches];
    int li[kListBatches];
#pragma unroll
    for (int u = 0; u < kListBatches; ++u) li[u] = list_index((int)(e0 + 64 * u + lane), lfirst, lshift);
#pragma unroll
    for (int u = 0; u < kListBatches; ++u) {
      const long long i = e0 + 64 * u + lane;
      o[u] = i < i1 ? a.pair_list[li[u]] : 0u;
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

// The vote at one depth when the reference token (the first voting site's) holds no strict
// majority among the na voting sites (alive and with a token at this depth), for at most
// kSmallVote voters: the count of every token, then the largest count and the smallest token
// among the largest.  x0 / x1 are this lane's two sites' tokens, V0 / V1 the voting sites, E0 /
// E1 those voting for ref (all wavefront-uniform but x0 / x1).  Returns count << 32 | token.
// One ballot pair per distinct token, until the best count exceeds every vote not yet counted
// (a tie with a smaller token still has to be looked at), or until neither the best count nor
// the votes left reach cmin: the count is then below cmin (the vote stops there, whatever the
// token).  After kSmallRounds tokens without an end it gives up (*fin false): the hash count
// then takes the vote.
constexpr int kSmallRounds = 12;
__device__ __forceinline__ uint64_t vote_small(int x0, int x1, uint64_t V0, uint64_t V1, int ref,
                                               uint64_t E0, uint64_t E1, int na, int cmin,
                                               bool* fin) {
  const int ce = __popcll(E0) + __popcll(E1);
  uint64_t key = ((uint64_t)ce << 32) | (uint32_t)(0x7FFFFFFF - ref);
  uint64_t r0 = V0 & ~E0, r1 = V1 & ~E1;
  int rest = na - ce;
  *fin = false;
#pragma nounroll
  for (int it = 0; it < kSmallRounds; ++it) {
    if (!((r0 | r1) && (int)(key >> 32) <= rest && (rest >= cmin || (int)(key >> 32) >= cmin))) {
      *fin = true;
      break;
    }
    const int tok = r0 ? __builtin_amdgcn_readlane(x0, __builtin_ctzll(r0))
                       : __builtin_amdgcn_readlane(x1, __builtin_ctzll(r1));
    const uint64_t e0 = __ballot(x0 == tok) & r0, e1 = __ballot(x1 == tok) & r1;
    const int ct = __popcll(e0) + __popcll(e1);
    const uint64_t k = ((uint64_t)ct << 32) | (uint32_t)(0x7FFFFFFF - tok);
    key = k > key ? k : key;
    r0 &= ~e0;
    r1 &= ~e1;
    rest -= ct;
  }
  return (key >> 32) << 32 | (uint32_t)(0x7FFFFFFF - (int)(uint32_t)(key & 0xFFFFFFFFu));
}

// The same vote for more than kSmallVote voters, or many distinct tokens, by counting in an LDS
// hash (a function of its own: this path is rare and its code is long).
__device__ __noinline__ uint64_t vote_split(int x0, int x1, uint64_t V0, uint64_t V1, int ref,
                                            uint64_t E0, uint64_t E1, lds_int* hk, lds_int* hc,
                                            int lane) {
  // wavefront-uniform arguments arrive in vector registers: make them scalar again
  auto u64 = [](uint64_t v) {
    return (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v) |
           ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32)) << 32);
  };
  V0 = u64(V0);
  V1 = u64(V1);
  E0 = u64(E0);
  E1 = u64(E1);
  ref = __builtin_amdgcn_readfirstlane(ref);
  const int ce = __popcll(E0) + __popcll(E1);
  // many voting sites: the reference's count is ce; the other voters' tokens are counted in an
  // LDS hash (at most 127 distinct in 256 slots), then the largest count and smallest token
  // over both
  static_assert(kVoteSlots == 4 * 64, "one 16-byte store per lane clears a table");
  const bool v0 = ((V0 & ~E0) >> lane) & 1, v1 = ((V1 & ~E1) >> lane) & 1;
  reinterpret_cast<lds_v4i*>(hk)[lane] = v4i{-1, -1, -1, -1};
  reinterpret_cast<lds_v4i*>(hc)[lane] = v4i{0, 0, 0, 0};
  wave_sync();
  int sl0, sl1;
  vote_insert2(hk, hc, v0, x0, v1, x1, &sl0, &sl1);
  wave_sync();
  const int cnt0 = sl0 >= 0 ? hc[sl0] : 0, cnt1 = sl1 >= 0 ? hc[sl1] : 0;
  uint64_t res;
  if (ref < (1 << 24) && __ballot((v0 && x0 >= (1 << 24)) || (v1 && x1 >= (1 << 24))) == 0) {
    // tokens below 2^24: count and token packed in one key, one reduction
    const uint32_t k0 = sl0 >= 0 ? ((uint32_t)cnt0 << 24) | (uint32_t)(0xFFFFFF - x0) : 0u;
    const uint32_t k1 = sl1 >= 0 ? ((uint32_t)cnt1 << 24) | (uint32_t)(0xFFFFFF - x1) : 0u;
    const uint32_t kr = ((uint32_t)ce << 24) | (uint32_t)(0xFFFFFF - ref);
    uint32_t key = wave_max_u32(k0 > k1 ? k0 : k1);
    key = key > kr ? key : kr;
    res = (uint64_t)(key >> 24) << 32 | (uint32_t)(0xFFFFFF - (int)(key & 0xFFFFFFu));
  } else {
    int c = wave_max(cnt0 > cnt1 ? cnt0 : cnt1);
    c = c > ce ? c : ce;
    int tmin = 0x7FFFFFFF;
    if (sl0 >= 0 && cnt0 == c) tmin = x0;
    if (sl1 >= 0 && cnt1 == c && x1 < tmin) tmin = x1;
    tmin = wave_min(tmin);
    if (ce == c && ref < tmin) tmin = ref;
    res = (uint64_t)(uint32_t)c << 32 | (uint32_t)tmin;
  }
  wave_sync();
  return res;
}

// Index of the lowest set bit of m, or KMAX when none is set below KMAX.
template <int KMAX>
__device__ __forceinline__ int first_set(uint32_t m) {
  const int f = m ? __builtin_ctz(m) : 32;
  return f < KMAX ? f : KMAX;
}

// The second half of vote_depth, for a caller that has the voting sites V0 / V1 (not both
// empty), the reference token ref (the first voting site's) and its voters E0 / E1 already.
__device__ __forceinline__ void vote_decide(int x0, int x1, uint64_t V0, uint64_t V1, int ref,
                                            uint64_t E0, uint64_t E1, int cmin, int* hk, int* hc,
                                            int lane, int* w, int* c) {
  *c = 0;
  *w = -1;
  const int na = __popcll(V0) + __popcll(V1);
  const int ce = __popcll(E0) + __popcll(E1);
  if (2 * ce > na) {
    *w = ref;
    *c = ce;
  } else if (na < cmin) {
    *c = na;  // no token reaches the stop count: any count below cmin stops the vote
  } else {
    bool fin = false;
    uint64_t rs = 0;
    if (na <= kSmallVote) rs = vote_small(x0, x1, V0, V1, ref, E0, E1, na, cmin, &fin);
    if (fin) {
      *c = (int)(rs >> 32);
      *w = (int)(uint32_t)rs;
      return;
    }
    // (the call returns in vector registers: readfirstlane tells the compiler that the winner
    // and its count are wavefront-uniform, or every loop around this becomes a divergent one)
    const uint64_t res = vote_split(x0, x1, V0, V1, ref, E0, E1, (lds_int*)hk, (lds_int*)hc, lane);
    *c = __builtin_amdgcn_readfirstlane((int)(res >> 32));
    *w = __builtin_amdgcn_readfirstlane((int)(uint32_t)res);
  }
}

// One depth of the vote, decided from scratch: x0 / x1 are this lane's two sites' tokens, A0 / A1
// the alive sites.  On return *w / *c hold the winner and its count, or *c = 0 when no alive
// site has a token here.
__device__ __forceinline__ void vote_depth(int x0, int x1, uint64_t A0, uint64_t A1, int cmin,
                                           int* hk, int* hc, int lane, int* w, int* c) {
  const uint64_t V0 = __ballot(x0 >= 0) & A0, V1 = __ballot(x1 >= 0) & A1;
  *c = 0;
  *w = -1;
  if ((V0 | V1) == 0) return;
  // the reference is the first voting site's token; when every voting site agrees with it, or a
  // strict majority does, it wins with their votes
  const int ref = V0 ? __builtin_amdgcn_readlane(x0, __builtin_ctzll(V0))
                     : __builtin_amdgcn_readlane(x1, __builtin_ctzll(V1));
  const uint64_t E0 = __ballot(x0 == ref) & V0, E1 = __ballot(x1 == ref) & V1;
  vote_decide(x0, x1, V0, V1, ref, E0, E1, cmin, hk, hc, lane, w, c);
}

// Scored selection: whether a candidate other than ci whose vote is final beats every score ci
// can still reach, bnum / bden (a higher score, or the same one earlier in candidate order), so
// that ci cannot be selected.  Scores compare by cross products (snum <= 4096, c0 <= 128).
__device__ __forceinline__ bool outscored(Smem& sm, int ci, int nb, int bnum, int bden,
                                          int lane) {
  const bool on = lane < 2 * nb && lane != ci;
  // a final vote's word carries its score: 1 << 30 | snum << 8 | c0 (one read, no fence)
  const int dn = on ? __hip_atomic_load(&sm.cand_done[lane], __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_WORKGROUP)
                    : 0;
  const int sj = (dn & 0x3FFFFFFF) >> 8, cj = dn & 0xFF;
  const int lhs = sj * bden, rhs = bnum * cj;
  return __ballot(dn != 0 && (lhs > rhs || (lhs == rhs && lane < ci))) != 0;
}

// w[e] for a wavefront-uniform e < KMAX (a power of two), by a tree of selects on e's bits:
// registers cannot be indexed at run time.
template <int KMAX>
__device__ __forceinline__ int pick_depth(const int (&w)[KMAX], int e) {
  int x[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) x[i] = w[i];
#pragma unroll
  for (int h = KMAX / 2; h >= 1; h /= 2) {
    const bool hi = (e & h) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) x[i] = hi ? x[i + h] : x[i];
  }
  return x[0];
}

// Depth-wise vote, depth by depth from depth d, with the alive sites as wavefront masks A0 / A1:
// lane l owns sites l and l + 64, whose windows are w0 / w1 (-1 past a window's end).  A depth
// whose voting sites all carry the first voting site's token is settled by one ballot pair;
// otherwise vote_depth decides it.  TWO: whether slot 1 holds sites (more than 64).
template <int KMAX, bool TWO>
__device__ __forceinline__ void vote_seq(const int (&w0)[KMAX], const int (&w1)[KMAX],
                                         uint64_t A0, uint64_t A1, int d, int dmax, int cmin,
                                         int* hk, int* hc, int lane, int* nout_io, int* snum_io,
                                         int* tokv_io) {
  int nout = *nout_io, snum = *snum_io, tokv = *tokv_io;
  bool done = false;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    if (done || i < d || i >= dmax) continue;
    // the depth's tokens pass through an empty asm, so that its compares are issued in depth
    // order: hoisted, the 64-bit masks of every depth would not fit the scalar registers
    int x0 = w0[i], x1 = TWO ? w1[i] : -1;
    asm volatile("" : "+v"(x0), "+v"(x1));
    const uint64_t V0 = __ballot(x0 >= 0) & A0;
    const uint64_t V1 = TWO ? __ballot(x1 >= 0) & A1 : 0ull;
    if ((V0 | V1) == 0) {
      done = true;
      continue;
    }
    const int ref = V0 ? __builtin_amdgcn_readlane(x0, __builtin_ctzll(V0))
                       : __builtin_amdgcn_readlane(x1, __builtin_ctzll(V1));
    const uint64_t E0 = __ballot(x0 == ref) & V0;
    const uint64_t E1 = TWO ? __ballot(x1 == ref) & V1 : 0ull;
    int w = ref, c;
    if (E0 == V0 && E1 == V1) {
      c = __popcll(V0) + (TWO ? __popcll(V1) : 0);
    } else {
      vote_decide(x0, x1, V0, V1, ref, E0, E1, cmin, hk, hc, lane, &w, &c);
    }
    if (c < cmin) {
      done = true;
      continue;
    }
    A0 = __ballot(x0 == w) & V0;
    if (TWO) A1 = __ballot(x1 == w) & V1;
    tokv = lane == i ? w : tokv;
    snum += c;
    nout = i + 1;
  }
  *nout_io = nout;
  *snum_io = snum;
  *tokv_io = tokv;
}

// Depth-wise vote of one candidate held by one wavefront: lane l owns sites l and l+64, whose
// continuation windows are w0 / w1 (-1 past the end of a continuation and from depth cap on;
// len0 / len1 leading tokens, windows end for good).  Writes the voted tokens to out[] and
// returns their number and the sum of their counts.  cmin is the smallest count the
// stop rule keeps (0 without a stop rule).  hk / hc: this voter's LDS table.
//
// With at most 64 sites, depths are first settled in passes against a representative site r.
// The sites that agree with r through depth d form r's group at d; when it is larger than all
// other sites voting at d together, r's token wins with the group's count (no other token can
// match it).  One pass takes each alive site's first disagreement with r, histograms those
// depths (LDS atomics), and by one suffix scan and one ballot finds the first depth that r's
// group does not settle or where the vote stops; every depth before it is settled at once.
// That depth is voted from scratch, the winner's first site becomes the representative, and
// the next pass starts after it.  Short votes, votes of more than 64 sites and what the passes
// leave go depth by depth.  Returns false when the vote was dropped because beaten(bound)
// reported that another candidate's final score beats the best this one can still reach (the
// sum bound / c0); n_out and snum_out are then 0.
// (a pass costs as much as several depths voted one by one: votes of up to 10 depths go depth
// by depth, which measured faster than passes from 4, 5, 7 or 9 depths on)
constexpr int kPathMinDepths = 11;
constexpr int kPathPasses = 3;
template <int KMAX, typename Beaten>
__device__ __forceinline__ bool vote_run(const int (&w0)[KMAX], const int (&w1)[KMAX], int len0,
                                         int c0, int cap, int cmin, int* hk, int* hc, int lane,
                                         Beaten&& beaten, int* out, int* n_out, int* snum_out,
                                         unsigned long long* vts) {
#if SFX_PHASE_TRACE
#define VSTAMP(i)                                                \
  do {                                                           \
    if (vts && lane == 0) vts[i] = __builtin_amdgcn_s_memtime(); \
  } while (0)
  if (vts) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the windows have landed
  VSTAMP(11);
#else
#define VSTAMP(i) \
  do {            \
  } while (0)
  (void)vts;
#endif
  uint64_t A0 = __ballot(lane < c0), A1 = __ballot(lane + 64 < c0);
  int nout = 0, snum = 0, tokv = -1;
  const int dmax = cap < KMAX ? cap : KMAX;
  int d = 0;  // next depth to vote
  bool done = dmax <= 0;
  // counts never grow with depth (the sites voting at a depth are the previous winner's), so
  // snum + clast * (dmax - nout) bounds the final sum; clast: the last count taken
  int clast = c0;
  bool cut = false;  // dropped: another candidate's final score beats every reachable one
  if (!done && c0 <= 64 && dmax >= kPathMinDepths) {
    int r = 0;
    for (int pass = 0; pass < kPathPasses; ++pass) {
      if (pass > 0 && beaten(snum + clast * (dmax - nout))) {
        cut = true;
        break;
      }
      // each site's first depth of disagreement with r (r's end counts as one); lane i picks up
      // r's token at depth i
      uint32_t mm = 0;
      int rtl = -1;
#pragma unroll
      for (int i = 0; i < KMAX; ++i) {
        int x = __builtin_amdgcn_readlane(w0[i], r);
        rtl = lane == i ? x : rtl;
        x = x < 0 ? (int)0x80000000 : x;
        mm |= (w0[i] != x ? 1u : 0u) << i;
      }
      const int lcp = first_set<KMAX>(mm);
      const int al = (int)((A0 >> lane) & 1);
      // histograms over depth bins: hk[m] = alive sites whose first disagreement is m,
      // hc[m] = those of them that still have a token at m
      if (lane <= KMAX) {
        hk[lane] = 0;
        hc[lane] = 0;
      }
      atomicAdd(&hk[lcp], al);
      atomicAdd(&hc[lcp], al & (len0 > lcp ? 1 : 0));
      wave_sync();
      // lane i: g = r's group at depth i (sites agreeing through i), o = other sites voting there
      const int h = lane <= KMAX ? hk[lane] : 0;
      const int o = lane < KMAX ? hc[lane] : 0;
      const int incl = wave_incl_add(h);
      const int g = __builtin_amdgcn_readlane(incl, 63) - incl;
      const bool in = lane >= d && lane < dmax;
      const bool stop = g + o == 0 || (g > o && g < cmin);
      const uint64_t ev = __ballot(in && (stop || g <= o));
      const int e = ev ? (int)__builtin_ctzll(ev) : dmax;
      if (pass == 0) VSTAMP(12);
      // depths d .. e-1 are settled: tokens r's, counts g
      const bool acc = lane >= d && lane < e;
      tokv = acc ? rtl : tokv;
      const int gs = wave_incl_add(acc ? g : 0);
      snum += __builtin_amdgcn_readlane(gs, 63);
      clast = e > d ? __builtin_amdgcn_readlane(g, e - 1) : clast;
      nout = e > d ? e : nout;
      wave_sync();
      if (e >= dmax || (__ballot(stop) >> e) & 1) {
        done = true;
        break;
      }
      // depth e from scratch, over the sites still on r's path
      const uint64_t B0 = __ballot(al && lcp >= e);
      const int xe = pick_depth<KMAX>(w0, e);
      const int x0 = ((B0 >> lane) & 1) && len0 > e ? xe : -1;
      int w, c;
      vote_depth(x0, -1, B0, 0ull, cmin, hk, hc, lane, &w, &c);
      if (pass == 0) VSTAMP(13);
      if (c == 0 || c < cmin) {
        done = true;
        break;
      }
      tokv = lane == e ? w : tokv;
      snum += c;
      clast = c;
      nout = e + 1;
      A0 = __ballot(x0 == w) & B0;
      d = e + 1;
      if (d >= dmax) {
        done = true;
        break;
      }
      r = (int)__builtin_ctzll(A0);
    }
  }
  VSTAMP(14);
  if (!done && !cut && beaten(snum + clast * (dmax - nout))) cut = true;
  if (!done && !cut) {
    if (c0 > 64) vote_seq<KMAX, true>(w0, w1, A0, A1, d, dmax, cmin, hk, hc, lane, &nout, &snum,
                                      &tokv);
    else vote_seq<KMAX, false>(w0, w1, A0, 0ull, d, dmax, cmin, hk, hc, lane, &nout, &snum,
                               &tokv);
  }
  VSTAMP(15);
#undef VSTAMP
  if (cut) {
    *n_out = 0;
    *snum_out = 0;
    return false;
  }
  if (lane < nout) out[lane] = tokv;
  *n_out = nout;
  *snum_out = snum;
  return true;
}

// Inclusive AND over lanes 0 .. lane (lanes take all-ones where a move has no source lane).
__device__ __forceinline__ uint32_t wave_incl_and(uint32_t v) {
  v &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, kDppRowShr1, 0xF, 0xF, false);
  v &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, kDppRowShr2, 0xF, 0xF, false);
  v &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, kDppRowShr4, 0xF, 0xF, false);
  v &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, kDppRowShr8, 0xF, 0xF, false);
  v &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, kDppRowBcast15, 0xA, 0xF, false);
  v &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, kDppRowBcast31, 0xC, 0xF, false);
  return v;
}

// v of a wavefront-uniform site s < CS (a chain of selects: registers cannot be indexed at run
// time).  Each step passes through an empty asm: the compiler would otherwise fold the chain into
// an indexed load and move the array to scratch memory, a memory round trip per use.
template <int CS, typename V>
__device__ __forceinline__ V pick_site(const V (&v)[CS], int s) {
  static_assert(sizeof(V) == 4, "one register per lane");
  V x = v[0];
#pragma unroll
  for (int q = 1; q < CS; ++q) {
    x = s == q ? v[q] : x;
    asm volatile("" : "+v"(x));
  }
  return x;
}

// Depth-wise vote of a candidate with at most CS <= 8 sites, in columns: lane i holds depth i,
// and T[s] is site s's column (its continuation token at each depth, -1 from its first depth
// without one on; len[s] leading tokens; every column ends by dmax <= 64).  Same result and
// outputs as vote_run.
//
// Sites are bits of 8-bit masks.  A pass takes the alive site with the longest column as the
// reference r, and each depth lane builds the mask of the sites whose token there equals r's
// (none where r has none): the sites alive at depth i are those alive at d that agree with r at
// every depth d .. i - 1 (an AND scan of that mask over the depth lanes).  At depth i the alive sites with a token vote: g_i of them with r's token, o_i with
// another.  Where g_i > o_i, r's token wins with count g_i whatever the others vote; the first
// depth where it does not (g_i <= o_i), or where the stop rule ends the chain, is found by one
// ballot over the depth lanes.  That depth is voted from scratch on the masks (one count per
// distinct token, stopping when the best count beats every vote not yet counted), the alive
// sites become the winner's, and the next pass starts after it.
template <int CS, typename Beaten>
__device__ __forceinline__ bool vote_columns(const int (&T)[CS], const int (&len)[CS], int c0,
                                             int dmax, int cmin, int* hk, int* hc, int lane,
                                             Beaten&& beaten, int* out, int* n_out,
                                             int* snum_out) {
  static_assert(CS <= 8, "sites as bits of an 8-bit mask");
  (void)hk;
  (void)hc;
  // per depth lane: the sites with a token there
  uint32_t vm = 0;
#pragma unroll
  for (int q = 0; q < CS; ++q) vm |= T[q] >= 0 ? (1u << q) : 0u;
  uint32_t AS = c0 >= 32 ? ~0u : ((1u << c0) - 1u);  // alive sites
  int nout = 0, snum = 0, tokv = -1, clast = c0;
  const int cstop = cmin > 1 ? cmin : 1;  // a depth with fewer votes than this ends the chain
  bool cut = false;
  int d = 0;
  for (int pass = 0; d < dmax && AS != 0; ++pass) {
    if (pass > 0 && beaten(snum + clast * (dmax - nout))) {
      cut = true;
      break;
    }
    // the reference: the first alive site of the longest column
    int rs = 0, rl = -1;
#pragma unroll
    for (int q = 0; q < CS; ++q) {
      const bool better = ((AS >> q) & 1) && len[q] > rl;
      rl = better ? len[q] : rl;
      rs = better ? q : rs;
    }
    const int tref = pick_site<CS>(T, rs);
    uint32_t gr = 0;  // the sites with r's token at this depth
#pragma unroll
    for (int q = 0; q < CS; ++q) gr |= T[q] == tref ? (1u << q) : 0u;
    gr = tref >= 0 ? gr : 0u;
    // alive entering depth i >= d: AS and agreement with r at every depth d .. i - 1 (no scan
    // when every alive site with a token agrees with r at every depth)
    uint32_t alive = AS;
    if (__ballot(lane >= d && lane < dmax && (AS & vm & ~gr) != 0) != 0) {
      const uint32_t incl = wave_incl_and(lane >= d ? gr : ~0u);
      const uint32_t before = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)incl, kDppWaveShr1,
                                                                    0xF, 0xF, false);
      alive = AS & (lane > d ? before : ~0u);
    }
    const uint32_t V = alive & vm;
    const int g = __popc(V & gr), na = __popc(V);
    const int o = na - g;
    const bool in = lane >= d && lane < dmax;
    const bool stop = in && (na < cstop || (g > o && g < cmin));
    const bool cont = in && !stop && g <= o;
    const uint64_t sb = __ballot(stop);
    const uint64_t ev = sb | __ballot(cont);
    const int e = ev ? (int)__builtin_ctzll(ev) : dmax;
    if (e > d) {
      const bool acc = lane >= d && lane < e;
      tokv = acc ? tref : tokv;
      snum += __builtin_amdgcn_readlane(wave_incl_add(acc ? g : 0), 63);
      clast = __builtin_amdgcn_readlane(g, e - 1);
      nout = e;
    }
    if (e >= dmax || ((sb >> e) & 1)) break;
    // depth e from scratch, in scalar registers: the voters and their tokens, then one count per
    // distinct token (the highest count, then the smallest token)
    const uint32_t Ve = (uint32_t)__builtin_amdgcn_readlane((int)V, e);
    int xe[CS];
#pragma unroll
    for (int q = 0; q < CS; ++q) xe[q] = __builtin_amdgcn_readlane(T[q], e);
    uint32_t R = Ve, bgrp = 0;
    int best = -1, btok = 0, rest = __popc(Ve);
    while (R && best <= rest) {
      const int q = __builtin_ctz(R);
      int tok = xe[0];
#pragma unroll
      for (int u = 1; u < CS; ++u) tok = q == u ? xe[u] : tok;
      uint32_t grp = 0;
#pragma unroll
      for (int u = 0; u < CS; ++u) grp |= xe[u] == tok ? (1u << u) : 0u;
      grp &= Ve;
      const int cnt = __popc(grp);
      if (cnt > best || (cnt == best && tok < btok)) {
        best = cnt;
        btok = tok;
        bgrp = grp;
      }
      R &= ~grp;
      rest -= cnt;
    }
    if (best <= 0 || best < cmin) break;
    tokv = lane == e ? btok : tokv;
    snum += best;
    clast = best;
    nout = e + 1;
    AS = bgrp;
    d = e + 1;
  }
  if (cut) {
    *n_out = 0;
    *snum_out = 0;
    return false;
  }
  if (lane < nout) out[lane] = tokv;
  *n_out = nout;
  *snum_out = snum;
  return true;
}

// Columns of a candidate's sites for vote_columns: lane i of T[s] gets the token at depth i of
// site s (s < c0), from its first depth without a token on -1; len[s] its leading tokens.  at(s,
// i) gives the token (or -1) at depth i < dmax of site s; it must read in bounds for every s < CS
// and lane i (its value is dropped where s >= c0 or i >= dmax), so that every site's read is
// issued before any is used.
template <int CS, typename At>
__device__ __forceinline__ void columns_cut(int (&T)[CS], int (&len)[CS], int c0, int dmax,
                                            int lane, At&& at) {
#pragma unroll
  for (int s = 0; s < CS; ++s) T[s] = at(s, lane);
#pragma unroll
  for (int s = 0; s < CS; ++s) T[s] = s < c0 && lane < dmax ? T[s] : -1;
#pragma unroll
  for (int s = 0; s < CS; ++s) {
    const uint64_t ok = __ballot(T[s] >= 0);
    len[s] = (int)__builtin_ctzll(~ok);
    T[s] = lane < len[s] ? T[s] : -1;
  }
}

// Windows of a corpus candidate: c0 sites (logical corpus positions, relative to the oldest live
// one, in gs), continuation tokens loaded all at once (each address is a live snapshot position
// or a ring slot, so always in bounds) and cut at each site's first separator.
template <int KMAX>
__device__ __forceinline__ void corpus_windows(const ProposeArgs& a, const Req& r, const int* gs,
                                               int c0, int cap, int lane, int (&w0)[KMAX],
                                               int (&w1)[KMAX], int* len0_out, int* len1_out) {
  const int act = r.act;
  const int32_t* text = act == 0 ? a.idx[0].text : (act == 1 ? a.idx[1].text : nullptr);
  const long long ss = r.snap_start, sn = r.snap_n;
  const int s0 = lane, s1 = lane + 64;
  // (both slots are read, together: a candidate's list holds kMaxM = 128 of them)
  const int g0 = gs[s0], g1 = gs[s1];
  const long long q0 = r.tail_w + (s0 < c0 ? g0 : 0), q1 = r.tail_w + (s1 < c0 ? g1 : 0);
  bool live0 = s0 < c0, live1 = s1 < c0;
  // offsets into the snapshot text (an unused slot reads its first token)
  const long long o0 = live0 ? q0 - ss : 0, o1 = live1 ? q1 - ss : 0;
  const bool in0 = text != nullptr && o0 >= 0 && o0 < sn;
  const bool in1 = text != nullptr && o1 >= 0 && o1 < sn;
  if (__ballot(!(in0 && in1)) == 0) {
    // every site inside the snapshot, whose text ends with a separator: a window runs at most to
    // it, and reads on past the text's end unclamped (the buffer holds kTextSlack >= KMAX more
    // positions), so that its loads share one address
    static_assert(KMAX <= kTextSlack, "windows inside the text buffer");
    const int32_t* t0p = text + o0;
    const int32_t* t1p = text + o1;
    if (c0 > 64) {  // (wavefront-uniform) a second site per lane
#pragma unroll
      for (int d = 0; d < KMAX; ++d) {
        w0[d] = t0p[d];
        w1[d] = t1p[d];
      }
    } else {
#pragma unroll
      for (int d = 0; d < KMAX; ++d) {
        w0[d] = t0p[d];
        w1[d] = -1;
      }
    }
  } else {
    const int rcap = (int)a.ring_cap;
    int r0 = (int)(q0 % a.ring_cap), r1 = (int)(q1 % a.ring_cap);
#pragma unroll
    for (int d = 0; d < KMAX; ++d) {
      w0[d] = *corpus_ptr(a, text, ss, sn, q0 + d, r0);
      w1[d] = *corpus_ptr(a, text, ss, sn, q1 + d, r1);
      r0 = ring_next(r0, rcap);
      r1 = ring_next(r1, rcap);
    }
  }
  int len0 = 0, len1 = 0;
#pragma unroll
  for (int d = 0; d < KMAX; ++d) {
    live0 = live0 && d < cap && w0[d] >= 0;
    live1 = live1 && d < cap && w1[d] >= 0;
    w0[d] = live0 ? w0[d] : -1;
    w1[d] = live1 ? w1[d] : -1;
    len0 += live0 ? 1 : 0;
    len1 += live1 ? 1 : 0;
  }
  *len0_out = len0;
  *len1_out = len1;
}

// The corpus wavefront of the fast path, first part, run while the other wavefronts stage the
// context: the tail (lane x holds ctx[L-1-x]) into LDS, the three n-gram probes, the heads of
// the three position-ordered groups into LDS, and the backward extension of the live 4-gram
// occurrences into a length histogram (lengths of the first kMaxM kept in LDS).
__device__ __forceinline__ void corpus_wave_probe(const ProposeArgs& a, const Req& r, Smem& sm,
                                                  int tailv, int lane) {
  const int Lcap = r.Lcap, M = a.M;
  if (lane < Lcap) sm.gtail[lane] = tailv;
  for (int i = lane; i <= kMaxD; i += 64) sm.ghist[i] = 0;
  wave_sync();
  const View ib = view_of(a, r.act, r.ht_mask);
  const long long dead_below = r.tail_w - r.snap_start;
  if (lane < kNG)
    probe_lane(ib, sm.gtail, Lcap, dead_below, lane, &sm.g_off[lane], &sm.g_live[lane]);
  wave_sync();
  // the first M entries of all three groups in one round trip, two per lane
  int ns[kNG], hv[kNG][2];
#pragma unroll
  for (int g = 0; g < kNG; ++g) {
    const int32_t* pl = (g == 0 ? ib.pl0 : (g == 1 ? ib.pl1 : ib.pl2)) + sm.g_off[g];
    ns[g] = sm.g_live[g] < M ? sm.g_live[g] : M;
#pragma unroll
    for (int h = 0; h < 2; ++h) hv[g][h] = lane + 64 * h < ns[g] ? pl[lane + 64 * h] : 0;
  }
#pragma unroll
  for (int g = 0; g < kNG; ++g)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (lane + 64 * h < ns[g]) sm.gpl[g][lane + 64 * h] = hv[g][h];
  const int live4 = sm.g_live[2];
  const bool hot = Lcap >= 5 && live4 > kHotGroup && dead_below <= 0;
  if (lane == 0) sm.ghot = hot;
  if (hot) {
    hot_bounds(ib, sm.gtail, Lcap, (int)r.snap_n, lane, sm.hsup, sm.hlo, sm.hoff, sm.hcnt);
  } else if (Lcap >= 5 && live4 > 0) {
    // two occurrences per lane per round (the first round's positions are loaded already)
    const int32_t* pl4 = ib.pl2 + sm.g_off[2];
    for (int base = 0; base < live4; base += 128) {
      const int x0 = base + lane, x1 = x0 + 64;
      const bool q0 = x0 < live4, q1 = x1 < live4;
      const int i0 = x0 < ns[2] ? hv[2][0] : (q0 ? pl4[x0] : 0);
      const int i1 = x1 < ns[2] ? hv[2][1] : (q1 ? pl4[x1] : 0);
      int m0, m1;
      extend4_pair(ib.text, sm.gtail, i0, q0, i1, q1, Lcap, &m0, &m1);
      if (q0 && x0 < kMaxM) {
        sm.gm4[x0] = m0;
        sm.gpl[2][x0] = i0;
      }
      if (q1 && x1 < kMaxM) {
        sm.gm4[x1] = m1;
        sm.gpl[2][x1] = i1;
      }
      if (q0 && m0 >= 5) atomicAdd(&sm.ghist[m0], 1);
      if (q1 && m1 >= 5) atomicAdd(&sm.ghist[m1], 1);
    }
  }
}

// Second part: the corpus ladder (lane l - 1 holds the support of length l) and the earliest
// sites of each level.
__device__ __forceinline__ void corpus_wave_sites(const ProposeArgs& a, const Req& r, Smem& sm,
                                                  int lane) {
  const int Lcap = r.Lcap, nb = a.nb, M = a.M;
  const int sbase = (int)(r.snap_start - r.tail_w);  // snapshot index -> site coordinate
  wave_sync();
  // support of length v = lane + 1 (lengths up to 64 on 64 lanes): the live v-gram group for
  // v <= 4, else the extensions reaching v
  const int v = lane + 1;
  const bool hot = sm.ghot;
  const int gh = (v >= 5 && v <= Lcap) ? sm.ghist[v] : 0;
  const int gin = wave_incl_add(gh);
  const int gsuf = __builtin_amdgcn_readlane(gin, 63) - gin + gh;
  const int hsup = (v >= 5 && v <= Lcap) ? sm.hsup[v] : 0;
  const int sup_l = v >= 2 && v <= 4 ? sm.g_live[v - 2] : (hot ? hsup : gsuf);
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
    int* gs = sm.gsites[ti];
    if (l <= 4) {
      const int g = l - 2;
      const int ns = sup < M ? sup : M;
      for (int x = lane; x < ns; x += 64) gs[x] = sm.gpl[g][x] + l + sbase;
    } else if (hot) {
      const View ib = view_of(a, r.act, r.ht_mask);
      const int got = hot_sites(ib, sm, sm.gtail, l, M, (int)r.snap_n, sbase,
                                ib.pl2 + sm.g_off[2], sm.g_live[2], gs, lane);
      if (lane == 0 && got < (sup < M ? sup : M)) sm.cand_c0[ci] = got;
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
        if (q && rk < M) gs[rk] = i + 4 + sbase;
        run += __popcll(bal);
      }
      // the vote reads exactly the sites written
      if (lane == 0 && run < (sup < M ? sup : M)) sm.cand_c0[ci] = run;
    }
  }
  wave_sync();
}

// Dynamic LDS of one request:
//   staged:    [context ints | hit bit words | two-token bit words | hit positions (u16) |
//               hit lengths (u8) | vote tables]
//   streaming: the same without the context.
// With a corpus, the region from the hit positions on also holds the delta scan's occurrence
// records (after the local sites are gathered), at least kDeltaMinRecs per wavefront.
constexpr int kVoteBytes = 2 * kVoteSlots * 4;  // one voter's keys and counts
// context ints, then 64 spare slots that absorb the staging stores of lanes past the row end
__host__ __device__ inline int ctx_ints(int S, int T) { return ((S + T + 4 + 3) & ~3) + 64; }
__host__ __device__ inline int ctx_spare(int S, int T) { return ctx_ints(S, T) - 64; }
// one bit word per 64 end positions (J <= S + T - 1), plus one
__host__ __device__ inline int bit_words(int S, int T) { return (S + T + 63) / 64 + 1; }
// Hit-list entries: wavefront w owns the entries of its end positions [cbeg, cend), from entry
// cbeg on (a list never holds more entries than its chunk has positions); J <= S + T - 1.
__host__ __device__ inline int hit_cap(int S, int T) { return (S + T + 63) & ~63; }
__host__ __device__ inline size_t bits_offset(bool staged, int S, int T) {
  return staged ? (size_t)4 * ctx_ints(S, T) : 0;
}
__host__ __device__ inline size_t bits2_offset(bool staged, int S, int T) {
  return bits_offset(staged, S, T) + (size_t)8 * bit_words(S, T);
}
__host__ __device__ inline size_t hpos_offset(bool staged, int S, int T) {
  return bits2_offset(staged, S, T) + (size_t)8 * bit_words(S, T);
}
__host__ __device__ inline size_t hmb_offset(bool staged, int S, int T) {
  return hpos_offset(staged, S, T) + (size_t)2 * hit_cap(S, T);
}
constexpr int kDeltaMinRecs = 256;
__host__ __device__ inline size_t vote_offset(bool staged, int S, int T, bool corpus) {
  size_t b = hmb_offset(staged, S, T) + (size_t)hit_cap(S, T);
  if (corpus) {
    const size_t need = hpos_offset(staged, S, T) + (size_t)4 * NW * kDeltaMinRecs;
    if (b < need) b = need;
  }
  return (b + 15) & ~(size_t)15;
}
// one vote table per voter: wavefronts 0 .. 2 nb - 1
__host__ __device__ inline size_t dyn_bytes(bool staged, int S, int T, bool corpus, int nb) {
  return vote_offset(staged, S, T, corpus) + (size_t)kVoteBytes * 2 * nb;
}

// 64-position words per screening group: 1536 positions (1024 with 32-token windows, whose
// vote needs the registers)
template <int KMAX>
constexpr int screen_loads() {
  return KMAX >= 32 ? 16 : 24;
}

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


// Local step 1 for one wavefront's chunk [cbeg, cend) of end positions, row part.  The row part
// [cbeg, rend), rend = min(cend, n), is read with bounds-checked buffer loads (every load of a
// lane in flight; lanes on consecutive positions, so each load instruction is one coalesced
// 256-byte run) and staged in LDS when STAGED.  For every 64 positions two ballots are kept as
// bit words: the end positions whose token is the last context token t0 (match length >= 1),
// and of those the ones whose previous token is the second-to-last context token t1 (length
// >= 2; the previous token is the next lower lane's, lane 0 taking the previous word's lane 63
// or, for the first word, prev0 = ctx[cbeg - 1]).  Word i covers positions cbeg + 64 i ...
// screen_issue loads the first group of positions (issued before the workgroup's set-up
// barrier, so the barrier waits under their latency); stage_screen consumes it and loads the
// rest.  Returns the number of row words; *nbits gets the number of set bits of the first kind.
struct ScreenSrc {
  __amdgpu_buffer_rsrc_t rs;
  int rend;
};

template <int G>
__device__ __forceinline__ ScreenSrc screen_issue(const int32_t* row, int n, int cbeg, int cend,
                                                  int lane, int (&v)[G]) {
  ScreenSrc src;
  src.rend = __builtin_amdgcn_readfirstlane(cend < n ? cend : n);
  src.rs = __builtin_amdgcn_make_buffer_rsrc((void*)row, (short)0,
                                             (src.rend > 0 ? src.rend : 0) * 4, kBufferWord3);
  // unconditional: a load at or past rend is out of the buffer's range and returns 0 without
  // touching memory (every load of an empty chunk is)
  const int vo = (cbeg + lane) * 4;
#pragma unroll
  for (int i = 0; i < G; ++i)
    v[i] = __builtin_amdgcn_raw_buffer_load_b32(src.rs, vo + 256 * i, 0, 0);
  return src;
}

template <bool STAGED, int G>
__device__ __forceinline__ int stage_screen(int* ctxs, int spare, uint64_t* b1w, uint64_t* b2w,
                                            const ScreenSrc& src, int (&v)[G],
                                            int cbeg, int t0, int t1, int prev0, int lane,
                                            int* nbits) {
  const int rend = src.rend;
  int nw = 0, cnt = 0;
  int carry = prev0;  // the token before the group's first position
  for (int g0 = cbeg; g0 < rend; g0 += 64 * G) {
    const int ne = (rend - g0 + 63) >> 6 < G ? (rend - g0 + 63) >> 6 : G;
    const int nfull = (rend - g0) >> 6;  // elements whose 64 positions all lie below rend
    uint32_t a1 = 0, a2 = 0;
    static_for<0, G>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (i < ne) {
        const int x = g0 + 64 * i + lane;
        // previous token: the lower lane's, lane 0 the previous element's lane 63
        const int old = i == 0 ? carry
                               : __builtin_amdgcn_update_dpp(0, v[i > 0 ? i - 1 : 0],
                                                             kDppWaveRor1, 0xF, 0xF, false);
        const int prv = __builtin_amdgcn_update_dpp(old, v[i], kDppWaveShr1, 0xF, 0xF, false);
        uint64_t w1;
        if (i < nfull) {
          if (STAGED) ctxs[x] = v[i];
          w1 = __ballot(v[i] == t0);
        } else {
          const int rem = rend - g0 - 64 * i;  // 1..63
          if (STAGED) ctxs[x < rend ? x : spare + lane] = v[i];
          w1 = __ballot(v[i] == t0) & ((1ull << rem) - 1ull);
        }
        const uint64_t w2 = w1 & __ballot(prv == t1);
        cnt += __popcll(w1);
        a1 = put_ballot<(2 * i) & 62>(a1, w1);
        a2 = put_ballot<(2 * i) & 62>(a2, w2);
      }
    });
    carry = __builtin_amdgcn_readlane(v[G - 1], 63);
    if (lane < 2 * ne) {
      reinterpret_cast<uint32_t*>(b1w + nw)[lane] = a1;
      reinterpret_cast<uint32_t*>(b2w + nw)[lane] = a2;
    }
    nw += ne;
    const int g1 = g0 + 64 * G;
    if (g1 < rend) {
      const int vo = (g1 + lane) * 4;
#pragma unroll
      for (int i = 0; i < G; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b32(src.rs, vo + 256 * i, 0, 0);
    }
  }
  *nbits = cnt;
  return nw;
}

// Positions of the set bits of nw words (word i based at base0 + 64 i), in order, into out[];
// returns their number.  Every lane of the wavefront takes part, on a 16-bit quarter of a word
// each, so that a lane walks at most 16 bits.
__device__ __forceinline__ int bits_to_list(const uint64_t* w, int nw, int base0, uint16_t* out,
                                            int lane) {
  int cnt = 0;
  const int nq = 4 * nw;
  for (int q0 = 0; q0 < nq; q0 += 64) {
    const int q = q0 + lane;
    const int wi = q >> 2, part = q & 3;
    const uint64_t wd = wi < nw ? w[wi] : 0ull;
    uint32_t piece = (uint32_t)(wd >> (16 * part)) & 0xFFFFu;
    const int base = base0 + 64 * wi + 16 * part;
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

// Local step 2 for one wavefront's chunk, run as soon as its own screen is done: the two-token
// hits listed in order and their backward match lengths against the tail.
// Offsets 2 .. kTailRegs + 1 of every listed hit are read at once and compared with tail values
// in scalar registers; longer matches (D > kTailRegs + 2) go on four offsets per round.  Lengths
// go to hmb[] and the wavefront's histogram; returns the number of two-token hits.
constexpr int kTailRegs = 24;
template <bool STAGED>
__device__ __forceinline__ int list_extend(const int* ctxs, const uint64_t* b2w, int nwt,
                                           int cbeg, uint16_t* hpos, uint8_t* hmb, int tailv,
                                           const int* tail, int D, int* whist, const int32_t* row,
                                           const int32_t* smp, int n, int lane) {
  const int nhit = bits_to_list(b2w, nwt, cbeg, hpos, lane);
  wave_sync();
  int tq[kTailRegs];
#pragma unroll
  for (int x = 0; x < kTailRegs; ++x) tq[x] = __builtin_amdgcn_readlane(tailv, 2 + x);
  const bool short_d = D <= 2 + kTailRegs;
  for (int e0 = 0; e0 < nhit; e0 += 64) {
    const int e = e0 + lane;
    const bool ok = e < nhit;
    const int j = ok ? hpos[e] : 0;
    const int lim = D < j + 1 ? D : j + 1;
    int m = 2;
    if (ok && lim > 2) {
      // offsets 2 .. 5 first (most hits end there), the other kTailRegs - 4 only when some lane
      // of the wavefront still matches
      int c[kTailRegs];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int o = 2 + q;
        const int at = o < lim ? j - o : 0;
        c[q] = STAGED ? ctxs[at] : ctx_at(row, smp, n, at);
      }
      bool go = true;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        go = go && 2 + q < lim && c[q] == tq[q];
        m += go ? 1 : 0;
      }
      if (__ballot(go && lim > 6) != 0) {
#pragma unroll
        for (int q = 4; q < kTailRegs; ++q) {
          const int o = 2 + q;
          const int at = o < lim ? j - o : 0;
          c[q] = STAGED ? ctxs[at] : ctx_at(row, smp, n, at);
        }
#pragma unroll
        for (int q = 4; q < kTailRegs; ++q) {
          go = go && 2 + q < lim && c[q] == tq[q];
          m += go ? 1 : 0;
        }
      } else {
        go = false;
      }
      if (go && !short_d) {
        // match lengths above kTailRegs + 2 (max_tree_depth up to 64)
        for (int o0 = 2 + kTailRegs; o0 < lim; o0 += 4) {
          int cc[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int at = o0 + q < lim ? j - o0 - q : 0;
            cc[q] = STAGED ? ctxs[at] : ctx_at(row, smp, n, at);
          }
          bool stop = false;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (!stop) {
              if (o0 + q < lim && cc[q] == tail[o0 + q]) ++m;
              else stop = true;
            }
          }
          if (stop) break;
        }
      }
    }
    if (ok) hmb[e] = (uint8_t)m;
    if (ok && m > 2) atomicAdd(&whist[m], 1);
  }
  return nhit;
}

// Local ladder rung t and, when it is the first rung of its length, its earliest continuation
// sites (run by wavefront t once every worker has published its counts, bit words and two-token
// lists).  Lane v - 1 of cg holds the end positions of length >= v.
__device__ __forceinline__ void local_candidate(const ProposeArgs& a, Smem& sm, int NWW, int maxl,
                                                int J, const uint64_t* bits,
                                                const uint16_t* hpos_all, const uint8_t* hmb_all,
                                                int t, int lane) {
  const int M = a.M;
  const int mins = a.min_self > 1 ? a.min_self : 1;
  int cg = 0;
  for (int w = 0; w < NWW; ++w) cg += sm.wsuf[w][lane + 1];
  int l = 0, sup = 0, src = 0, prev_l = -1, prev_src = -1;
  for (int ti = 0; ti <= t; ++ti) {
    const uint64_t ok = __ballot(lane + 1 <= maxl && cg >= ti + 1);
    l = ok ? 64 - __builtin_clzll(ok) : 0;
    sup = l ? __builtin_amdgcn_readlane(cg, l - 1) : 0;
    src = (ti > 0 && l == prev_l) ? prev_src : ti;
    prev_l = l;
    prev_src = src;
  }
  const int c0 = sup < M ? sup : M;
  if (lane == 0) {
    sm.cand_len[t] = l;
    sm.cand_sup[t] = sup;
    sm.cand_valid[t] = l >= mins;
    sm.cand_c0[t] = c0;
    sm.cand_src[t] = src;
  }
  if (t == 0) {
    // (the longest-match mode's corpus voter waits for candidate 0's length)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) __hip_atomic_store(&sm.lready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  if (l < mins || src != t) return;
  int* ls = sm.lsites[t];
  if (l == 1) {
    // every end position whose token is the last context token: the set bits of the bit words
    // (a whole word per lane: the earliest c0 often lie far apart, and a round per 64 words
    // instead of per 16 makes up for the longer walk of a dense word, which stops at c0)
    const int nwords = (J + 63) >> 6;
    int found = 0;
    for (int w0 = 0; found < c0 && w0 < nwords; w0 += 64) {
      const int wi = w0 + lane;
      uint64_t wd = wi < nwords ? bits[wi] : 0ull;
      const int c = __popcll(wd);
      const int incl = wave_incl_add(c);
      int at = found + incl - c;
      while (wd && at < c0) {
        ls[at++] = 64 * wi + __builtin_ctzll(wd) + 1;
        wd &= wd - 1;
      }
      found += __builtin_amdgcn_readlane(incl, 63);
    }
    // the vote reads exactly the sites written: a count that disagreed with the bit words
    // could otherwise leave site slots unwritten
    if (lane == 0 && found < c0) sm.cand_c0[t] = found;
    return;
  }
  // the two-token lists of the workers that hold an end position of length >= l, concatenated
  // in wavefront (so position) order, filtered by length
  const int q = lane < NWW ? sm.wsuf[lane][l] : 0;
  const int c2 = lane < NWW ? sm.wsuf[lane][2] : 0;
  const int sc = q > 0 ? c2 : 0;
  const int inc = wave_incl_add(sc);
  const int total = __builtin_amdgcn_readlane(inc, 63);
  if (lane < NW) sm.vex[t][lane] = inc - sc;
  wave_sync();
  const uint64_t below = lanes_below(lane);
  int found = 0;
  for (int base = 0; base < total && found < c0; base += 64) {
    const int e = base + lane;
    int ex = 0, bs = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int xw = sm.vex[t][w];
      if (w < NWW && e >= xw) {
        ex = xw;
        bs = sm.wbeg[w];
      }
    }
    const bool in = e < total;
    const int x = bs + e - ex;
    const int j = in ? hpos_all[x] : 0;
    const int m = in ? hmb_all[x] : 0;
    const bool qq = in && m >= l;
    const uint64_t bal = __ballot(qq);
    const int rk = found + __popcll(bal & below);
    if (qq && rk < c0) ls[rk] = j + 1;
    found += __popcll(bal);
  }
  if (lane == 0 && found < c0) sm.cand_c0[t] = found;  // as above
}

// Windows of local candidate t, from the staged or streamed context.  Every load is issued
// unconditionally at a position clamped into [0, L) (all of which are staged, or readable from
// the row and the sampled ids), and what lies outside a window is set to -1 afterwards.  A
// window holds min(cap, L - p) tokens and ends early at a negative id.
template <int KMAX, bool STAGED>
__device__ __forceinline__ void local_windows(const Smem& sm, const int* ctxs, const int32_t* row,
                                              const int32_t* smp, int n, int L, int t, int c0,
                                              int cap, int lane, int (&w0)[KMAX],
                                              int (&w1)[KMAX], int* len0_out, int* len1_out) {
  const int* ls = sm.lsites[t];
  const int s0 = lane, s1 = lane + 64;
  const int l0 = ls[s0], l1 = ls[s1];  // (read together: the list holds kMaxM = 128 slots)
  const int p0 = s0 < c0 ? l0 : 0, p1 = s1 < c0 ? l1 : 0;
  const int cap0 = cap < KMAX ? cap : KMAX;
  const int e0 = s0 < c0 ? (L - p0 < cap0 ? L - p0 : cap0) : 0;
  const int e1 = s1 < c0 ? (L - p1 < cap0 ? L - p1 : cap0) : 0;
  // staged, a window reads on past L (the stage holds L + 64 positions; what lies past L is cut
  // below), so that its reads share one address; from HBM it stops at the last context token
  auto at = [&](int p, int d) {
    if (STAGED) return ctxs[p + d];
    const int x = p + d < L ? p + d : L - 1;
    return *(x < n ? row + x : smp + (x - n));
  };
  if (c0 > 64) {  // (wavefront-uniform) a second site per lane
#pragma unroll
    for (int d = 0; d < KMAX; ++d) {
      w0[d] = at(p0, d);
      w1[d] = at(p1, d);
    }
  } else {
#pragma unroll
    for (int d = 0; d < KMAX; ++d) {
      w0[d] = at(p0, d);
      w1[d] = -1;
    }
  }
  // a site stops voting for good at its first depth without a token (a negative id counts as
  // none), so its window ends there
  bool live0 = true, live1 = true;
  int len0 = 0, len1 = 0;
#pragma unroll
  for (int d = 0; d < KMAX; ++d) {
    live0 = live0 && d < e0 && w0[d] >= 0;
    live1 = live1 && d < e1 && w1[d] >= 0;
    w0[d] = live0 ? w0[d] : -1;
    w1[d] = live1 ? w1[d] : -1;
    len0 += live0 ? 1 : 0;
    len1 += live1 ? 1 : 0;
  }
  *len0_out = len0;
  *len1_out = len1;
}

#if SFX_PHASE_TRACE
#define PHASE(p)                                                                 \
  do {                                                                           \
    if (a.trace && lane == 0) sm.ts[wid][p] = __builtin_amdgcn_s_memtime();      \
  } while (0)
#define PHASE_FLUSH()                                                            \
  do {                                                                           \
    if (a.trace && lane < kTracePhases)                                          \
      a.trace[((size_t)b * NW + wid) * kTracePhases + lane] = sm.ts[wid][lane];  \
  } while (0)
#else
#define PHASE(p) \
  do {           \
  } while (0)
#define PHASE_FLUSH() \
  do {                \
  } while (0)
#endif

// GENERAL: whether the general path (section 2) is compiled in.  Without it the kernel is for
// calls that the host knows see no delta: no document ingested since the live snapshot was
// taken.  Then the general path would only run without a live snapshot, and it finds no corpus
// candidate there, so leaving it out changes no result; its code (about a quarter of the
// kernel's) is then out of the instruction cache and the register allocation.
template <int KMAX, bool STAGED, bool GENERAL>
__global__ __launch_bounds__(NT) void propose_kernel(ProposeArgs a) {
  extern __shared__ int4 dyn4[];
  unsigned char* dyn = reinterpret_cast<unsigned char*>(dyn4);
  int* ctxs = reinterpret_cast<int*>(dyn);  // the context (STAGED only)
  uint64_t* bits_all = reinterpret_cast<uint64_t*>(dyn + bits_offset(STAGED, a.S, a.T));
  uint64_t* bits2_all = reinterpret_cast<uint64_t*>(dyn + bits2_offset(STAGED, a.S, a.T));
  uint16_t* hpos_all = reinterpret_cast<uint16_t*>(dyn + hpos_offset(STAGED, a.S, a.T));
  uint8_t* hmb_all = dyn + hmb_offset(STAGED, a.S, a.T);
  int* vote_all = reinterpret_cast<int*>(dyn + vote_offset(STAGED, a.S, a.T, a.ctl != nullptr));
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform (SGPR)
  const int b = blockIdx.x;
  const int32_t* row = a.tok + (int64_t)b * a.S;
  const int32_t* smp = a.samp + (int64_t)b * a.T;
  const int D = a.D, nb = a.nb, M = a.M;
#if SFX_PHASE_TRACE
  if (lane < kTracePhases) sm.ts[wid][lane] = 0;
#endif
  PHASE(0);

  // Set-up, first round of loads, all issued together: the row length, the sampled ids (lane
  // i < T holds sampled[i]), the control block (lane i holds its word i) and the two per-call
  // tables (thread x holds entry x of each).
  constexpr int kCtlWords = (int)(sizeof(Ctl) / 4);
  static_assert(kCtlWords <= 64 && sizeof(Ctl) % 8 == 0, "control block in one wavefront");
  const int nraw = a.ntns[b];
  // the request's delta group, read now so that it has landed when the delta walk needs it
  const int pgroup = GENERAL && a.pair_group != nullptr ? a.pair_group[b] : -1;
  const int sl = lane < a.T ? smp[lane] : -1;
  const int cw = a.ctl != nullptr && lane < kCtlWords
                     ? reinterpret_cast<const int*>(a.ctl)[lane] : 0;
  const int capv = tid <= kMaxD ? a.cap_of_len[tid] : 0;
  const int minv = tid <= kMaxM ? a.min_count[tid] : 0;
  // The first kPrefetchTokens of the row, one 128-byte line per thread, start their way from
  // HBM now, while the set-up round trip runs and HBM is otherwise idle; the screen reads them
  // again from L2.  (Past the row's capacity a load reads nothing; a row shorter than this
  // fetches at most 8 KB it does not use.)  The value is kept in LDS at the end, so the load
  // stays.
  const int pf_ints = a.S < kPrefetchTokens ? a.S : kPrefetchTokens;
  const __amdgpu_buffer_rsrc_t pf_rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)row, (short)0, pf_ints * 4, kBufferWord3);
  const int pf = __builtin_amdgcn_raw_buffer_load_b32(pf_rs, tid * 128, 0, 0);

  Req r;
  {
    const int n = nraw < 0 ? 0 : (nraw > a.S ? a.S : nraw);
    // the leading sampled ids that are tokens (lanes from T on hold -1)
    const int t = __builtin_ctzll(~__ballot(sl >= 0));
    r.n = n;
    r.t = t;
    r.t0 = t > 0 ? __builtin_amdgcn_readlane(sl, t - 1) : -1;
    r.L = n + t;
    r.J = r.L > 0 ? r.L - 1 : 0;
    r.Lcap = D < r.L ? D : r.L;
    r.has = a.ctl != nullptr;
    r.act = -1;
    r.fast = false;
    r.delta = false;
    r.snap_start = r.snap_n = r.tail_w = r.delta_lo = r.delta_hi = 0;
    r.ht_mask = 0;
    if (r.has) {
      auto w32 = [&](size_t off) { return __builtin_amdgcn_readlane(cw, (int)(off / 4)); };
      auto w64 = [&](size_t off) {
        return (long long)(((uint64_t)(uint32_t)w32(off + 4) << 32) | (uint32_t)w32(off));
      };
      r.act = w32(offsetof(Ctl, active));
      r.tail_w = w64(offsetof(Ctl, tail));
      r.delta_hi = w64(offsetof(Ctl, head));
      if (r.act >= 0) {
        const int i = r.act == 0 ? 0 : 1;
        r.ht_mask = (uint32_t)w32(offsetof(Ctl, ht_mask) + 4 * i);
        r.snap_start = w64(offsetof(Ctl, snap_start) + 8 * i);
        const long long se = w64(offsetof(Ctl, snap_end) + 8 * i);
        r.snap_n = se - r.snap_start;
        r.delta_lo = se > r.tail_w ? se : r.tail_w;
      } else {
        r.delta_lo = r.tail_w;
      }
      r.delta = r.delta_hi - r.delta_lo > 1;
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
  PHASE(1);
  // LDS set-up (the tables' loads have landed with the row length's)
  for (int i = tid; i < NW * (kMaxD + 2); i += NT) (&sm.wsuf[0][0])[i] = 0;
  if (tid < 2 * kMaxNB) {
    sm.cand_valid[tid] = 0;
    sm.cand_done[tid] = 0;
  }
  if (tid == 0) {
    sm.wbar = 0;
    sm.gready = 0;
    sm.lready = 0;
  }
  if (tid <= kMaxD) sm.cap_tab[tid] = (uint8_t)capv;
  if (tid <= kMaxM) sm.min_tab[tid] = (uint8_t)minv;
  // every site slot holds a valid position before any is written (a site read past a list's
  // end can then only name a real context or corpus position)
  static_assert(kMaxNB * kMaxM <= NT, "one site slot per thread");
  (&sm.lsites[0][0])[tid] = 1;
  (&sm.gsites[0][0])[tid] = 0;

  // Second round of loads, in flight across the set-up barrier: the tail (lane x holds
  // ctx[L-1-x]), and for a worker the first group of its chunk, the 64 positions before the
  // chunk (the extension of hits near its start reads them; lane 63 holds the token before the
  // chunk) and the sampled ids it stages.
  //
  // Wavefront w < NWW owns end positions [cbeg, cend): it stages them (STAGED) and marks the
  // ones whose token equals the last context token.  The ranges are runs of 64 positions in
  // wavefront order, sized by the wavefront's age on its SIMD (wavefront w is the (w / 4)-th
  // on SIMD w % 4): a SIMD issues for its oldest ready wavefront first, so its younger ones
  // get fewer positions and every worker reaches the barrier at about the same time.
  const int NWW = fast ? NW - 1 : NW;
  const bool cwave = fast && wid == GW;  // the corpus wavefront of the fast path
  const int tailv = lane < Lcap ? ctx_at(row, smp, n, L - 1 - lane) : -1;
  int cbeg = 0, cend = 0;
  if (!cwave) {
    const int nch = (J + 63) >> 6;
    cbeg = 64 * (fast ? first_run<NW - 1>(nch, wid) : first_run<NW>(nch, wid));
    cend = wid + 1 == NWW
               ? J
               : 64 * (fast ? first_run<NW - 1>(nch, wid + 1) : first_run<NW>(nch, wid + 1));
    cbeg = cbeg < J ? cbeg : J;
    cend = cend < J ? cend : J;
  }
  const int hx = cbeg - 64 + lane;
  const bool hld = !cwave && cbeg < cend && hx >= 0 && (STAGED || lane == 63);
  const int halo = hld ? ctx_at(row, smp, n, hx) : -1;
  constexpr int G = screen_loads<KMAX>();
  int sv[G];
  const ScreenSrc ssrc = screen_issue<G>(row, n, cbeg, cwave ? cbeg : cend, lane, sv);
  __syncthreads();

  // ---------------------------------------------------------------- 1. local match
  if (cwave) {
    corpus_wave_probe(a, r, sm, tailv, lane);
    PHASE(2);
    if (!r.delta) {
      corpus_wave_sites(a, r, sm, lane);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (lane == 0) __hip_atomic_store(&sm.gready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      PHASE(3);
    }
  } else {
    // (the last worker stages the sampled ids in any case: windows reach the last context token)
    const bool son = STAGED && lane < t && (wid == NWW - 1 || (cbeg < cend && cend > n));
    uint64_t* b1w = bits_all + (cbeg >> 6);
    uint64_t* b2w = bits2_all + (cbeg >> 6);
    // the second-to-last context token (compared as it is, like every context token) and the
    // token before the chunk
    const bool has_t1 = Lcap >= 2;
    const int t1 = has_t1 ? __builtin_amdgcn_readlane(tailv, 1) : -1;
    const int prev0 = __builtin_amdgcn_readlane(halo, 63);
    int c1 = 0;
    const int nwr = stage_screen<STAGED, G>(ctxs, ctx_spare(a.S, a.T), b1w, b2w, ssrc, sv, cbeg,
                                         r.t0, t1, prev0, lane, &c1);
    if (STAGED && hld) ctxs[hx] = halo;
    if (son) ctxs[n + lane] = sl;
    int nwt = nwr;
    if (cend > n && cend > cbeg) {
      // end positions among the sampled ids (at most T - 1, after every row position): their
      // bits join the words of the row (positions sb ..).  A wavefront with an empty chunk
      // (cbeg == cend, short rows) owns no word and writes none.
      const int sb = cbeg > n ? cbeg : n;
      const int x = sb + lane;
      const bool in = x < cend;
      // sampled id x - n (lanes from T on hold -1; x - n < T - 1 for every lane in range)
      const int sx = __builtin_amdgcn_ds_bpermute(4 * (in ? x - n : 63), sl);
      const uint64_t s1 = __ballot(in && sx == r.t0);
      const int pvx = in && x >= 1 ? ctx_at(row, smp, n, x - 1) : -1;
      const uint64_t s2 = s1 & __ballot(pvx == t1);
      c1 += __popcll(s1);
      const int sw = (sb >> 6) - (cbeg >> 6), sh = sb & 63;
      if (lane == 0) {
        const uint64_t lo = s1 << sh, hi = sh ? s1 >> (64 - sh) : 0ull;
        const uint64_t lo2 = s2 << sh, hi2 = sh ? s2 >> (64 - sh) : 0ull;
        b1w[sw] = (sw < nwr ? b1w[sw] : 0ull) | lo;
        b2w[sw] = (sw < nwr ? b2w[sw] : 0ull) | lo2;
        if (sh && ((cend - 1) >> 6) > (sb >> 6)) {
          b1w[sw + 1] = hi;
          b2w[sw + 1] = hi2;
        }
      }
      nwt = ((cend + 63) >> 6) - (cbeg >> 6);
    }
    wave_sync();
    PHASE(2);
    // every worker writes the same tail values (its longest matches read them back)
    if (lane < Lcap) sm.tail[lane] = tailv;
    if (lane == 0) sm.wbeg[wid] = cbeg;
    // two-token hits and their match lengths
    int c2 = 0;
    if (has_t1 && nwt > 0) {
      c2 = list_extend<STAGED>(ctxs, b2w, nwt, cbeg, hpos_all + cbeg, hmb_all + cbeg, tailv,
                               sm.tail, D, sm.wsuf[wid], row, smp, n, lane);
    }
    PHASE(10);
    wave_sync();
    {
      // this wavefront's suffix counts, in place over its histogram: wsuf[w][v] = its end
      // positions with length >= v, for v = lane + 1 (lengths 1 .. 64 on 64 lanes)
      const int v = lane + 1;
      const int h = (v >= 3 && v <= D) ? sm.wsuf[wid][v] : 0;
      const int incl = wave_incl_add(h);
      int s = __builtin_amdgcn_readlane(incl, 63) - incl + h;
      s = v == 1 ? c1 : (v == 2 ? c2 : s);
      sm.wsuf[wid][v] = s;
    }
    PHASE(3);
    if (fast) worker_barrier(&sm.wbar, NWW, lane, a.err);
    else __syncthreads();
    PHASE(4);
    // ladder rung, sites, windows and vote of local candidate wid
    if (wid < nb) {
      const int maxl = D < J ? D : J;
      local_candidate(a, sm, NWW, maxl, J, bits_all, hpos_all, hmb_all, wid, lane);
      wave_sync();
      PHASE(5);
    }
  }

  // ---------------------------------------------------------------- 2. global (general path)
  if (GENERAL && r.has && (!fast || r.delta) && Lcap >= 2) {
    // this wavefront's slices of the request's delta group (read before the barrier, so that
    // they land while the local candidates finish)
    const long long dlo = r.delta_lo, dhi = r.delta_hi;
    const bool has_delta = dhi - dlo > 1;
    const bool listed = has_delta && a.pair_group != nullptr;
    const int sj = wid * kListSlices + lane;
    const PairSeg pseg = (listed && pgroup >= 0 && lane < kListSlices)
                             ? a.pair_seg[(size_t)sj * (size_t)(a.B + 1) + pgroup]
                             : PairSeg{0, 0};
    // The local sites are gathered and the hit lists are dead.  With a live snapshot and a
    // delta, the corpus wavefront has probed the snapshot beside the local phase (its results
    // stand).
    __syncthreads();
    if (tid <= kMaxD) {
      if (!fast) sm.ghist[tid] = 0;
      sm.dhist[tid] = 0;
    }
    for (int i = tid; i < NW * (kMaxD + 2); i += NT) (&sm.wsuf[0][0])[i] = 0;
    __syncthreads();
    const int act = r.act;
    const long long snap_start = r.snap_start;
    const long long dead_below = r.tail_w - snap_start;
    const int sbase = (int)(snap_start - r.tail_w);  // snapshot index -> site coordinate
    const View ib = view_of(a, act >= 0 ? act : 0, r.ht_mask);
    if (tid == 0) {
      sm.plp[0] = ib.pl0;
      sm.plp[1] = ib.pl1;
      sm.plp[2] = ib.pl2;
    }
    if (fast) {
      // probed already
    } else if (act >= 0 && r.snap_n > 0) {
      if (tid < kNG)
        probe_lane(ib, sm.tail, Lcap, dead_below, tid, &sm.g_off[tid], &sm.g_live[tid]);
    } else if (tid < kNG) {
      sm.g_off[tid] = 0;
      sm.g_live[tid] = 0;
    }
    __syncthreads();
    const int live4 = sm.g_live[2];
    // the same choice as the corpus wavefront's (the same inputs), which stands on the fast path
    const bool hot = act >= 0 && Lcap >= 5 && live4 > kHotGroup && dead_below <= 0;
    if (!fast && hot) {
      if (wid == 0)
        hot_bounds(ib, sm.tail, Lcap, (int)r.snap_n, lane, sm.hsup, sm.hlo, sm.hoff, sm.hcnt);
    } else if (!fast && act >= 0 && Lcap >= 5 && live4 > 0) {
      const int32_t* pl4 = ib.pl2 + sm.g_off[2];
      for (int x = tid; x < live4; x += NT) {
        const int m = extend4(ib.text, sm.tail, pl4[x], Lcap);
        if (m >= 5) atomicAdd(&sm.ghist[m], 1);
      }
    }
    // delta: documents appended since the live snapshot.  With the per-call pair index,
    // wavefront w owns the request's group entries in its slices (numbered [sb, se)); without
    // it, the end positions [sb, se), scanned by brute force.  It keeps its occurrences of length >= 2 in
    // LDS, in position order (coordinate offset from sb << 6 | length - 2; the context hit
    // lists are dead by now), at most H of them, plus a length histogram.
    long long sb, se;
    int lfirst = 0, lshift = 0;  // slice table of the listed walk (list_index)
    if (listed) {
      // this wavefront's slices of the request's group: entries numbered 0 .. se - 1
      const long long sg = pair_seg(dhi - dlo - 2);
      const PairSeg e = pseg;
      const int incl = wave_incl_add(e.cnt);
      lfirst = incl - e.cnt;
      lshift = (int)((long long)sj * sg + e.off - lfirst);
      sb = 0;
      se = __builtin_amdgcn_readlane(incl, 63);
    } else {
      const long long dseg = has_delta ? ((dhi - 1 - dlo + NW - 1) / NW + 63) / 64 * 64 : 0;
      sb = dlo + (long long)wid * dseg;
      se = has_delta ? (sb + dseg < dhi - 1 ? sb + dseg : dhi - 1) : sb;
    }
    PHASE(11);  // (slots 11-15 of the voters are the vote's own; wavefronts from 2 nb on keep these)
    const size_t dbase = hpos_offset(STAGED, a.S, a.T);
    const int H = (int)((vote_offset(STAGED, a.S, a.T, true) - dbase) / (4 * NW));
    uint32_t* recs = reinterpret_cast<uint32_t*>(dyn + dbase) + wid * H;
    int nrec = 0;
    if (has_delta) {
      int* wh = sm.wsuf[wid];  // this wavefront's length histogram, then (in place) suffix sums
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
      if (listed) delta_list_wave(a, dlo, sb, se, Lcap, sm.tail, lane, lfirst, lshift, keep);
      else delta_scan_wave(a, dlo, sb, se, Lcap, sm.tail, lane, keep);
      wave_sync();
      // this wavefront's suffix sums: wsuf[w][v] = its occurrences of length >= v, v = lane + 1
      const int h = lane + 1 <= Lcap ? wh[lane + 1] : 0;
      wave_sync();
      const int incl = wave_incl_add(h);
      sm.wsuf[wid][lane + 1] = __builtin_amdgcn_readlane(incl, 63) - incl + h;
    }
    __syncthreads();
    PHASE(12);
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
      const int hsup = (v >= 5 && v <= Lcap) ? sm.hsup[v] : 0;
      int snap = v >= 2 && v <= 4 ? sm.g_live[v - 2] : (hot ? hsup : gsuf);
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
    PHASE(13);
    // earliest sites: live snapshot occurrences in position order, then delta occurrences
    for (int ti = 0; ti < nb; ++ti) {
      const int ci = nb + ti;
      if (!sm.cand_valid[ci] || sm.cand_src[ci] != ci) continue;  // uniform
      const int l = sm.cand_len[ci];
      int* gs = sm.gsites[ti];
      int nsnap = 0;
      if (act >= 0) {
        if (l <= 4) {
          const int g = l - 2;
          const int live = sm.g_live[g];
          const int32_t* pl = sm.plp[g] + sm.g_off[g];
          nsnap = live < M ? live : M;
          for (int x = tid; x < nsnap; x += NT) gs[x] = pl[x] + l + sbase;
        } else if (hot) {
          if (wid == 0) {
            const int got = hot_sites(ib, sm, sm.tail, l, M, (int)r.snap_n, sbase,
                                      ib.pl2 + sm.g_off[2], live4, gs, lane);
            if (lane == 0) sm.hn = got;
          }
          __syncthreads();
          nsnap = sm.hn;
        } else if (fast) {
          // the corpus wavefront has the first kMaxM occurrences' extension lengths: one
          // wavefront walks the occurrences in position order, extending only past those
          if (wid == 0) {
            const int32_t* pl4 = ib.pl2 + sm.g_off[2];
            const uint64_t below = lanes_below(lane);
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
                  q = extend4(ib.text, sm.tail, i, l) >= l;
                }
              }
              const uint64_t bal = __ballot(q);
              const int rk = run + __popcll(bal & below);
              if (q && rk < M) gs[rk] = i + 4 + sbase;
              run += __popcll(bal);
            }
            if (lane == 0) sm.hn = run < M ? run : M;
          }
          __syncthreads();
          nsnap = sm.hn;
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
              if (extend4(ib.text, sm.tail, i, l) >= l) gs[rk++] = i + 4 + sbase;
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
          const long long u = sb + (long long)(rc >> 6);
          const int li = listed ? list_index((int)u, lfirst, lshift) : 0;  // (every lane)
          if (q && rk < M)
            gs[rk] = (int)((listed ? dlo + (long long)a.pair_list[li] : u) + 1 - r.tail_w);
          off += __popcll(bal);
        }
        if (nrec > H && off < M) {
          const long long from = sb + (long long)(recs[H - 1] >> 6) + 1;
          auto site = [&](long long, long long x, int m) {
            const bool q = m >= l;
            const uint64_t bal = __ballot(q);
            const int rk = off + lanes_before(bal);
            if (q && rk < M) gs[rk] = (int)(x + 1 - r.tail_w);
            off += __popcll(bal);
            return off < M;
          };
          if (listed) delta_list_wave(a, dlo, from, se, Lcap, sm.tail, lane, lfirst, lshift, site);
          else delta_scan_wave(a, dlo, from, se, Lcap, sm.tail, lane, site);
        }
      }
      // no barrier per candidate: each writes only its own site array, and the workgroup scan
      // of the next one ends with its own barriers
    }
    __syncthreads();
  }

  PHASE(14);
  // ---------------------------------------------------------------- 3. votes
  // One call site for every vote: wavefront ci votes candidate ci.  Without the general path,
  // local candidate t is voted right after its sites, and corpus candidate nb + t as soon as the
  // corpus wavefront has published its sites (while other wavefronts still work).  In the
  // longest-match mode only the candidate that the lengths select is voted.  In the scored mode
  // a vote is dropped between its passes once another candidate's final score beats every score
  // it can still reach (its score is then left at 0, which still loses to that one); it is not
  // checked before the vote starts, when the other votes have rarely ended.
  if (wid < 2 * nb) {
    const int ci = wid;
    const bool general = GENERAL && r.has && (!fast || r.delta) && Lcap >= 2;
    const bool gwait = fast && !general;  // corpus candidates arrive by flag
    if (gwait && ci >= nb && wid != GW) wait_flag(&sm.gready, lane, a.err);
    // the longest-match mode compares candidate 0 with candidate nb: wait for, or look at,
    // the flag of the one this wavefront does not produce
    bool known = true;
    if (a.mode == 0 && gwait) {
      if (ci == nb) {
        wait_flag(&sm.lready, lane, a.err);
      } else if (ci == 0) {
        known = __hip_atomic_load(&sm.gready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      }
    }
    // two rounds of LDS reads: lane j < 2 nb takes candidate j's fields, every lane its site
    // slot of candidate ci (slots past c0 hold harmless initial positions), then the cap and
    // the stop count of lane j's candidate
    const bool cl = lane < 2 * nb;
    const int fv = cl ? sm.cand_valid[lane] : 0;
    const int fs = cl ? sm.cand_src[lane] : -1;
    const int fc = cl ? sm.cand_c0[lane] : 0;
    const int fl = cl ? sm.cand_len[lane] : 0;
    const int sv_all = ci < nb ? sm.lsites[ci][lane] : sm.gsites[ci - nb][lane];
    const int fcap = sm.cap_tab[fl];
    const int fmin = sm.min_tab[fc];
    bool need = __builtin_amdgcn_readlane(fv, ci) && __builtin_amdgcn_readlane(fs, ci) == ci;
    const int c0 = __builtin_amdgcn_readlane(fc, ci);
    const int cap = __builtin_amdgcn_readlane(fcap, ci);
    const int cmin = __builtin_amdgcn_readlane(fmin, ci);
    const int dmax = cap < KMAX ? cap : KMAX;
    if (need && a.mode == 0) {
      if (ci != 0 && ci != nb) {
        need = false;
      } else if (known) {
        const bool lv = __builtin_amdgcn_readlane(fv, 0), gv = __builtin_amdgcn_readlane(fv, nb);
        const bool local_wins = lv && (!gv || __builtin_amdgcn_readlane(fl, 0) >=
                                                  __builtin_amdgcn_readlane(fl, nb));
        need = (ci == 0) == local_wins;
      }
    }
    if (!need) {
      if (lane == 0) {
        sm.cand_n[ci] = 0;
        sm.cand_snum[ci] = 0;
      }
    } else {
      int* hk = vote_all + ci * (2 * kVoteSlots);
      int nout = 0, snum = 0;
#if SFX_PHASE_TRACE
      unsigned long long* vts = a.trace ? sm.ts[wid] : nullptr;
#else
      unsigned long long* vts = nullptr;
#endif
      // (scored mode) whether a final score beats every score this vote can still reach
      auto beaten = [&](int bnum) { return a.mode == 1 && outscored(sm, ci, nb, bnum, c0, lane); };
      const bool loc = ci < nb;
      // few sites (and, for a corpus candidate, all of them in the snapshot text): columns
      const int32_t* text = r.act == 0 ? a.idx[0].text : (r.act == 1 ? a.idx[1].text : nullptr);
      const int sv = lane < c0 ? sv_all : 0;
      bool cols = c0 <= kColSites;
      if (cols && !loc) {
        const long long o = r.tail_w + sv - r.snap_start;
        cols = text != nullptr && __ballot(lane < c0 && (o < 0 || o >= r.snap_n)) == 0;
      }
      bool fin;
      if (cols) {
        // lane s: site s's first position (local) or text offset (corpus, < 2^30), and the
        // depths it can reach before the context or the text ends (the text's last token is a
        // separator: depths past it read that one)
        int lim;
        if (loc) {
          lim = L - sv;
        } else {
          const int o = (int)(r.tail_w + sv - r.snap_start);
          lim = lane < c0 ? (int)r.snap_n - 1 - o : 0;
        }
        const int so = loc ? sv : (int)(r.tail_w + sv - r.snap_start);
        // (a site from c0 on reads at position 0 with limit 0 (corpus: the text buffer holds the
        // ring's capacity) or L (local): in bounds)
        auto at_corpus = [&](int si, int i) {
          const int p = si < c0 ? __builtin_amdgcn_readlane(so, si) : 0;
          const int lm = __builtin_amdgcn_readlane(lim, si);
          return text[p + (i < lm ? i : lm)];
        };
        auto at_local = [&](int si, int i) {
          const int p = si < c0 ? __builtin_amdgcn_readlane(so, si) : 0;
          const int lm = __builtin_amdgcn_readlane(lim, si);
          int v;
          if (STAGED) {
            v = ctxs[p + i];  // p + i < L + 64: inside the stage
          } else {
            const int xc = i < lm ? p + i : L - 1;
            v = *(xc < n ? row + xc : smp + (xc - n));
          }
          return i < lm ? v : -1;
        };
        // the site loops are unrolled: instantiated for 1, 2, 4 and 8 sites
        auto run = [&](auto csc) {
          constexpr int CS = decltype(csc)::value;
          int T[CS], len[CS];
          if (loc) columns_cut<CS>(T, len, c0, dmax, lane, at_local);
          else columns_cut<CS>(T, len, c0, dmax, lane, at_corpus);
          PHASE(6);
          return vote_columns<CS>(T, len, c0, dmax, cmin, hk, hk + kVoteSlots, lane, beaten,
                                  sm.cand_out[ci], &nout, &snum);
        };
        static_assert(kColSites == 8, "column instantiations");
        static_assert(kPairSlices % NW == 0 && kListSlices <= 64, "listed slices per wavefront");
        if (c0 <= 1) fin = run(std::integral_constant<int, 1>{});
        else if (c0 <= 2) fin = run(std::integral_constant<int, 2>{});
        else if (c0 <= 4) fin = run(std::integral_constant<int, 4>{});
        else fin = run(std::integral_constant<int, 8>{});
      } else {
        int w0[KMAX], w1[KMAX];
        int len0 = 0, len1 = 0;
        if (loc)
          local_windows<KMAX, STAGED>(sm, ctxs, row, smp, n, L, ci, c0, cap, lane, w0, w1, &len0,
                                      &len1);
        else
          corpus_windows<KMAX>(a, r, sm.gsites[ci - nb], c0, cap, lane, w0, w1, &len0, &len1);
        PHASE(6);
        fin = vote_run<KMAX>(w0, w1, len0, c0, cap, cmin, hk, hk + kVoteSlots, lane, beaten,
                             sm.cand_out[ci], &nout, &snum, vts);
      }
      if (lane == 0) {
        sm.cand_n[ci] = nout;
        sm.cand_snum[ci] = snum;
      }
      // a final vote publishes its score in its done word (snum <= 4096 < 2^22 and
      // c0 <= 128 < 2^8 fit beside the flag bit); the selection reads the fields after a barrier
      static_assert(kMaxK * kMaxM < (1 << 22) && kMaxM < 256, "score packed in the done word");
      if (fin && lane == 0)
        __hip_atomic_store(&sm.cand_done[ci], (1 << 30) | (snum << 8) | c0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  if (lane == 0) sm.sink[wid] = pf;
  PHASE(7);
  __syncthreads();
  PHASE(8);

  // selection and output row, by wavefront 0.  Only a candidate that is the first of its length
  // in its source takes part: a later one shares that one's sites and vote, so it has the same
  // score and loses the tie to the earlier one.
  if (wid != 0) {
    PHASE_FLUSH();
    return;
  }
  // (every lane reads, lanes from 2 nb on candidate 0's fields, so that the six reads are
  // issued together; only lanes below 2 nb are used)
  const bool cl = lane < 2 * nb;
  const int li = cl ? lane : 0;
  const int fvalid = sm.cand_valid[li];
  const int fsrc = sm.cand_src[li];
  const int csn = sm.cand_snum[li];
  const int cc0 = sm.cand_c0[li];
  const int clen = sm.cand_len[li];
  const int fn = sm.cand_n[li];
  const bool cv = cl && (fvalid != 0) & (fsrc == lane);
  const int cn = cv ? fn : 0;
  const uint64_t vmask = __ballot(cv);
  int win = -1;
  if (a.mode == 0) {
    const bool lv = (vmask >> 0) & 1, gv = (vmask >> nb) & 1;
    const int l0 = __builtin_amdgcn_readlane(clen, 0), g0 = __builtin_amdgcn_readlane(clen, nb);
    if (lv && (!gv || l0 >= g0)) win = 0;
    else if (gv) win = nb;
  } else {
    // the highest score snum / c0, the first candidate among equal ones.  Scores become exact
    // integer keys: with snum <= 64 * 128 = 2^13 and 1 <= c0 <= 128, two different fractions
    // differ by at least 1 / 128^2 = 2^-14, so floor(snum * 2^14 / c0) keeps their order and
    // gives equal fractions equal keys.  The low four bits prefer the earlier candidate (lane i
    // holds candidate i < 16), and one maximum over the 16 lanes picks the winner.
    static_assert(2 * kMaxNB <= 16, "candidates in one row of 16 lanes");
    const uint32_t q = ((uint32_t)csn << 14) / (uint32_t)(cc0 > 0 ? cc0 : 1);
    const uint32_t key = cv ? ((q << 4) | (uint32_t)(15 - lane)) + 1u : 0u;
    const uint32_t best = row16_max_u32(key);
    win = best ? 15 - (int)((best - 1u) & 15u) : -1;
  }
  const int ws = win;
  const int nv = win >= 0 ? __builtin_amdgcn_readlane(cn, win) : 0;
  const int fill = a.mode == 0 ? r.t0 : -1;
  const int wlen = win >= 0 ? __builtin_amdgcn_readlane(clen, win) : 0;
  for (int i = lane; i < a.k; i += 64) drow[i] = i < nv ? sm.cand_out[ws][i] : fill;
  if (lane == 0) {
    a.nvalid[b] = nv;
    a.pick[b] = win >= 0 ? (nv << 16) | ((win >= nb ? 1 : 0) << 8) | wlen : -1;
  }
  PHASE(9);
  PHASE_FLUSH();
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
hipError_t launch_k(const ProposeArgs& a, bool staged, bool general, size_t dyn, hipStream_t st) {
  if (staged && general)
    hipLaunchKernelGGL((propose_kernel<KMAX, true, true>), dim3(a.B), dim3(NT), dyn, st, a);
  else if (staged)
    hipLaunchKernelGGL((propose_kernel<KMAX, true, false>), dim3(a.B), dim3(NT), dyn, st, a);
  else if (general)
    hipLaunchKernelGGL((propose_kernel<KMAX, false, true>), dim3(a.B), dim3(NT), dyn, st, a);
  else
    hipLaunchKernelGGL((propose_kernel<KMAX, false, false>), dim3(a.B), dim3(NT), dyn, st, a);
  return hipGetLastError();
}

}  // namespace

size_t propose_dynamic_lds(bool staged, int S, int T, bool corpus, int nb) {
  return dyn_bytes(staged, S, T, corpus, nb);
}

namespace {
size_t g_static_lds = 0;  // largest static LDS over the propose instantiations (queried)
}

size_t propose_static_lds() { return g_static_lds ? g_static_lds : sizeof(Smem); }

bool propose_staged(int S, int T, bool stream_ctx, bool corpus, int nb) {
  return !stream_ctx && dyn_bytes(true, S, T, corpus, nb) + propose_static_lds() <= kLdsBytes;
}

hipError_t propose_prepare() {
  const void* fns[] = {
      (const void*)propose_kernel<8, true, true>,   (const void*)propose_kernel<8, false, true>,
      (const void*)propose_kernel<16, true, true>,  (const void*)propose_kernel<16, false, true>,
      (const void*)propose_kernel<32, true, true>,  (const void*)propose_kernel<32, false, true>,
      (const void*)propose_kernel<8, true, false>,  (const void*)propose_kernel<8, false, false>,
      (const void*)propose_kernel<16, true, false>, (const void*)propose_kernel<16, false, false>,
      (const void*)propose_kernel<32, true, false>, (const void*)propose_kernel<32, false, false>};
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

hipError_t launch_propose(const ProposeArgs& a, bool general, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const bool corpus = a.ctl != nullptr;
  const bool staged = propose_staged(a.S, a.T, a.stream_ctx != 0, corpus, a.nb);
  const size_t dyn = dyn_bytes(staged, a.S, a.T, corpus, a.nb);
  if (dyn + propose_static_lds() > kLdsBytes) return hipErrorInvalidValue;
  if (a.k <= 8) return launch_k<8>(a, staged, general, dyn, st);
  if (a.k <= 16) return launch_k<16>(a, staged, general, dyn, st);
  return launch_k<32>(a, staged, general, dyn, st);
}

hipError_t launch_update_state(int B, int S, int T, int32_t* tok, const int32_t* ntns,
                               const int32_t* samp, int32_t* nout, hipStream_t st) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(update_state_kernel, dim3((B + 255) / 256), dim3(256), 0, st, B, S, T, tok,
                     ntns, samp, nout);
  return hipGetLastError();
}

}  // namespace sfx
