// propose.hip -- the drafter step on gfx950: one workgroup (16 wavefronts) per request.
//
// Steps, in the order of the suffix-gpu page, How it works:
//   1. local match: a backward match length against the tail for every earlier position,
//      kept as bytes in LDS with a length histogram -> num_backoff ladder lengths (t-th largest
//      value) and, per ladder length, the earliest max_occurrences continuation sites;
//   2. global match (vLLM docs, Model Runner V2: probe by the last 2 and last 4 tokens, extend
//      to the longest match): 2-, 3- and 4-gram probes into hash tables over the suffix-array
//      groups of the live snapshot, backward extension of the 4-gram occurrences, plus a
//      brute-force scan of the not-yet-indexed delta documents;
//   3. expansion: one wavefront per candidate votes depth by depth over its sites with an LDS
//      hash of token counts; stop rule and score use integer cross-multiplication; selection
//      and the [k] output row are written by thread 0.
#include "propose.h"

namespace sfx {

namespace {

constexpr int NT = 1024;
constexpr int NW = NT / 64;
constexpr int kVoteSlots = 256;

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

// Exclusive prefix sum of one int per thread over the workgroup; *total gets the sum.
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
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

__device__ __forceinline__ int ctx_at(const int32_t* row, const int32_t* smp, int n, int x) {
  return x < n ? row[x] : smp[x - n];
}

// Count one vote for `tok` in the wavefront's LDS table; returns the slot used.
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
  int n, t, L, Lcap;
  int has_index, active;
  long long snap_start, snap_n, tail_w, delta_lo, delta_hi;
  uint32_t ht_mask;
  int tail[kMaxD];
  int hist[kMaxD + 1];
  int ghist[kMaxD + 1];
  int dhist[kMaxD + 1];
  int g_off[kNG], g_live[kNG];
  int cand_len[2 * kMaxNB], cand_sup[2 * kMaxNB], cand_c0[2 * kMaxNB], cand_valid[2 * kMaxNB];
  int cand_src[2 * kMaxNB], cand_n[2 * kMaxNB];
  long long cand_snum[2 * kMaxNB];
  int cand_out[2 * kMaxNB][kMaxK];
  int lsites[kMaxNB][kMaxM];
  long long gsites[kMaxNB][kMaxM];
  const int32_t* plp[kNG];  // position lists of the live buffer, indexable by n-gram size
  int wsum[NW + 1];
  int vkey[NW][kVoteSlots];
  int vcnt[NW][kVoteSlots];
};

__device__ __forceinline__ int spec_cap(const ProposeArgs& a, int l) {
  if (a.mode != 1) return a.k;
  long long c = (a.factor_ppm * (long long)l + a.offset_ppm) / 1000000;
  if (c < 0) c = 0;
  return c < a.k ? (int)c : a.k;
}

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
__device__ __forceinline__ View view_of(const ProposeArgs& a, int act) {
  const bool z = act == 0;
  View v;
  v.mask = 0;
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
__device__ void probe_ngram(const View& ib, const int* tail, int Lcap, long long dead_below,
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

// Corpus token at logical position q: snapshot text below snap_end, ring slot above.
__device__ __forceinline__ int corpus_at(const ProposeArgs& a, const int32_t* text,
                                         long long snap_start, long long snap_n, long long q) {
  long long s = q - snap_start;
  if (s >= 0 && s < snap_n) return text[s];
  return a.ring[q % a.ring_cap];
}

template <int KMAX, bool VEC>
__global__ __launch_bounds__(NT) void propose_kernel(ProposeArgs a) {
  extern __shared__ uint8_t mbs[];
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.x;
  const int32_t* row = a.tok + (int64_t)b * a.S;
  const int32_t* smp = a.samp + (int64_t)b * a.T;
  const int D = a.D, nb = a.nb, M = a.M;

  if (tid == 0) {
    int n = a.ntns[b];
    n = n < 0 ? 0 : (n > a.S ? a.S : n);
    int t = 0;
    while (t < a.T && smp[t] >= 0) ++t;
    sm.n = n;
    sm.t = t;
    sm.L = n + t;
    sm.Lcap = D < n + t ? D : n + t;
    int has = 0, act = -1;
    if (a.ctl) {
      act = a.ctl->active;
      has = 1;
      sm.tail_w = a.ctl->tail;
      long long head = a.ctl->head;
      if (act >= 0) {
        sm.ht_mask = a.ctl->ht_mask[act];
        sm.snap_start = a.ctl->snap_start[act];
        sm.snap_n = a.ctl->snap_end[act] - sm.snap_start;
        long long lo = a.ctl->snap_end[act];
        sm.delta_lo = lo > sm.tail_w ? lo : sm.tail_w;
      } else {
        sm.snap_start = 0;
        sm.snap_n = 0;
        sm.delta_lo = sm.tail_w;
      }
      sm.delta_hi = head;
    }
    sm.has_index = has;
    sm.active = act;
  }
  if (tid <= kMaxD) {
    sm.hist[tid] = 0;
    sm.ghist[tid] = 0;
    sm.dhist[tid] = 0;
  }
  __syncthreads();
  const int n = sm.n, t = sm.t, L = sm.L, Lcap = sm.Lcap;
  int32_t* drow = a.draft + (int64_t)b * a.k;
  if (t == 0) {
    for (int i = tid; i < a.k; i += NT) drow[i] = -1;
    if (tid == 0) a.nvalid[b] = 0;
    return;
  }
  for (int i = tid; i < Lcap; i += NT) sm.tail[i] = ctx_at(row, smp, n, L - 1 - i);
  __syncthreads();

  // ---------------------------------------------------------------- 1. local match lengths
  const int J = L - 1;  // candidate ends j = 0..L-2
  {
    const int t0 = sm.tail[0];
    int ones = 0;
    for (int j0 = tid * 4; j0 < J; j0 += NT * 4) {
      int v[4];
      if (VEC && j0 + 3 < n) {
        int4 q = *reinterpret_cast<const int4*>(row + j0);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = j0 + u < J ? ctx_at(row, smp, n, j0 + u) : 0;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int jj = j0 + u;
        if (jj < J) {
          int m = 0;
          if (v[u] == t0) {
            m = 1;
            const int lim = D < jj + 1 ? D : jj + 1;
            while (m < lim && ctx_at(row, smp, n, jj - m) == sm.tail[m]) ++m;
          }
          mbs[jj] = (uint8_t)m;
          if (m == 1) ++ones;
          else if (m > 1) atomicAdd(&sm.hist[m], 1);
        }
      }
    }
    ones = wave_sum(ones);
    if (lane == 0 && ones) atomicAdd(&sm.hist[1], ones);
  }
  __syncthreads();

  // local ladder: l_t = t-th largest match length
  if (tid == 0) {
    int cum = 0, ti = 0;
    const int maxl = D < J ? D : J;
    for (int l = maxl; l >= 1 && ti < nb; --l) {
      cum += sm.hist[l];
      while (ti < nb && cum >= ti + 1) {
        sm.cand_len[ti] = l;
        sm.cand_sup[ti] = cum;
        ++ti;
      }
    }
    for (; ti < nb; ++ti) {
      sm.cand_len[ti] = 0;
      sm.cand_sup[ti] = 0;
    }
    const int mins = a.min_self > 1 ? a.min_self : 1;
    for (int i = 0; i < nb; ++i) {
      sm.cand_valid[i] = sm.cand_len[i] >= mins;
      sm.cand_c0[i] = sm.cand_sup[i] < M ? sm.cand_sup[i] : M;
      sm.cand_src[i] = (i > 0 && sm.cand_len[i] == sm.cand_len[i - 1]) ? sm.cand_src[i - 1] : i;
    }
  }
  __syncthreads();

  // earliest sites per distinct ladder length: ordered compaction over the LDS lengths
  {
    const int seg = (J + NT - 1) / NT;
    const int lo = tid * seg < J ? tid * seg : J;
    const int hi = lo + seg < J ? lo + seg : J;
    for (int ti = 0; ti < nb; ++ti) {
      if (!sm.cand_valid[ti] || sm.cand_src[ti] != ti) continue;  // uniform
      const int l = sm.cand_len[ti];
      int c = 0;
      for (int j = lo; j < hi; ++j) c += mbs[j] >= l;
      int total;
      int r = block_exclusive_scan(c, sm.wsum, &total);
      if (c && r < M) {
        for (int j = lo; j < hi && r < M; ++j)
          if (mbs[j] >= l) sm.lsites[ti][r++] = j + 1;
      }
    }
  }

  // ---------------------------------------------------------------- 2. global match
  for (int i = tid; i < nb; i += NT) sm.cand_valid[nb + i] = 0;
  __syncthreads();
  if (sm.has_index && Lcap >= 2) {
    const int act = sm.active;
    const long long snap_start = sm.snap_start;
    const long long dead_below = sm.tail_w - snap_start;  // snapshot coords of live start
    View ib = view_of(a, act >= 0 ? act : 0);
    ib.mask = sm.ht_mask;
    if (tid == 0) {
      sm.plp[0] = ib.pl0;
      sm.plp[1] = ib.pl1;
      sm.plp[2] = ib.pl2;
    }
    // probes: thread g looks up the (g+2)-gram ending at the last token
    if (act >= 0 && sm.snap_n > 0) {
      if (tid == 0) probe_ngram<0>(ib, sm.tail, Lcap, dead_below, &sm.g_off[0], &sm.g_live[0]);
      if (tid == 1) probe_ngram<1>(ib, sm.tail, Lcap, dead_below, &sm.g_off[1], &sm.g_live[1]);
      if (tid == 2) probe_ngram<2>(ib, sm.tail, Lcap, dead_below, &sm.g_off[2], &sm.g_live[2]);
    } else if (tid < kNG) {
      sm.g_off[tid] = 0;
      sm.g_live[tid] = 0;
    }
    __syncthreads();
    // backward extension of the live 4-gram occurrences
    const int live4 = sm.g_live[2];
    if (act >= 0 && Lcap >= 5 && live4 > 0) {
      const int32_t* pl4 = ib.pl2 + sm.g_off[2];
      const int32_t* text = ib.text;
      for (int x = tid; x < live4; x += NT) {
        const int i = pl4[x];
        int m = 4;
        while (m < Lcap && i - 1 - (m - 4) >= 0) {
          int c = text[i - 1 - (m - 4)];
          if (c < 0 || c != sm.tail[m]) break;
          ++m;
        }
        if (m >= 5) atomicAdd(&sm.ghist[m], 1);
      }
    }
    // delta: documents appended since the live snapshot, scanned by brute force
    const long long dlo = sm.delta_lo, dhi = sm.delta_hi;
    if (dhi - dlo > 1) {
      const int t0 = sm.tail[0];
      for (long long e = dlo + tid; e + 1 < dhi; e += NT) {
        const int c = a.ring[e % a.ring_cap];
        if (c != t0) continue;
        if (a.ring[(e + 1) % a.ring_cap] < 0) continue;
        int m = 1;
        while (m < Lcap && e - m >= dlo) {
          int x = a.ring[(e - m) % a.ring_cap];
          if (x < 0 || x != sm.tail[m]) break;
          ++m;
        }
        if (m >= 2) atomicAdd(&sm.dhist[m], 1);
      }
    }
    __syncthreads();
    // global ladder: count_ge(l) = snapshot support + delta support
    if (tid == 0) {
      int dcum = 0, gcum = 0, ti = 0;
      for (int l = Lcap; l >= 2 && ti < nb; --l) {
        dcum += sm.dhist[l];
        gcum += sm.ghist[l];
        int snap = l <= 4 ? sm.g_live[l - 2] : gcum;
        if (act < 0) snap = 0;
        const int cnt = snap + dcum;
        while (ti < nb && cnt >= ti + 1) {
          sm.cand_len[nb + ti] = l;
          sm.cand_sup[nb + ti] = cnt;
          ++ti;
        }
      }
      for (; ti < nb; ++ti) {
        sm.cand_len[nb + ti] = 0;
        sm.cand_sup[nb + ti] = 0;
      }
      const int minc = a.min_corpus > 2 ? a.min_corpus : 2;
      for (int i = 0; i < nb; ++i) {
        const int ci = nb + i;
        sm.cand_valid[ci] = sm.cand_len[ci] >= minc;
        sm.cand_c0[ci] = sm.cand_sup[ci] < M ? sm.cand_sup[ci] : M;
        sm.cand_src[ci] = (i > 0 && sm.cand_len[ci] == sm.cand_len[ci - 1]) ? sm.cand_src[ci - 1]
                                                                             : ci;
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
          const int32_t* text = ib.text;
          const int seg = (live4 + NT - 1) / NT;
          const int lo = tid * seg < live4 ? tid * seg : live4;
          const int hi = lo + seg < live4 ? lo + seg : live4;
          int c = 0;
          for (int x = lo; x < hi; ++x) {
            const int i = pl4[x];
            int m = 4;
            while (m < l && i - 1 - (m - 4) >= 0) {
              int cc = text[i - 1 - (m - 4)];
              if (cc < 0 || cc != sm.tail[m]) break;
              ++m;
            }
            c += m >= l;
          }
          int total;
          int r = block_exclusive_scan(c, sm.wsum, &total);
          if (c && r < M) {
            for (int x = lo; x < hi && r < M; ++x) {
              const int i = pl4[x];
              int m = 4;
              while (m < l && i - 1 - (m - 4) >= 0) {
                int cc = text[i - 1 - (m - 4)];
                if (cc < 0 || cc != sm.tail[m]) break;
                ++m;
              }
              if (m >= l) gs[r++] = (long long)i + 4 + snap_start;
            }
          }
          nsnap = total < M ? total : M;
        }
      }
      // delta occurrences follow every snapshot occurrence in logical order
      if (nsnap < M && dhi - dlo > 1) {
        const long long span = dhi - dlo;
        const long long seg = (span + NT - 1) / NT;
        const long long lo = dlo + (long long)tid * seg < dhi ? dlo + (long long)tid * seg : dhi;
        const long long hi = lo + seg < dhi ? lo + seg : dhi;
        int c = 0;
        for (long long e = lo; e < hi; ++e) {
          if (e + 1 >= dhi) break;
          if (a.ring[(e + 1) % a.ring_cap] < 0) continue;
          int m = 0;
          while (m < l && e - m >= dlo) {
            int x = a.ring[(e - m) % a.ring_cap];
            if (x < 0 || x != sm.tail[m]) break;
            ++m;
          }
          c += m >= l;
        }
        int total;
        int r = block_exclusive_scan(c, sm.wsum, &total) + nsnap;
        if (c && r < M) {
          for (long long e = lo; e < hi && r < M; ++e) {
            if (e + 1 >= dhi) break;
            if (a.ring[(e + 1) % a.ring_cap] < 0) continue;
            int m = 0;
            while (m < l && e - m >= dlo) {
              int x = a.ring[(e - m) % a.ring_cap];
              if (x < 0 || x != sm.tail[m]) break;
              ++m;
            }
            if (m >= l) gs[r++] = e + 1;
          }
        }
      }
      __syncthreads();
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- 3. expansion and vote
  if (wid < 2 * nb && sm.cand_valid[wid]) {
    const int ci = wid;
    const int src = sm.cand_src[ci];
    const bool local = ci < nb;
    const int c0 = sm.cand_c0[ci];
    const int cap = spec_cap(a, sm.cand_len[ci]);
    const int s0 = lane, s1 = lane + 64;
    int w0[KMAX], w1[KMAX];
    if (local) {
      const int* ls = sm.lsites[src];
      const int p0 = s0 < c0 ? ls[s0] : 0, p1 = s1 < c0 ? ls[s1] : 0;
#pragma unroll
      for (int d = 0; d < KMAX; ++d) {
        w0[d] = (s0 < c0 && d < cap && p0 + d < L) ? ctx_at(row, smp, n, p0 + d) : -1;
        w1[d] = (s1 < c0 && d < cap && p1 + d < L) ? ctx_at(row, smp, n, p1 + d) : -1;
      }
    } else {
      const long long* gs = sm.gsites[src - nb];
      const int act = sm.active;
      const int32_t* text = act == 0 ? a.idx[0].text : (act == 1 ? a.idx[1].text : nullptr);
      const long long ss = sm.snap_start, sn = sm.snap_n;
      const long long q0 = s0 < c0 ? gs[s0] : 0, q1 = s1 < c0 ? gs[s1] : 0;
      bool live0 = s0 < c0, live1 = s1 < c0;
#pragma unroll
      for (int d = 0; d < KMAX; ++d) {
        int x0 = -1, x1 = -1;
        if (live0 && d < cap) x0 = corpus_at(a, text, ss, sn, q0 + d);
        if (live1 && d < cap) x1 = corpus_at(a, text, ss, sn, q1 + d);
        live0 = live0 && x0 >= 0;
        live1 = live1 && x1 >= 0;
        w0[d] = x0;
        w1[d] = x1;
      }
    }
    int* hk = sm.vkey[wid];
    int* hc = sm.vcnt[wid];
    bool al0 = s0 < c0, al1 = s1 < c0;
    int nout = 0;
    long long snum = 0;
    for (int d = 0; d < cap; ++d) {
      // the window arrays act as shift registers: slot 0 is always the current depth
      const int cur0 = w0[0], cur1 = w1[0];
#pragma unroll
      for (int x = 0; x + 1 < KMAX; ++x) {
        w0[x] = w0[x + 1];
        w1[x] = w1[x + 1];
      }
      w0[KMAX - 1] = -1;
      w1[KMAX - 1] = -1;
      for (int x = lane; x < kVoteSlots; x += 64) {
        hk[x] = -1;
        hc[x] = 0;
      }
      wave_sync();
      const int tk0 = al0 ? cur0 : -1, tk1 = al1 ? cur1 : -1;
      int sl0 = -1, sl1 = -1;
      if (tk0 >= 0) sl0 = vote_insert(hk, hc, tk0);
      if (tk1 >= 0) sl1 = vote_insert(hk, hc, tk1);
      wave_sync();
      uint64_t key = 0;
      if (sl0 >= 0) {
        uint64_t k0 = ((uint64_t)(uint32_t)hc[sl0] << 32) | (uint32_t)(0x7FFFFFFF - tk0);
        key = k0 > key ? k0 : key;
      }
      if (sl1 >= 0) {
        uint64_t k1 = ((uint64_t)(uint32_t)hc[sl1] << 32) | (uint32_t)(0x7FFFFFFF - tk1);
        key = k1 > key ? k1 : key;
      }
      key = wave_max_u64(key);
      if (key == 0) break;
      const int c = (int)(key >> 32);
      const int w = 0x7FFFFFFF - (int)(uint32_t)(key & 0xFFFFFFFFu);
      if (a.mode == 1 && (long long)c * 1000000 < a.prob_ppm * (long long)c0) break;
      if (lane == 0) sm.cand_out[ci][nout] = w;
      ++nout;
      snum += c;
      al0 = tk0 == w;
      al1 = tk1 == w;
      wave_sync();
    }
    if (lane == 0) {
      sm.cand_n[ci] = nout;
      sm.cand_snum[ci] = snum;
    }
  }
  __syncthreads();

  // selection and output row
  if (tid == 0) {
    int win = -1;
    if (a.mode == 0) {
      const int lv = sm.cand_valid[0], gv = sm.cand_valid[nb];
      if (lv && (!gv || sm.cand_len[0] >= sm.cand_len[nb])) win = 0;
      else if (gv) win = nb;
    } else {
      for (int i = 0; i < 2 * nb; ++i) {
        if (!sm.cand_valid[i]) continue;
        if (win < 0 ||
            sm.cand_snum[i] * (long long)sm.cand_c0[win] > sm.cand_snum[win] * (long long)sm.cand_c0[i])
          win = i;
      }
    }
    sm.wsum[0] = win;
    sm.wsum[1] = win >= 0 ? sm.cand_n[win] : 0;
  }
  __syncthreads();
  const int win = sm.wsum[0], nv = sm.wsum[1];
  const int fill = a.mode == 0 ? sm.tail[0] : -1;
  for (int i = tid; i < a.k; i += NT) drow[i] = i < nv ? sm.cand_out[win][i] : fill;
  if (tid == 0) a.nvalid[b] = nv;
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
hipError_t launch_k(const ProposeArgs& a, bool vec, size_t dyn, hipStream_t st) {
  if (vec)
    hipLaunchKernelGGL((propose_kernel<KMAX, true>), dim3(a.B), dim3(NT), dyn, st, a);
  else
    hipLaunchKernelGGL((propose_kernel<KMAX, false>), dim3(a.B), dim3(NT), dyn, st, a);
  return hipGetLastError();
}

}  // namespace

size_t propose_dynamic_lds(int S, int T) { return ((size_t)S + T + 16) & ~(size_t)15; }

hipError_t propose_prepare(size_t dyn) {
  const void* fns[] = {
      (const void*)propose_kernel<8, true>,  (const void*)propose_kernel<8, false>,
      (const void*)propose_kernel<16, true>, (const void*)propose_kernel<16, false>,
      (const void*)propose_kernel<32, true>, (const void*)propose_kernel<32, false>};
  for (const void* f : fns) {
    hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_propose(const ProposeArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const bool vec = (a.S % 4 == 0) && ((uintptr_t)a.tok % 16 == 0);
  const size_t dyn = propose_dynamic_lds(a.S, a.T);
  if (a.k <= 8) return launch_k<8>(a, vec, dyn, st);
  if (a.k <= 16) return launch_k<16>(a, vec, dyn, st);
  return launch_k<32>(a, vec, dyn, st);
}

hipError_t launch_update_state(int B, int S, int T, int32_t* tok, const int32_t* ntns,
                               const int32_t* samp, int32_t* nout, hipStream_t st) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(update_state_kernel, dim3((B + 255) / 256), dim3(256), 0, st, B, S, T, tok,
                     ntns, samp, nout);
  return hipGetLastError();
}

}  // namespace sfx
