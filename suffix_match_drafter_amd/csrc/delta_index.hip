// delta_index.hip -- per-call index of the delta's occurrences of the batch's tail pairs.
//
// suffix-gpu page, How it works step 2 and Highlights: documents appended since the live
// snapshot are not in the suffix array and are matched by position.  A request's corpus
// candidates there start from the positions x whose token is its last context token and whose
// previous token (still inside the delta) is its second-to-last, with a real token after x.
// The drafter step used to find them by scanning the whole delta in every request.  One pass
// finds them once per call for every request at the same time: positions are grouped by the
// pair (token before, token at x), for the pairs that end some request's context, slice by
// slice, and each group keeps position order inside a slice, which with the slices in order is
// the logical order the step's site rule needs.
#include "delta_index.h"

namespace sfx {

namespace {

constexpr unsigned long long kNoPair = ~0ull;  // a pair whose first token is -1: never a key

__device__ __forceinline__ unsigned long long pair_key(int first, int second) {
  return ((unsigned long long)(uint32_t)first << 32) | (uint32_t)second;
}

__device__ __forceinline__ uint32_t pair_hash(unsigned long long k) {
  k ^= k >> 33;
  k *= 0xff51afd7ed558ccdull;
  k ^= k >> 33;
  k *= 0xc4ceb9fe1a85ec53ull;
  k ^= k >> 33;
  return (uint32_t)k;
}

// The delta's logical range [lo, hi) under the control block, by the drafter step's rule: it
// starts at the live snapshot's end (or at the oldest live document, if later).  Returns
// whether it holds a candidate end position (at least two tokens).
__device__ __forceinline__ bool delta_range(const Ctl* ctl, long long* lo, long long* hi) {
  const Ctl c = *ctl;
  long long l = c.tail;
  if (c.active >= 0) {
    const long long se = c.active == 0 ? c.snap_end[0] : c.snap_end[1];
    l = se > l ? se : l;
  }
  *lo = l;
  *hi = c.head;
  return c.head - l > 1;
}

// The tail pair of request b when its step reads the delta -- a non-empty sampled prefix, a
// two-token tail within max_tree_depth and a non-negative second-to-last token -- else kNoPair.
__device__ __forceinline__ unsigned long long tail_pair(const PairIndexArgs& a, int b) {
  int n = a.ntns[b];
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  const int32_t* smp = a.samp + (int64_t)b * a.T;
  const int32_t* row = a.tok + (int64_t)b * a.S;
  int t = 0;
  while (t < a.T && smp[t] >= 0) ++t;
  const int L = n + t;
  const int lcap = a.D < L ? a.D : L;
  if (t == 0 || lcap < 2) return kNoPair;
  const int last = smp[t - 1];
  const int before = L - 2 >= n ? smp[L - 2 - n] : row[L - 2];
  return before >= 0 ? pair_key(before, last) : kNoPair;
}

constexpr int kSliceRuns = 4;  // 64-position runs whose loads a wavefront issues together
constexpr int kSliceThreads = 64 * kPairWaves;

// The group of end position x (ring slot sl): (token before, token at x) is the group's pair and
// a real token follows; -1 otherwise.
__device__ __forceinline__ int group_at(const unsigned long long* hk, const int* hg,
                                        uint32_t mask, int p, int c, int nx) {
  if (p < 0 || nx < 0) return -1;
  const unsigned long long key = pair_key(p, c);
  uint32_t h = pair_hash(key) & mask;
  for (;;) {
    const unsigned long long k = hk[h];
    if (k == key) return hg[h];
    if (k == kNoPair) return -1;
    h = (h + 1) & mask;
  }
}

// One workgroup per delta slice (see delta_index.h).  Wavefront w of slice s walks its own
// run of the slice twice, first counting per group, then writing; cw[w][g] holds its counts,
// then its next list entry of group g.
__global__ __launch_bounds__(kSliceThreads) void pair_index_kernel(PairIndexArgs a) {
  __shared__ unsigned long long hk[2 * kPairMaxBatch];
  __shared__ int hg[2 * kPairMaxBatch];
  __shared__ int cw[kPairWaves][kPairMaxBatch + 1];
  __shared__ int wsum[kPairWaves];
  const uint32_t mask = a.slots - 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sidx = blockIdx.x;
  const int ng = a.B + 1;
  long long lo, hi;
  const bool any = delta_range(a.ctl, &lo, &hi);
  // this slice's end positions [xb, xe) and this wavefront's run [wb, we) of them
  const long long nd = any ? hi - lo - 2 : 0;
  const long long sg = pair_seg(nd);
  const long long xb = lo + 1 + (long long)sidx * sg;
  const long long xe = xb + sg < hi - 1 ? xb + sg : hi - 1;
  const long long wn = ((sg + kPairWaves - 1) / kPairWaves + 63) / 64 * 64;
  const long long wb = xb + (long long)w * wn;
  const long long we = wb + wn < xe ? wb + wn : xe;
  const int cap = (int)a.ring_cap;
  const int s0 = any && wb < we ? (int)((wb + lane) % a.ring_cap) : 0;  // the lane's first slot
  // the first kSliceRuns runs' tokens, loaded before the table is built so that both wait
  // together; their groups are kept for the writing walk
  int p1[kSliceRuns], c1[kSliceRuns], n1[kSliceRuns], g1[kSliceRuns];
  int s1 = s0;
#pragma unroll
  for (int u = 0; u < kSliceRuns; ++u) {
    const bool in = wb + 64 * u + lane < we;
    const int sp = s1 == 0 ? cap - 1 : s1 - 1;
    const int sn = s1 + 1 == cap ? 0 : s1 + 1;
    p1[u] = in ? a.ring[sp] : -1;
    c1[u] = in ? a.ring[s1] : -1;
    n1[u] = in ? a.ring[sn] : -1;
    s1 += 64;
    while (s1 >= cap) s1 -= cap;
  }
  // the table of the batch's tail pairs, and zero counters
  constexpr int kReq = kPairMaxBatch / kSliceThreads;
  unsigned long long rk[kReq];
#pragma unroll
  for (int j = 0; j < kReq; ++j) {
    const int b = tid + kSliceThreads * j;
    rk[j] = b < a.B ? tail_pair(a, b) : kNoPair;
  }
  for (uint32_t i = tid; i < a.slots; i += kSliceThreads) {
    hk[i] = kNoPair;
    hg[i] = INT32_MAX;
  }
  for (int e = tid; e < kPairWaves * (kPairMaxBatch + 1); e += kSliceThreads)
    (&cw[0][0])[e] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kReq; ++j) {
    if (rk[j] == kNoPair) continue;
    uint32_t h = pair_hash(rk[j]) & mask;
    for (;;) {
      const unsigned long long prev = atomicCAS(&hk[h], kNoPair, rk[j]);
      if (prev == kNoPair || prev == rk[j]) break;
      h = (h + 1) & mask;
    }
    atomicMin(&hg[h], tid + kSliceThreads * j);
  }
  __syncthreads();
  if (sidx == 0) {
#pragma unroll
    for (int j = 0; j < kReq; ++j) {
      const int b = tid + kSliceThreads * j;
      if (b >= a.B) continue;
      int g = -1;
      if (rk[j] != kNoPair) {
        uint32_t h = pair_hash(rk[j]) & mask;
        while (hk[h] != rk[j]) h = (h + 1) & mask;
        g = hg[h];
      }
      a.group[b] = g;
    }
  }
  if (!any) return;  // uniform over the grid: the step reads no list
  uint32_t* part = a.list + (size_t)sidx * (size_t)sg;
  for (int pass = 0; pass < 2; ++pass) {
    int s = s1;  // slot past the first runs
    for (long long x0 = wb; x0 < we; x0 += 64 * kSliceRuns) {
      const bool first = x0 == wb;
      int p[kSliceRuns], c[kSliceRuns], nx[kSliceRuns];
      if (!first) {
#pragma unroll
        for (int u = 0; u < kSliceRuns; ++u) {
          const bool in = x0 + 64 * u + lane < we;
          const int sp = s == 0 ? cap - 1 : s - 1;
          const int sn = s + 1 == cap ? 0 : s + 1;
          p[u] = in ? a.ring[sp] : -1;
          c[u] = in ? a.ring[s] : -1;
          nx[u] = in ? a.ring[sn] : -1;
          s += 64;
          while (s >= cap) s -= cap;
        }
      }
#pragma unroll
      for (int u = 0; u < kSliceRuns; ++u) {
        const long long x = x0 + 64 * u + lane;
        int g;
        if (first) {
          if (pass == 0) g1[u] = group_at(hk, hg, mask, p1[u], c1[u], n1[u]);
          g = g1[u];
        } else {
          g = group_at(hk, hg, mask, p[u], c[u], nx[u]);
        }
        if (pass == 0) {
          if (g >= 0) atomicAdd(&cw[w][g], 1);
        } else {
          // one group at a time: the lanes of group gg take consecutive list entries
          uint64_t pend = __ballot(g >= 0);
          while (pend) {
            const int gg = __builtin_amdgcn_readlane(g, __builtin_ctzll(pend));
            const uint64_t same = __ballot(g == gg);
            const int base = cw[w][gg];
            if (g == gg) part[base + __popcll(same & ((1ull << lane) - 1))] = (uint32_t)(x - lo);
            __builtin_amdgcn_wave_barrier();
            if (lane == 0) cw[w][gg] = base + __popcll(same);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            pend &= ~same;
          }
        }
      }
    }
    if (pass == 1) break;
    __syncthreads();
    // per group: its count in the slice, its offset (the counts of the groups before it), and
    // each wavefront's first entry (after the wavefronts before it); thread t takes groups
    // kPer * t .. kPer * t + kPer - 1
    constexpr int kPer = (kPairMaxBatch + 1 + kSliceThreads - 1) / kSliceThreads;
    int cnt[kPer], sum = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int g = kPer * tid + k;
      cnt[k] = 0;
      if (g < ng)
#pragma unroll
        for (int v = 0; v < kPairWaves; ++v) cnt[k] += cw[v][g];
      sum += cnt[k];
    }
    int incl = sum;
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int v = 0; v < w; ++v) run += wsum[v];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int g = kPer * tid + k;
      if (g < ng) {
        a.seg[(size_t)sidx * ng + g] = PairSeg{run, cnt[k]};
        int b = run;
#pragma unroll
        for (int v = 0; v < kPairWaves; ++v) {
          const int t = cw[v][g];
          cw[v][g] = b;
          b += t;
        }
      }
      run += cnt[k];
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_pair_index(const PairIndexArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  if (a.B > kPairMaxBatch || a.slots < 2u * (uint32_t)a.B || a.slots > 2u * kPairMaxBatch ||
      (a.slots & (a.slots - 1)) != 0)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(pair_index_kernel, dim3(kPairSlices), dim3(kSliceThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sfx
