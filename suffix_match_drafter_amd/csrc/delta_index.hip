// delta_index.hip -- per-call index of the delta's occurrences of the batch's tail pairs.
//
// suffix-gpu page, How it works step 2 and Highlights: documents appended since the live
// snapshot are not in the suffix array and are matched by position.  A request's corpus
// candidates there start from the positions x whose token is its last context token and whose
// previous token (still inside the delta) is its second-to-last, with a real token after x.
// The drafter step used to find them by scanning the whole delta in every request.  These
// passes find them once per call for every request at the same time: positions are grouped by
// the pair (token before, token at x), for the pairs that end some request's context, and each
// group keeps position order, which is the logical order the step's site rule needs.
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

// Pass 1 (count) and pass 3 (scatter), workgroups of kPairColsPerBlock wavefronts, one delta
// slice each.  The count pass first builds the table of the batch's tail pairs in LDS: a group
// is named by its first request (the smallest b with that pair), the same in every workgroup
// whatever the order of insertion; workgroup 0 also stores every request's group for the
// step.  The delta's end positions lo + 1 .. hi - 2 are cut into kPairCols slices of whole
// 64-position runs, and wavefront column c takes slice c.  A position belongs to group g when
// (token before, token at it) is group g's pair and a real token follows it.  COUNT: each
// position's group goes to pos_group (for the scatter pass), and the slice's count per group
// to off[g * kPairCols + c] (zeros too, so the scan sees every entry).  Otherwise off
// holds those counts' exclusive prefix within each group and tot the group totals; the
// workgroup derives the group starts (and workgroup 0 stores them), and the slice writes its
// positions' offsets from lo to list[] from base[g] + off[g * kPairCols + c] on, in position
// order within each group.  The workgroup moves its
// block of columns to and from off[] together, so that each group's kPairColsPerBlock
// consecutive entries are one access.
constexpr int kSliceThreads = 64 * kPairColsPerBlock;

template <bool COUNT>
__global__ __launch_bounds__(kSliceThreads) void pair_slices_kernel(PairIndexArgs a) {
  __shared__ unsigned long long hk[2 * kPairMaxBatch];
  __shared__ int hg[2 * kPairMaxBatch];
  __shared__ int cur[kPairColsPerBlock][kPairMaxBatch + 1];
  __shared__ int gbase[kPairMaxBatch + 1];
  const uint32_t mask = a.slots - 1;
  __shared__ int wsum[kPairColsPerBlock];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = blockIdx.x * kPairColsPerBlock + w;
  const int ng = a.B + 1;
  long long lo, hi;
  const bool any = delta_range(a.ctl, &lo, &hi);
  if (!COUNT && !any) return;  // uniform over the grid: the step reads no list
  {
    // the table (at most 2048 slots) and the block's counters, loads issued together; entry
    // e of the block is group e / kPairColsPerBlock of column e % kPairColsPerBlock
    constexpr int kTab = 2 * kPairMaxBatch / kSliceThreads;
    constexpr int kCur = (kPairColsPerBlock * (kPairMaxBatch + 1) + kSliceThreads - 1) / kSliceThreads;
    const int col0 = blockIdx.x * kPairColsPerBlock;
    constexpr int kTot = (kPairMaxBatch + 1 + kSliceThreads - 1) / kSliceThreads;
    constexpr int kReq = kPairMaxBatch / kSliceThreads;
    unsigned long long rk[kReq];
    int tc[kCur], tt[kTot];
#pragma unroll
    for (int j = 0; j < kReq; ++j) {
      const int b = tid + kSliceThreads * j;
      rk[j] = (COUNT && b < a.B) ? tail_pair(a, b) : kNoPair;
    }
#pragma unroll
    for (int j = 0; j < kCur; ++j) {
      const int e = tid + kSliceThreads * j;
      const int g = e / kPairColsPerBlock, c = e % kPairColsPerBlock;
      tc[j] = (!COUNT && g < ng) ? a.off[(int64_t)g * kPairCols + col0 + c] : 0;
    }
    // thread t holds the totals of groups kTot * t .. kTot * t + kTot - 1
#pragma unroll
    for (int j = 0; j < kTot; ++j) {
      const int g = kTot * tid + j;
      tt[j] = (!COUNT && g < ng) ? a.tot[g] : 0;
    }
    if (COUNT) {
#pragma unroll
      for (int j = 0; j < kTab; ++j) {
        const uint32_t i = tid + kSliceThreads * j;
        if (i < a.slots) {
          hk[i] = kNoPair;
          hg[i] = INT32_MAX;
        }
      }
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
      if (blockIdx.x == 0) {
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
    } else {
      // group starts: exclusive prefix of the totals over the workgroup
      int sum = 0;
#pragma unroll
      for (int j = 0; j < kTot; ++j) sum += tt[j];
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
      for (int j = 0; j < kTot; ++j) {
        const int g = kTot * tid + j;
        if (g < ng) {
          gbase[g] = run;
          if (blockIdx.x == 0) a.base[g] = run;
        }
        run += tt[j];
      }
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < kCur; ++j) {
      const int e = tid + kSliceThreads * j;
      const int g = e / kPairColsPerBlock, c = e % kPairColsPerBlock;
      if (g < ng) cur[c][g] = COUNT ? tc[j] : tc[j] + gbase[g];
    }
  }
  __syncthreads();
  const long long nd = any ? hi - lo - 2 : 0;
  if (nd > 0) {
    const long long seg = ((nd + kPairCols - 1) / kPairCols + 63) / 64 * 64;
    const long long xb = lo + 1 + (long long)col * seg;
    const long long xe = xb + seg < hi - 1 ? xb + seg : hi - 1;
    const int cap = (int)a.ring_cap;
    int s = xb < xe ? (int)((xb + lane) % a.ring_cap) : 0;  // slot of this lane's position
    for (long long x0 = xb; x0 < xe; x0 += 64 * kSliceRuns) {
      // COUNT: the tokens around each position; otherwise the group the count pass stored
      int p[kSliceRuns], c[kSliceRuns], nx[kSliceRuns];
#pragma unroll
      for (int u = 0; u < kSliceRuns; ++u) {
        const long long x = x0 + 64 * u + lane;
        const bool in = x < xe;
        if (COUNT) {
          const int sp = s == 0 ? cap - 1 : s - 1;
          const int sn = s + 1 == cap ? 0 : s + 1;
          p[u] = in ? a.ring[sp] : -1;
          c[u] = in ? a.ring[s] : -1;
          nx[u] = in ? a.ring[sn] : -1;
          s += 64;
          while (s >= cap) s -= cap;
        } else {
          p[u] = in ? (int)(int16_t)a.pos_group[x - lo - 1] : -1;
        }
      }
#pragma unroll
      for (int u = 0; u < kSliceRuns; ++u) {
        const long long x = x0 + 64 * u + lane;
        int g = -1;
        if (!COUNT) {
          g = p[u];
        } else if (p[u] >= 0 && nx[u] >= 0) {
          const unsigned long long key = pair_key(p[u], c[u]);
          uint32_t h = pair_hash(key) & mask;
          for (;;) {
            const unsigned long long k = hk[h];
            if (k == key) {
              g = hg[h];
              break;
            }
            if (k == kNoPair) break;
            h = (h + 1) & mask;
          }
        }
        if (COUNT) {
          if (x < xe) a.pos_group[x - lo - 1] = (uint16_t)g;
          if (g >= 0) atomicAdd(&cur[w][g], 1);
        } else {
          // one group at a time: the lanes of group gg take consecutive list entries
          uint64_t pend = __ballot(g >= 0);
          while (pend) {
            const int gg = __builtin_amdgcn_readlane(g, __builtin_ctzll(pend));
            const uint64_t same = __ballot(g == gg);
            const int base = cur[w][gg];
            if (g == gg) a.list[base + __popcll(same & ((1ull << lane) - 1))] = (uint32_t)(x - lo);
            __builtin_amdgcn_wave_barrier();
            if (lane == 0) cur[w][gg] = base + __popcll(same);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            pend &= ~same;
          }
        }
      }
    }
  }
  if (COUNT) {
    __syncthreads();
    const int col0 = blockIdx.x * kPairColsPerBlock;
    for (int e = tid; e < kPairColsPerBlock * ng; e += kSliceThreads) {
      const int g = e / kPairColsPerBlock, c = e % kPairColsPerBlock;
      a.off[(int64_t)g * kPairCols + col0 + c] = cur[c][g];
    }
  }
}

// Pass 2 (one 256-thread workgroup per group g <= B): the exclusive prefix of the group's
// per-slice counts over the slices, in place, and its total.
constexpr int kRowThreads = 256;
constexpr int kRowItems = kPairCols / kRowThreads;

__global__ __launch_bounds__(kRowThreads) void pair_rowscan_kernel(PairIndexArgs a) {
  __shared__ int wsum[kRowThreads / 64];
  long long lo, hi;
  if (!delta_range(a.ctl, &lo, &hi)) return;  // uniform over the grid: the step reads no list
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int32_t* row = a.off + (int64_t)blockIdx.x * kPairCols + kRowItems * tid;
  int v[kRowItems];
#pragma unroll
  for (int j = 0; j < kRowItems; ++j) v[j] = row[j];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kRowItems; ++j) sum += v[j];
  int incl = sum;
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int run = incl - sum, total = 0;
  for (int u = 0; u < kRowThreads / 64; ++u) {
    if (u < w) run += wsum[u];
    total += wsum[u];
  }
#pragma unroll
  for (int j = 0; j < kRowItems; ++j) {
    const int x = v[j];
    row[j] = run;
    run += x;
  }
  if (tid == 0) a.tot[blockIdx.x] = total;
}

}  // namespace

hipError_t launch_pair_index(const PairIndexArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  if (a.B > kPairMaxBatch || a.slots < 2u * (uint32_t)a.B || a.slots > 2u * kPairMaxBatch ||
      (a.slots & (a.slots - 1)) != 0)
    return hipErrorInvalidValue;
  const dim3 grid(kPairCols / kPairColsPerBlock);
  hipLaunchKernelGGL((pair_slices_kernel<true>), grid, dim3(kSliceThreads), 0, st, a);
  hipLaunchKernelGGL(pair_rowscan_kernel, dim3(a.B + 1), dim3(kRowThreads), 0, st, a);
  hipLaunchKernelGGL((pair_slices_kernel<false>), grid, dim3(kSliceThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sfx
