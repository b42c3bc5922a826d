// sa_build.hip -- suffix array by prefix doubling over a stable LSD radix sort, and the n-gram
// probe tables derived from it.
//
// suffix-gpu page, Highlights and References: the cross-request memory is a suffix array built
// by Manber & Myers prefix doubling.  Round h sorts every suffix start i by the pair
// (rank_h[i], rank_h[i+h]) -- rank 0 standing for "past the end", so a proper prefix sorts
// first -- and re-ranks each suffix by the index of the first member of its group.  Rounds stop
// when all ranks differ.  Tokens compare as signed int32, so the -1 document separator sorts
// before every token.
//
// The sort is an LSD radix sort with 8-bit digits: per-tile digit histograms, one exclusive
// scan in digit-major order, then a stable scatter in which each wavefront ranks equal digits
// with eight ballots.  Keys of a round pack both ranks into 2*bits(n) bits so only the needed
// digits are sorted.  A suffix whose rank is already unique keeps its place in every later
// round, so after the first sort each round sorts only the suffixes of groups of two or more:
// they are compacted in suffix-array order, sorted by (group rank, rank at i + h), and written
// back into the same positions, which their groups still occupy.
#include "sa_build.h"

#include <algorithm>

namespace sfx {

namespace {

constexpr int RS_T = 256;              // threads per radix tile
constexpr int RS_I = 16;               // items per thread
static_assert(RS_T * RS_I == kSaRadixTile, "radix tile");
constexpr int SC_T = 1024;             // scan block
constexpr int SC_I = 4;
static_assert(SC_T * SC_I == kSaScanTile, "scan tile");
constexpr int RS_TILE = kSaRadixTile;  // 4096 keys per tile
constexpr int SC_TILE = kSaScanTile;

constexpr int64_t cdiv(int64_t a, int64_t b) { return sa_cdiv(a, b); }

// Element count of a launch: the static bound m, or, when the count lives on the device (mp),
// the smaller of the two.  Grids are sized for the bound; threads past the count do nothing.
__device__ __forceinline__ int64_t dyn_count(int64_t m, const int32_t* mp) {
  if (!mp) return m;
  const int64_t d = *mp;
  return d < m ? d : m;
}

// ------------------------------------------------------------------ generic int32 scans
// Three phases: per-tile reduction, scan of tile totals, per-tile apply.  Op: 0 sum, 1 max.
template <int OP>
__device__ __forceinline__ int sc_op(int a, int b) { return OP == 0 ? a + b : (a > b ? a : b); }

template <int OP>
__device__ int block_scan_incl(int v, int* wbuf) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x = sc_op<OP>(x, y);
  }
  if (lane == 63) wbuf[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int s = lane < SC_T / 64 ? wbuf[lane] : (OP == 0 ? 0 : INT32_MIN);
#pragma unroll
    for (int o = 1; o < SC_T / 64; o <<= 1) {
      int y = __shfl_up(s, o, 64);
      if (lane >= o) s = sc_op<OP>(s, y);
    }
    if (lane < SC_T / 64) wbuf[lane] = s;
  }
  __syncthreads();
  if (wid) x = sc_op<OP>(x, wbuf[wid - 1]);
  __syncthreads();
  return x;
}

template <int OP>
__global__ __launch_bounds__(SC_T) void scan_reduce_kernel(const int32_t* in, int64_t m,
                                                           const int32_t* mp, int32_t* tile_tot) {
  __shared__ int wbuf[SC_T / 64];
  m = dyn_count(m, mp);
  const int64_t base = (int64_t)blockIdx.x * SC_TILE + (int64_t)threadIdx.x * SC_I;
  int acc = OP == 0 ? 0 : INT32_MIN;
  for (int u = 0; u < SC_I; ++u)
    if (base + u < m) acc = sc_op<OP>(acc, in[base + u]);
  int r = block_scan_incl<OP>(acc, wbuf);
  if (threadIdx.x == SC_T - 1) tile_tot[blockIdx.x] = r;
}

// Exclusive scan of the tile totals in one block (loops over chunks of SC_T).
template <int OP>
__global__ __launch_bounds__(SC_T) void scan_tiles_kernel(int32_t* tile_tot, int64_t ntiles) {
  __shared__ int wbuf[SC_T / 64];
  __shared__ int incl_buf[SC_T];
  __shared__ int carry;
  constexpr int ID = OP == 0 ? 0 : INT32_MIN;
  if (threadIdx.x == 0) carry = ID;
  __syncthreads();
  for (int64_t c = 0; c < ntiles; c += SC_T) {
    const int64_t i = c + threadIdx.x;
    const int v = i < ntiles ? tile_tot[i] : ID;
    const int incl = block_scan_incl<OP>(v, wbuf);
    const int cin = carry;
    incl_buf[threadIdx.x] = incl;
    __syncthreads();
    const int excl = threadIdx.x ? sc_op<OP>(cin, incl_buf[threadIdx.x - 1]) : cin;
    if (i < ntiles) tile_tot[i] = excl;
    __syncthreads();
    if (threadIdx.x == SC_T - 1) carry = sc_op<OP>(cin, incl);
    __syncthreads();
  }
}

// Inclusive (INCL=1) or exclusive scan of `in` into `out` with the tile prefixes.
template <int OP, int INCL>
__global__ __launch_bounds__(SC_T) void scan_apply_kernel(const int32_t* in, int32_t* out,
                                                          int64_t m, const int32_t* mp,
                                                          const int32_t* tile_pre) {
  __shared__ int wbuf[SC_T / 64];
  __shared__ int incl_buf[SC_T];
  constexpr int ID = OP == 0 ? 0 : INT32_MIN;
  m = dyn_count(m, mp);
  const int64_t base = (int64_t)blockIdx.x * SC_TILE + (int64_t)threadIdx.x * SC_I;
  int v[SC_I];
  int acc = ID;
#pragma unroll
  for (int u = 0; u < SC_I; ++u) {
    v[u] = base + u < m ? in[base + u] : ID;
    acc = sc_op<OP>(acc, v[u]);
  }
  const int incl = block_scan_incl<OP>(acc, wbuf);
  incl_buf[threadIdx.x] = incl;
  __syncthreads();
  int run = threadIdx.x ? incl_buf[threadIdx.x - 1] : ID;
  run = sc_op<OP>(run, tile_pre[blockIdx.x]);
#pragma unroll
  for (int u = 0; u < SC_I; ++u) {
    const int nxt = sc_op<OP>(run, v[u]);
    if (base + u < m) out[base + u] = INCL ? nxt : run;
    run = nxt;
  }
}

// Scan of in[0, m) into out; with mp, of in[0, min(m, *mp)) (m the bound the grids are sized
// for).
template <int OP, int INCL>
hipError_t scan_i32(const int32_t* in, int32_t* out, int64_t m, int32_t* tmp, hipStream_t st,
                    const int32_t* mp = nullptr) {
  if (m <= 0) return hipSuccess;
  const int64_t nt = cdiv(m, SC_TILE);
  hipLaunchKernelGGL((scan_reduce_kernel<OP>), dim3(nt), dim3(SC_T), 0, st, in, m, mp, tmp);
  hipLaunchKernelGGL((scan_tiles_kernel<OP>), dim3(1), dim3(SC_T), 0, st, tmp, nt);
  hipLaunchKernelGGL((scan_apply_kernel<OP, INCL>), dim3(nt), dim3(SC_T), 0, st, in, out, m, mp,
                     tmp);
  return hipGetLastError();
}

// ------------------------------------------------------------------ stable LSD radix sort
template <typename K>
__global__ __launch_bounds__(RS_T) void rs_hist_kernel(const K* keys, int64_t n, const int32_t* mp,
                                                       int shift, int32_t* hist, int64_t ntiles) {
  __shared__ int h[256];
  n = dyn_count(n, mp);
  h[threadIdx.x] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * RS_TILE;
#pragma unroll 4
  for (int i = 0; i < RS_I; ++i) {
    const int64_t e = base + (int64_t)i * RS_T + threadIdx.x;
    if (e < n) atomicAdd(&h[(int)((keys[e] >> shift) & 255)], 1);
  }
  __syncthreads();
  hist[(int64_t)threadIdx.x * ntiles + blockIdx.x] = h[threadIdx.x];
}

template <typename K>
__global__ __launch_bounds__(RS_T) void rs_scatter_kernel(const K* kin, const int32_t* vin,
                                                          K* kout, int32_t* vout, int64_t n,
                                                          const int32_t* mp, int shift,
                                                          const int32_t* offs, int64_t ntiles) {
  __shared__ int run[256];
  n = dyn_count(n, mp);
  if ((int64_t)blockIdx.x * RS_TILE >= n) return;  // (the whole block: every key past the count)
  __shared__ int gbase[256];
  __shared__ int wcnt[RS_T / 64][256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  run[tid] = 0;
  gbase[tid] = offs[(int64_t)tid * ntiles + blockIdx.x];
#pragma unroll
  for (int x = 0; x < RS_T / 64; ++x) wcnt[x][tid] = 0;
  __syncthreads();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t base = (int64_t)blockIdx.x * RS_TILE;
  for (int r = 0; r < RS_I; ++r) {
    const int64_t e = base + (int64_t)r * RS_T + tid;
    const bool valid = e < n;
    const K key = valid ? kin[e] : K(0);
    const int32_t val = valid ? vin[e] : 0;
    const int d = (int)((key >> shift) & 255);
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const uint64_t bb = __ballot(valid && ((d >> bit) & 1));
      m &= ((d >> bit) & 1) ? bb : ~bb;
    }
    const int wrank = __popcll(m & below);
    if (valid && wrank == 0) wcnt[w][d] = __popcll(m);
    __syncthreads();
    int pre = 0;
    if (valid) {
      pre = run[d];
      for (int x = 0; x < w; ++x) pre += wcnt[x][d];
    }
    __syncthreads();
    {
      int s = 0;
#pragma unroll
      for (int x = 0; x < RS_T / 64; ++x) {
        s += wcnt[x][tid];
        wcnt[x][tid] = 0;
      }
      run[tid] += s;
    }
    if (valid) {
      const int64_t pos = (int64_t)gbase[d] + pre + wrank;
      kout[pos] = key;
      vout[pos] = val;
    }
    __syncthreads();
  }
}

// Sorts (k[0..n), v[0..n)) by the key bits [0, bits) stably; the result ends in buffer
// `*which` (0: k0/v0, 1: k1/v1).  With mp the count is min(n, *mp), read on the device (n
// sizes the grids; the passes run whatever the count, so *which does not depend on it).
template <typename K>
hipError_t radix_sort(K* k0, int32_t* v0, K* k1, int32_t* v1, int64_t n, int bits,
                      int32_t* hist, int32_t* tmp, int* which, hipStream_t st,
                      const int32_t* mp = nullptr) {
  *which = 0;
  if (n <= 1 && !mp) return hipSuccess;
  if (n <= 0) return hipSuccess;
  const int64_t nt = cdiv(n, RS_TILE);
  K* ka = k0;
  int32_t* va = v0;
  K* kb = k1;
  int32_t* vb = v1;
  for (int shift = 0; shift < bits; shift += 8) {
    hipLaunchKernelGGL((rs_hist_kernel<K>), dim3(nt), dim3(RS_T), 0, st, ka, n, mp, shift, hist,
                       nt);
    hipError_t e = scan_i32<0, 0>(hist, hist, 256 * nt, tmp, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((rs_scatter_kernel<K>), dim3(nt), dim3(RS_T), 0, st, ka, va, kb, vb, n,
                       mp, shift, hist, nt);
    std::swap(ka, kb);
    std::swap(va, vb);
    *which ^= 1;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ prefix doubling kernels
__global__ __launch_bounds__(256) void minmax_kernel(const int32_t* text, int64_t n,
                                                     int32_t* mm) {
  __shared__ int slo[4], shi[4];
  int lo = INT32_MAX, hi = INT32_MIN;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int v = text[i];
    lo = v < lo ? v : lo;
    hi = v > hi ? v : hi;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const int a = __shfl_xor(lo, o, 64), b = __shfl_xor(hi, o, 64);
    lo = a < lo ? a : lo;
    hi = b > hi ? b : hi;
  }
  if ((threadIdx.x & 63) == 0) {
    slo[threadIdx.x >> 6] = lo;
    shi[threadIdx.x >> 6] = hi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) {
      lo = slo[w] < lo ? slo[w] : lo;
      hi = shi[w] > hi ? shi[w] : hi;
    }
    atomicMin(&mm[0], lo);
    atomicMax(&mm[1], hi);
  }
}

// First keys: the tokens minus the smallest one (mm[0], found on the device), as 32-bit keys.
__global__ void init_keys_kernel(const int32_t* text, int64_t n, const int32_t* mm, uint64_t* k,
                                 int32_t* v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  k[i] = (uint64_t)(uint32_t)((int64_t)text[i] - mm[0]);
  v[i] = (int32_t)i;
}

// mm[0], mm[1]: the token range to find; gate: open (a round runs) until a round finds no
// suffix left to sort.
__global__ void minmax_init_kernel(int32_t* mm, int32_t* gate) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    mm[0] = INT32_MAX;
    mm[1] = INT32_MIN;
    *gate = INT32_MAX;
  }
}

// head[j] = j+1 if key[j] differs from key[j-1] (or j == 0), else 0; any equal neighbour
// raises *dup (a plain store of the same value from any number of wavefronts).
__global__ void heads_kernel(const uint64_t* k, int64_t n, int32_t* head, uint32_t* dup) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  bool same = false;
  if (j < n) {
    same = j > 0 && k[j] == k[j - 1];
    head[j] = same ? 0 : (int32_t)(j + 1);
  }
  if (__ballot(same) && (threadIdx.x & 63) == 0) *dup = 1u;
}

// rank[v[j]] = index + 1 of the first member of j's group (inclusive max scan of heads)
__global__ void rank_kernel(const int32_t* v, const int32_t* headmax, int64_t n, int32_t* rank) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < n) rank[v[j]] = headmax[j];
}

// cnt[j] = 1 when position j's group has two or more members (heads: nonzero at group starts).
// Nothing once the gate is shut.
__global__ void active_flags_kernel(const int32_t* head, int64_t n, const int32_t* gate,
                                    int32_t* cnt) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= dyn_count(n, gate)) return;
  const bool single = head[j] != 0 && (j + 1 == n || head[j + 1] != 0);
  cnt[j] = single ? 0 : 1;
}

// incl[j]: active positions in [0, j].  The t-th active position gets its suffix i, the key
// (rank[i] << bits) | rank[i + h] (0 past the end), and its position.  The number of active
// positions goes to *m (the round's sort size, read by the round's other kernels), and the
// gate shuts when it is 0.  Nothing once the gate is shut (*m is 0 by then).
__global__ void gather_active_kernel(const int32_t* incl, const int32_t* sa, const int32_t* rank,
                                     int64_t n, int64_t h, int bits, int32_t* act, uint64_t* k,
                                     int32_t* v, int32_t* m, int32_t* gate) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n || *gate == 0) return;
  const int c = incl[j];
  if (j == n - 1) {
    *m = c;
    if (c == 0) *gate = 0;
  }
  if (c == (j ? incl[j - 1] : 0)) return;  // not active
  const int t = c - 1;
  const int64_t i = sa[j];
  const uint64_t r1 = (uint32_t)rank[i];
  const uint64_t r2 = i + h < n ? (uint32_t)rank[i + h] : 0u;
  k[t] = (r1 << bits) | r2;
  v[t] = (int32_t)i;
  act[t] = (int32_t)j;
}

// The sorted active suffixes back into their positions; a new group starts wherever the key
// changes, and hv[t] = position + 1 at a start (else 0) for the max scan that ranks them.
__global__ void scatter_back_kernel(const int32_t* act, const uint64_t* k, const int32_t* v,
                                    int64_t m, const int32_t* mp, int32_t* sa, int32_t* head,
                                    int32_t* hv) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= dyn_count(m, mp)) return;
  const int32_t p = act[t];
  sa[p] = v[t];
  const bool start = t == 0 || k[t] != k[t - 1];
  head[p] = start ? p + 1 : 0;
  hv[t] = start ? p + 1 : 0;
}

__global__ void rerank_kernel(const int32_t* v, const int32_t* hmax, int64_t m, const int32_t* mp,
                              int32_t* rank) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < dyn_count(m, mp)) rank[v[t]] = hmax[t];
}

__global__ void copy_i32_kernel(const int32_t* a, int32_t* b, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) b[i] = a[i];
}

inline int bits_for(uint64_t maxv) {
  int b = 0;
  while (b < 64 && (maxv >> b) != 0) ++b;
  return b < 1 ? 1 : b;
}

}  // namespace

// ------------------------------------------------------------------ workspace
size_t sa_workspace_bytes(int64_t n) { return sa_ws_bytes(n); }

SaWork sa_carve(void* ws, int64_t n) {
  const int64_t nn = n < 1 ? 1 : n;
  const int64_t nt = cdiv(nn, RS_TILE);
  uintptr_t p = ((uintptr_t)ws + 255) & ~(uintptr_t)255;
  auto take = [&](size_t bytes) {
    void* r = (void*)p;
    p = (p + bytes + 255) & ~(uintptr_t)255;
    return r;
  };
  SaWork w;
  w.k0 = (uint64_t*)take(sizeof(uint64_t) * nn);
  w.k1 = (uint64_t*)take(sizeof(uint64_t) * nn);
  w.v0 = (int32_t*)take(sizeof(int32_t) * nn);
  w.v1 = (int32_t*)take(sizeof(int32_t) * nn);
  w.rank = (int32_t*)take(sizeof(int32_t) * nn);
  w.head = (int32_t*)take(sizeof(int32_t) * nn);
  w.aux = (int32_t*)take(sizeof(int32_t) * nn);
  w.act = (int32_t*)take(sizeof(int32_t) * nn);
  w.hist = (int32_t*)take(sizeof(int32_t) * (256 * nt + 64));
  w.tiles = (int32_t*)take(sizeof(int32_t) * (cdiv(256 * nt + nn, SC_TILE) + 64));
  w.counters = (uint32_t*)take(256);
  w.n = nn;
  return w;
}

hipError_t sa_build(const int32_t* text, int64_t n, int32_t* sa, const SaWork& w, hipStream_t st,
                    const SaPoll* poll, int* rounds_out) {
  if (rounds_out) *rounds_out = 0;
  if (n <= 0) return hipSuccess;
  const int TB = 256;
  const int64_t gb = cdiv(n, TB);
  int32_t* mm = (int32_t*)w.counters;       // token range
  int32_t* mdev = (int32_t*)w.counters + 4;  // the current round's sort size
  int32_t* gate = (int32_t*)w.counters + 5;  // INT32_MAX while rounds run, then 0
  // first sort: by token, on 32-bit keys relative to the smallest token (found on the device)
  hipLaunchKernelGGL(minmax_init_kernel, dim3(1), dim3(64), 0, st, mm, gate);
  hipLaunchKernelGGL(minmax_kernel, dim3((unsigned)std::min<int64_t>(gb, 256)), dim3(TB), 0, st,
                     text, n, mm);
  hipLaunchKernelGGL(init_keys_kernel, dim3(gb), dim3(TB), 0, st, text, n, mm, w.k0, w.v0);
  int which = 0;
  hipError_t e = radix_sort<uint64_t>(w.k0, w.v0, w.k1, w.v1, n, 32, w.hist, w.tiles, &which, st);
  if (e != hipSuccess) return e;
  uint64_t* kc = which ? w.k1 : w.k0;
  int32_t* vc = which ? w.v1 : w.v0;
  // round 0 ranks: groups of equal first tokens
  hipLaunchKernelGGL(copy_i32_kernel, dim3(gb), dim3(TB), 0, st, vc, sa, n);
  hipLaunchKernelGGL(heads_kernel, dim3(gb), dim3(TB), 0, st, kc, n, w.head, w.counters + 8);
  if ((e = scan_i32<1, 1>(w.head, w.aux, n, w.tiles, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(rank_kernel, dim3(gb), dim3(TB), 0, st, vc, w.aux, n, w.rank);
  // Doubling rounds h = 1, 2, 4, ... < n.  Each sorts the suffixes still sharing a rank; how
  // many there are is counted on the device and read there by the round's kernels, so a round
  // after convergence does nothing.  Without a poll every round is enqueued; with one, the
  // host reads each round's count through pinned memory kPollLag rounds late (the device is
  // still busy with the rounds in between) and stops enqueueing once a count is 0.
  const int rbits = bits_for((uint64_t)n);
  int rounds = 1, r = 0;
  bool known_done = false;
  for (int64_t h = 1; h < n && !known_done; h *= 2, ++r) {
    hipLaunchKernelGGL(active_flags_kernel, dim3(gb), dim3(TB), 0, st, w.head, n, gate, w.aux);
    if ((e = scan_i32<0, 1>(w.aux, w.aux, n, w.tiles, st, gate)) != hipSuccess) return e;
    hipLaunchKernelGGL(gather_active_kernel, dim3(gb), dim3(TB), 0, st, w.aux, sa, w.rank, n, h,
                       rbits, w.act, w.k0, w.v0, mdev, gate);
    e = radix_sort<uint64_t>(w.k0, w.v0, w.k1, w.v1, n, 2 * rbits, w.hist, w.tiles, &which, st,
                             mdev);
    if (e != hipSuccess) return e;
    const uint64_t* ks = which ? w.k1 : w.k0;
    const int32_t* vs = which ? w.v1 : w.v0;
    hipLaunchKernelGGL(scatter_back_kernel, dim3(gb), dim3(TB), 0, st, w.act, ks, vs, n, mdev, sa,
                       w.head, w.aux);
    if ((e = scan_i32<1, 1>(w.aux, w.aux, n, w.tiles, st, mdev)) != hipSuccess) return e;
    hipLaunchKernelGGL(rerank_kernel, dim3(gb), dim3(TB), 0, st, vs, w.aux, n, mdev, w.rank);
    if (poll && r < kPollRounds) {
      if ((e = hipMemcpyAsync(poll->counts + r, mdev, sizeof(int32_t), hipMemcpyDeviceToHost,
                              st)) != hipSuccess)
        return e;
      if ((e = hipEventRecord(poll->ev[r], st)) != hipSuccess) return e;
      if (r >= kPollLag) {
        if ((e = hipEventSynchronize(poll->ev[r - kPollLag])) != hipSuccess) return e;
        known_done = poll->counts[r - kPollLag] == 0;
      }
    }
  }
  if (poll) const_cast<SaPoll*>(poll)->enqueued = r < kPollRounds ? r : kPollRounds;
  if (rounds_out) {
    // the rounds that sorted something, plus the first sort (one more wait, at the end)
    if (poll) {
      const int last = r < kPollRounds ? r : kPollRounds;
      if (last > 0 && (e = hipEventSynchronize(poll->ev[last - 1])) != hipSuccess) return e;
      for (int i = 0; i < last && poll->counts[i] > 0; ++i) ++rounds;
    }
    *rounds_out = rounds;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ n-gram probe tables
namespace {

// The flags of all three n-gram lengths from one gather of each suffix's first kNG + 2 tokens
// (and its suffix-array predecessor's): bit g of flags[j] = the (g+2)-gram at sa[j] continues,
// bit 8 + g = it also starts a group (its predecessor's differs or does not continue).
__global__ void ng_flags_kernel(const int32_t* text, const int32_t* sa, int64_t n,
                                int32_t* flags) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  constexpr int W = kNG + 2;  // tokens that decide the longest n-gram and its continuation
  const int64_t i = sa[j];
  int t[W], q[W];
#pragma unroll
  for (int x = 0; x < W; ++x) t[x] = i + x < n ? text[i + x] : -1;
  const int64_t p = j > 0 ? sa[j - 1] : -1;
#pragma unroll
  for (int x = 0; x < W; ++x) q[x] = p >= 0 && p + x < n ? text[p + x] : -1;
  int f = 0;
  bool okt = t[0] >= 0 && t[1] >= 0, okq = q[0] >= 0 && q[1] >= 0, same = t[0] == q[0];
#pragma unroll
  for (int g = 0; g < kNG; ++g) {
    const int ng = g + 2;
    okt = okt && t[ng] >= 0;      // tokens 0..ng real: the n-gram and its next token
    okq = okq && q[ng] >= 0;
    same = same && t[ng - 1] == q[ng - 1];
    if (okt) f |= 1 << g;
    if (okt && !(okq && same)) f |= 1 << (8 + g);
  }
  flags[j] = f;
}

__global__ void ng_unpack_kernel(const int32_t* flags, int64_t n, int g, int32_t* valid,
                                 int32_t* head) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const int f = flags[j];
  valid[j] = (f >> g) & 1;
  head[j] = (f >> (8 + g)) & 1;
}

// At each group head: record the group's offset in the position list by group id.
__global__ void ng_heads_kernel(const int32_t* head, const int32_t* gid_incl,
                                const int32_t* cvalid_excl, int64_t n, int32_t* goff) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  if (head[j]) goff[gid_incl[j] - 1] = cvalid_excl[j];
}

__global__ void ng_total_kernel(const int32_t* valid, const int32_t* cvalid_excl,
                                const int32_t* gid_incl, int64_t n, int32_t* goff,
                                int32_t* ngroups) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const int32_t G = gid_incl[n - 1];
  goff[G] = cvalid_excl[n - 1] + valid[n - 1];
  *ngroups = G;
}

// Group key of every position (by suffix-array scatter) and the hash insert of each group.
__global__ void ng_groups_kernel(const int32_t* text, const int32_t* sa, int64_t n, int ng,
                                 const int32_t* valid, const int32_t* head,
                                 const int32_t* gid_incl, const int32_t* goff,
                                 const int32_t* ngroups, uint32_t* gkey, NgramSlot* ht,
                                 uint32_t mask) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const int64_t i = sa[j];
  const uint32_t none = (uint32_t)(*ngroups);
  gkey[i] = valid[j] ? (uint32_t)(gid_incl[j] - 1) : none;
  if (!head[j]) return;
  const int32_t g = gid_incl[j] - 1;
  int key[4] = {-1, -1, -1, -1};
  for (int x = 0; x < ng; ++x) key[x] = text[i + x];
  uint32_t h = ngram_hash(key, ng) & mask;
  for (;;) {
    const int prev = atomicCAS(&ht[h].owner, 0, g + 1);
    if (prev == 0) break;
    h = (h + 1) & mask;
  }
  for (int x = 0; x < 4; ++x) ht[h].key[x] = key[x];
  ht[h].off = goff[g];
  ht[h].cnt = goff[g + 1] - goff[g];
  ht[h].sa_lo = (int32_t)j;
}

__global__ void iota_kernel(int32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = (int32_t)i;
}

}  // namespace

hipError_t ngram_tables_build(const int32_t* text, const int32_t* sa, int64_t n, int32_t* pl[kNG],
                              NgramSlot* ht[kNG], uint32_t ht_slots, const SaWork& w,
                              hipStream_t st) {
  if (n <= 0) {
    // an empty snapshot still gets empty tables, so every probe ends at an empty slot
    for (int g = 0; g < kNG; ++g) {
      hipError_t e = hipMemsetAsync(ht[g], 0, sizeof(NgramSlot) * (size_t)ht_slots, st);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int TB = 256;
  const int64_t gb = cdiv(n, TB);
  const uint32_t mask = ht_slots - 1;
  // workspace reuse: valid/head/gid/cvalid in the int32 arrays, group offsets in k1 (before
  // the sort needs it), group keys of positions in k0 (as uint32)
  int32_t* valid = w.head;
  int32_t* head = w.rank;
  int32_t* gid = w.aux;
  int32_t* cval = w.v1;
  int32_t* goff = (int32_t*)w.k1;
  uint32_t* gkey0 = (uint32_t*)w.k0;
  uint32_t* gkey1 = (uint32_t*)w.k1;
  int32_t* ngroups = (int32_t*)(w.counters + 16);
  const int kbits = bits_for((uint64_t)n);
  hipError_t e;
  hipLaunchKernelGGL(ng_flags_kernel, dim3(gb), dim3(TB), 0, st, text, sa, n, w.act);
  for (int g = 0; g < kNG; ++g) {
    const int ng = g + 2;
    hipLaunchKernelGGL(ng_unpack_kernel, dim3(gb), dim3(TB), 0, st, w.act, n, g, valid, head);
    if ((e = scan_i32<0, 1>(head, gid, n, w.tiles, st)) != hipSuccess) return e;
    if ((e = scan_i32<0, 0>(valid, cval, n, w.tiles, st)) != hipSuccess) return e;
    hipLaunchKernelGGL(ng_heads_kernel, dim3(gb), dim3(TB), 0, st, head, gid, cval, n, goff);
    hipLaunchKernelGGL(ng_total_kernel, dim3(1), dim3(64), 0, st, valid, cval, gid, n, goff,
                       ngroups);
    if ((e = hipMemsetAsync(ht[g], 0, sizeof(NgramSlot) * (size_t)ht_slots, st)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(ng_groups_kernel, dim3(gb), dim3(TB), 0, st, text, sa, n, ng, valid, head,
                       gid, goff, ngroups, gkey0, ht[g], mask);
    // positions in increasing order, stably sorted by group id: each group's occurrences
    // end up in position order
    hipLaunchKernelGGL(iota_kernel, dim3(gb), dim3(TB), 0, st, w.v0, n);
    int which = 0;
    e = radix_sort<uint32_t>(gkey0, w.v0, gkey1, pl[g], n, kbits, w.hist, w.tiles, &which, st);
    if (e != hipSuccess) return e;
    if (!which) hipLaunchKernelGGL(copy_i32_kernel, dim3(gb), dim3(TB), 0, st, w.v0, pl[g], n);
  }
  return hipGetLastError();
}

}  // namespace sfx
