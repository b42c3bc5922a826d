// accept.hip -- per-slot acceptance estimate of the drafts, learned online.
//
// vLLM docs "Suffix Decoding", Use adaptive verification at higher concurrency: the drafter
// keeps, for each draft position, a running estimate of how likely it is to be accepted,
// keyed by where the draft came from and how long its match was; the scheduler uses it to
// skip verifying positions that are unlikely to pay off.
//
// sfx_propose records each request's winner (source: local or corpus; its match length; the
// number of drafted tokens).  Verifier feedback then adds, for every drafted slot d, one
// proposal to the (source, length, d) cell, and one acceptance when the request accepted more
// than d tokens (accepted tokens form a prefix of the draft).  The estimate of a cell is
// Laplace's rule of succession, (accepted + 1) / (proposed + 2), in parts per million.
#include "accept.h"

namespace sfx {

namespace {

__device__ __forceinline__ size_t cell(int src, int len, int d) {
  return (((size_t)src * kAcceptLens + len) * kMaxK + d) * 2;
}

// One workgroup.  Every request adds one to the histograms of its cell (source, length): by its
// draft length nv and by its accepted count na (clamped to [0, nv]); a slot d of the cell was
// then proposed by the requests with nv > d and accepted by those with na > d (suffix sums),
// which go to the table with one atomic per nonzero count.  Consumes the picks (a second
// feedback for the same propose adds nothing).
constexpr int kFeedbackThreads = 1024;
constexpr int kHistBins = kMaxK + 1;  // nv and na range over 0..kMaxK

__global__ __launch_bounds__(kFeedbackThreads) void accept_feedback_kernel(
    int B, int32_t* pick, const int32_t* num_accepted, unsigned long long* table) {
  __shared__ int hnv[2 * kAcceptLens * kHistBins];
  __shared__ int hna[2 * kAcceptLens * kHistBins];
  const int tid = threadIdx.x;
  for (int i = tid; i < 2 * kAcceptLens * kHistBins; i += kFeedbackThreads) hnv[i] = hna[i] = 0;
  __syncthreads();
  for (int b = tid; b < B; b += kFeedbackThreads) {
    const int p = pick[b];
    if (p < 0) continue;
    pick[b] = -1;
    const int nv = (p >> 16) & 0xff, src = (p >> 8) & 1, len = p & 0xff;
    if (nv <= 0 || nv > kMaxK || len > kMaxD) continue;
    int na = num_accepted[b];
    na = na < 0 ? 0 : (na > nv ? nv : na);
    const int base = (src * kAcceptLens + len) * kHistBins;
    atomicAdd(&hnv[base + nv], 1);
    atomicAdd(&hna[base + na], 1);
  }
  __syncthreads();
  for (int cl = tid; cl < 2 * kAcceptLens; cl += kFeedbackThreads) {
    const int base = cl * kHistBins;
    int prop = 0, acc = 0;
    for (int d = kMaxK - 1; d >= 0; --d) {  // requests with nv > d, with na > d
      prop += hnv[base + d + 1];
      acc += hna[base + d + 1];
      unsigned long long* c = table + ((size_t)cl * kMaxK + d) * 2;
      if (prop) atomicAdd(c, (unsigned long long)prop);
      if (acc) atomicAdd(c + 1, (unsigned long long)acc);
    }
  }
}

// One thread per (request, slot): slots past the draft get 0.
__global__ void accept_estimate_kernel(int B, int k, const int32_t* pick,
                                       const unsigned long long* table, int32_t* est) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)B * k) return;
  const int b = (int)(i / k), d = (int)(i % k);
  const int p = pick[b];
  int e = 0;
  if (p >= 0) {
    const int nv = (p >> 16) & 0xff, src = (p >> 8) & 1, len = p & 0xff;
    if (d < nv && d < kMaxK && len <= kMaxD) {
      const unsigned long long* c = table + cell(src, len, d);
      const unsigned long long prop = c[0], acc = c[1];
      e = (int)((1000000ull * (acc + 1)) / (prop + 2));
    }
  }
  est[i] = e;
}

__global__ void accept_reset_kernel(unsigned long long* table, int32_t* pick, int rows) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < kAcceptEntries) table[i] = 0;
  if (i < (size_t)rows) pick[i] = -1;
}

}  // namespace

hipError_t launch_accept_feedback(int B, int32_t* pick, const int32_t* num_accepted,
                                  unsigned long long* table, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(accept_feedback_kernel, dim3(1), dim3(kFeedbackThreads), 0, st, B, pick,
                     num_accepted, table);
  return hipGetLastError();
}

hipError_t launch_accept_estimate(int B, int k, const int32_t* pick,
                                  const unsigned long long* table, int32_t* est_ppm,
                                  hipStream_t st) {
  const long long n = (long long)B * k;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(accept_estimate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     B, k, pick, table, est_ppm);
  return hipGetLastError();
}

hipError_t launch_accept_reset(unsigned long long* table, int32_t* pick, int rows,
                               hipStream_t st) {
  const size_t n = kAcceptEntries > (size_t)rows ? kAcceptEntries : (size_t)rows;
  hipLaunchKernelGGL(accept_reset_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     table, pick, rows);
  return hipGetLastError();
}

}  // namespace sfx
