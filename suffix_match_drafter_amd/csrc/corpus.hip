// corpus.hip -- the shared corpus on the device: ingest (scatter_append), eviction, snapshot of
// the live documents for an index rebuild, and the swap that makes a rebuilt index live.
//
// suffix-gpu page, How it works step 4: new documents are appended, the oldest are evicted when
// the ring is full, and a suffix array rebuilt off the critical path is swapped in without moving
// buffers.  vLLM docs "Suffix Decoding", Model Runner V2: the corpus has a token budget and
// drops the oldest first.  Every decision is taken on the device from the control block, so the
// host never reads a device value on the ingest path.
#include "corpus.h"

namespace sfx {

namespace {

constexpr int PT = 1024;  // plan kernel threads

// Length of entry r's document, or -1 when the entry appends no document at all.
__device__ __forceinline__ int64_t doc_len(const IngestArgs& a, int r) {
  if (a.doc_offsets) {
    const int64_t l = a.doc_offsets[r + 1] - a.doc_offsets[r];
    return l < 0 ? 0 : l;
  }
  if (a.seg_len) return a.seg_len[r];
  const int row = a.row_indices[r];
  if (row < 0 || row >= a.num_rows) return 0;
  int l = a.lengths[r];
  return l < 0 ? 0 : (l > a.S ? a.S : l);
}

__device__ __forceinline__ const int32_t* doc_src(const IngestArgs& a, int r) {
  if (a.doc_offsets) return a.tokens + a.doc_offsets[r];
  const int row = a.row_indices[r];
  const int32_t* base = a.tokens + (int64_t)(row < 0 ? 0 : row) * a.S;
  return a.seg_start ? base + a.seg_start[r] : base;
}

// Offsets of the new documents (each takes len + 1 ring tokens), new head, and the eviction
// that keeps the longest run of most recent documents fitting in the capacity.
// Each entry's value packs its ring tokens above bit 20 and its document count (0 or 1) below, so
// one scan gives both the offsets and the document numbers (at most 2^16 entries per launch).
constexpr int kDocBits = 20;
__global__ __launch_bounds__(PT) void ingest_plan_kernel(IngestArgs a) {
  __shared__ int64_t wsum[PT / 64];
  __shared__ int64_t carry;
  __shared__ int64_t s_base, s_doc_tail;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int c = 0; c < a.R; c += PT) {
    const int r = c + tid;
    const int64_t l = r < a.R ? doc_len(a, r) : -1;
    const int64_t v = l >= 0 ? ((l + 1) << kDocBits) | 1 : 0;
    int64_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    __syncthreads();
    int64_t pre = carry;
    for (int w = 0; w < wid; ++w) pre += wsum[w];
    if (r < a.R) {
      const int64_t before = pre + x - v;
      a.doc_off[r] = before >> kDocBits;
      a.doc_idx[r] = (int32_t)(before & ((1 << kDocBits) - 1));
    }
    __syncthreads();
    if (tid == PT - 1) carry = pre + x;
    __syncthreads();
  }
  Ctl* ctl = a.ctl;
  if (tid == 0) {
    const int64_t total = carry >> kDocBits;
    const int32_t ndocs = (int32_t)(carry & ((1 << kDocBits) - 1));
    a.doc_off[a.R] = total;
    a.doc_idx[a.R] = ndocs;
    const int64_t base = ctl->head;
    const int64_t new_head = base + total;
    const int64_t thr = new_head - a.cap;
    int64_t new_tail = ctl->tail, new_doc_tail = ctl->doc_tail;
    const int64_t dh = ctl->doc_head;
    if (thr > ctl->tail) {
      int64_t lo = ctl->doc_tail, hi = dh;
      while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (a.doc_start[mid % a.dcap] < thr) lo = mid + 1;
        else hi = mid;
      }
      if (lo < dh) {
        new_tail = a.doc_start[lo % a.dcap];
        new_doc_tail = lo;
      } else {
        int rl = 0, rh = a.R;
        while (rl < rh) {
          const int mid = (rl + rh) >> 1;
          if (base + a.doc_off[mid] < thr) rl = mid + 1;
          else rh = mid;
        }
        new_tail = rl < a.R ? base + a.doc_off[rl] : new_head;
        new_doc_tail = dh + a.doc_idx[rl];
      }
    }
    s_base = base;
    s_doc_tail = new_doc_tail;
    ctl->ingest_base = base;
    ctl->head = new_head;
    ctl->tail = new_tail;
    ctl->doc_head = dh + ndocs;
    ctl->doc_tail = new_doc_tail;
    carry = dh;
  }
  __syncthreads();
  const int64_t dh = carry, base = s_base, ndt = s_doc_tail;
  for (int r = tid; r < a.R; r += PT) {
    const int64_t d = dh + a.doc_idx[r];
    if (doc_len(a, r) >= 0 && d >= ndt) a.doc_start[d % a.dcap] = base + a.doc_off[r];
  }
}

// In-flight ingest, per entry r: a row listed again later in the same call is claimed by its
// first entry only (claim = the smallest r); the claimed entry's chunk is the row's tokens past
// its cursor, appended once it holds min_chunk tokens or, with final_flags[r], whenever it is not
// empty.  The cursor then moves to the row's length, or back to 0 after a final flush.  A length
// below the cursor means the row was reused without a flush: its cursor restarts at 0.
__global__ void inflight_claim_kernel(InflightArgs a) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= a.R) return;
  const int row = a.row_indices[r];
  if (row >= 0 && row < a.num_rows && row < a.max_rows) atomicMin(&a.claim[row], r);
}

__global__ void inflight_prepare_kernel(InflightArgs a) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= a.R) return;
  const int row = a.row_indices[r];
  int start = 0, len = -1;
  if (row >= 0 && row < a.num_rows && row < a.max_rows && a.claim[row] == r) {
    int n = a.lengths[r];
    n = n < 0 ? 0 : (n > a.S ? a.S : n);
    int c = a.cursor[row];
    if (n < c) c = 0;
    const bool fin = a.final_flags && a.final_flags[r] != 0;
    const int chunk = n - c;
    const int need = a.min_chunk > 1 ? a.min_chunk : 1;
    const bool take = chunk >= need || (fin && chunk > 0);
    if (take) {
      start = c;
      len = chunk;
    }
    a.cursor[row] = fin ? 0 : (take ? n : c);
    a.claim[row] = 0x7fffffff;
  }
  a.seg_start[r] = start;
  a.seg_len[r] = len;
}

__global__ void claims_init_kernel(int32_t* claim, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) claim[i] = 0x7fffffff;
}

// Ring slots of a grid-stride walk: one division per thread, then steps of stride % cap.
struct SlotWalk {
  int64_t slot, step, cap;
  __device__ SlotWalk(int64_t pos, int64_t stride, int64_t m)
      : slot(pos % m), step(stride % m), cap(m) {}
  __device__ void next() {
    slot += step;
    if (slot >= cap) slot -= cap;
  }
};

// Copy the surviving tokens of document blockIdx.x (and its -1 separator) into the ring.
__global__ __launch_bounds__(256) void ingest_scatter_kernel(IngestArgs a) {
  const int r = blockIdx.x;
  const int64_t len = doc_len(a, r);
  if (len < 0) return;  // no document
  const int32_t* src = doc_src(a, r);
  const int64_t start = a.ctl->ingest_base + a.doc_off[r];
  const int64_t live_from = a.ctl->tail;
  const int64_t x0 = (int64_t)blockIdx.y * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.y * blockDim.x;
  SlotWalk w(start + x0, stride, a.cap);
  for (int64_t x = x0; x <= len; x += stride, w.next())
    if (start + x >= live_from) a.ring[w.slot] = x < len ? src[x] : -1;
}

// Linear copy of the live corpus [tail, head) into a snapshot text; records its range.
__global__ void snapshot_kernel(Ctl* ctl, const int32_t* ring, int64_t cap, int32_t* text,
                                int buf, int64_t* range_out) {
  const int64_t tail = ctl->tail, head = ctl->head;
  const int64_t n = head - tail;
  const int64_t x0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  SlotWalk w(tail + x0, stride, cap);
  for (int64_t x = x0; x < n; x += stride, w.next()) text[x] = ring[w.slot];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ctl->pending_start = tail;
    ctl->pending_end = head;
    ctl->pending = buf;
    if (range_out) {
      range_out[0] = tail;
      range_out[1] = head;
    }
  }
}

__global__ void swap_kernel(Ctl* ctl, int buf, uint32_t mask) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  ctl->snap_start[buf] = ctl->pending_start;
  ctl->snap_end[buf] = ctl->pending_end;
  ctl->ht_mask[buf] = mask;
  ctl->active = buf;
  ctl->pending = -1;
}

__global__ void ctl_init_kernel(Ctl* ctl) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  ctl->head = ctl->tail = ctl->doc_head = ctl->doc_tail = 0;
  ctl->snap_start[0] = ctl->snap_start[1] = ctl->snap_end[0] = ctl->snap_end[1] = 0;
  ctl->ingest_base = ctl->pending_start = ctl->pending_end = 0;
  ctl->ht_mask[0] = ctl->ht_mask[1] = 0;
  ctl->active = -1;
  ctl->pending = -1;
}

__global__ void live_range_kernel(const Ctl* ctl, int64_t* out) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    out[0] = ctl->tail;
    out[1] = ctl->head;
  }
}

__global__ void ring_copy_kernel(const Ctl* ctl, const int32_t* ring, int64_t cap, int32_t* out,
                                 int64_t out_cap) {
  const int64_t tail = ctl->tail, n = ctl->head - tail;
  const int64_t x0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  SlotWalk w(tail + x0, stride, cap);
  for (int64_t x = x0; x < n && x < out_cap; x += stride, w.next()) out[x] = ring[w.slot];
}

}  // namespace

hipError_t launch_ingest(const IngestArgs& a, int max_doc_len_hint, hipStream_t st) {
  if (a.R <= 0) return hipSuccess;
  hipLaunchKernelGGL(ingest_plan_kernel, dim3(1), dim3(PT), 0, st, a);
  int gy = (int)((max_doc_len_hint + 1 + 1023) / 1024);
  gy = gy < 1 ? 1 : (gy > 64 ? 64 : gy);
  hipLaunchKernelGGL(ingest_scatter_kernel, dim3(a.R, gy), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_inflight_prepare(const InflightArgs& a, hipStream_t st) {
  if (a.R <= 0) return hipSuccess;
  const int blocks = (a.R + 255) / 256;
  hipLaunchKernelGGL(inflight_claim_kernel, dim3(blocks), dim3(256), 0, st, a);
  hipLaunchKernelGGL(inflight_prepare_kernel, dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_claims_init(int32_t* claim, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(claims_init_kernel, dim3((n + 255) / 256), dim3(256), 0, st, claim, n);
  return hipGetLastError();
}

hipError_t launch_snapshot(Ctl* ctl, const int32_t* ring, int64_t cap, int32_t* text, int buf,
                           int64_t* range_out, hipStream_t st) {
  int64_t blocks = (cap + 1023) / 1024;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(snapshot_kernel, dim3((unsigned)blocks), dim3(256), 0, st, ctl, ring, cap,
                     text, buf, range_out);
  return hipGetLastError();
}

hipError_t launch_swap(Ctl* ctl, int buf, uint32_t mask, hipStream_t st) {
  hipLaunchKernelGGL(swap_kernel, dim3(1), dim3(64), 0, st, ctl, buf, mask);
  return hipGetLastError();
}

hipError_t launch_ctl_init(Ctl* ctl, hipStream_t st) {
  hipLaunchKernelGGL(ctl_init_kernel, dim3(1), dim3(64), 0, st, ctl);
  return hipGetLastError();
}

hipError_t launch_live_range(const Ctl* ctl, int64_t* out, hipStream_t st) {
  hipLaunchKernelGGL(live_range_kernel, dim3(1), dim3(64), 0, st, ctl, out);
  return hipGetLastError();
}

hipError_t launch_ring_copy(const Ctl* ctl, const int32_t* ring, int64_t cap, int32_t* out,
                            int64_t out_cap, hipStream_t st) {
  int64_t blocks = (cap + 1023) / 1024;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(ring_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, ctl, ring, cap,
                     out, out_cap);
  return hipGetLastError();
}

}  // namespace sfx
