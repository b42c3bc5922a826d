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

__device__ __forceinline__ int64_t doc_len(const IngestArgs& a, int r) {
  if (a.doc_offsets) {
    const int64_t l = a.doc_offsets[r + 1] - a.doc_offsets[r];
    return l < 0 ? 0 : l;
  }
  const int row = a.row_indices[r];
  if (row < 0 || row >= a.num_rows) return 0;
  int l = a.lengths[r];
  return l < 0 ? 0 : (l > a.S ? a.S : l);
}

__device__ __forceinline__ const int32_t* doc_src(const IngestArgs& a, int r) {
  if (a.doc_offsets) return a.tokens + a.doc_offsets[r];
  const int row = a.row_indices[r];
  return a.tokens + (int64_t)(row < 0 ? 0 : row) * a.S;
}

// Offsets of the new documents (each takes len + 1 ring tokens), new head, and the eviction
// that keeps the longest run of most recent documents fitting in the capacity.
__global__ __launch_bounds__(PT) void ingest_plan_kernel(IngestArgs a) {
  __shared__ int64_t wsum[PT / 64];
  __shared__ int64_t carry;
  __shared__ int64_t s_base, s_doc_tail;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int c = 0; c < a.R; c += PT) {
    const int r = c + tid;
    const int64_t v = r < a.R ? doc_len(a, r) + 1 : 0;
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
    if (r < a.R) a.doc_off[r] = pre + x - v;
    __syncthreads();
    if (tid == PT - 1) carry = pre + x;
    __syncthreads();
  }
  Ctl* ctl = a.ctl;
  if (tid == 0) {
    const int64_t total = carry;
    a.doc_off[a.R] = total;
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
        new_doc_tail = dh + rl;
      }
    }
    s_base = base;
    s_doc_tail = new_doc_tail;
    ctl->ingest_base = base;
    ctl->head = new_head;
    ctl->tail = new_tail;
    ctl->doc_head = dh + a.R;
    ctl->doc_tail = new_doc_tail;
    carry = dh;
  }
  __syncthreads();
  const int64_t dh = carry, base = s_base, ndt = s_doc_tail;
  for (int r = tid; r < a.R; r += PT)
    if (dh + r >= ndt) a.doc_start[(dh + r) % a.dcap] = base + a.doc_off[r];
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
