// checks.hip -- optional input checks (SFX_FLAG_CHECK_INPUTS): every value the device clamps or
// ignores instead of the host rejecting it (the host cannot see device arrays without a
// synchronisation) sets a bit of a sticky error word that sfx_debug_errors reads and clears.
// One workgroup per row or document; one atomic per workgroup.
#include "checks.h"

#include "../../include/sfx.h"

namespace sfx {

namespace {

constexpr int CT = 256;

__device__ __forceinline__ void raise_bits(uint32_t* err, uint32_t bits) {
  __shared__ uint32_t acc;
  if (threadIdx.x == 0) acc = 0;
  __syncthreads();
  if (bits) atomicOr(&acc, bits);
  __syncthreads();
  if (threadIdx.x == 0 && acc) atomicOr(err, acc);
}

__global__ __launch_bounds__(CT) void check_propose_kernel(int S, int T, const int32_t* ntns,
                                                           const int32_t* tok,
                                                           const int32_t* samp,
                                                           const int32_t* counts, uint32_t* err) {
  const int b = blockIdx.x;
  const int n_raw = ntns[b];
  const int n = n_raw < 0 ? 0 : (n_raw > S ? S : n_raw);
  uint32_t bits = 0;
  if (threadIdx.x == 0) {
    if (n_raw != n) bits |= SFX_ERR_LENGTH;
    int c = T;
    if (counts) {
      const int c_raw = counts[b];
      c = c_raw < 0 ? 0 : (c_raw > T ? T : c_raw);
      if (c != c_raw) bits |= SFX_ERR_LENGTH;
    }
    bool pad = false;
    for (int x = 0; x < c; ++x) {
      const int v = samp[(int64_t)b * T + x];
      if (v < 0) pad = true;
      else if (pad) bits |= SFX_ERR_SAMPLED_AFTER_PAD;
    }
  }
  const int32_t* row = tok + (int64_t)b * S;
  for (int x = threadIdx.x; x < n; x += CT)
    if (row[x] < 0) bits |= SFX_ERR_NEGATIVE_TOKEN;
  raise_bits(err, bits);
}

__global__ __launch_bounds__(CT) void check_ingest_kernel(const int32_t* rows,
                                                          const int32_t* lengths, int num_rows,
                                                          int S, const int64_t* offs,
                                                          const int32_t* tokens, uint32_t* err) {
  const int r = blockIdx.x;
  uint32_t bits = 0;
  const int32_t* doc = nullptr;
  int64_t len = 0;
  if (offs) {
    len = offs[r + 1] - offs[r];
    if (len < 0) {
      if (threadIdx.x == 0) bits |= SFX_ERR_LENGTH;
      len = 0;
    }
    doc = tokens + offs[r];
  } else {
    const int row = rows[r];
    const int l = lengths[r];
    if (row < 0 || row >= num_rows) {
      if (threadIdx.x == 0) bits |= SFX_ERR_ROW_INDEX;
    } else {
      if (threadIdx.x == 0 && (l < 0 || l > S)) bits |= SFX_ERR_LENGTH;
      len = l < 0 ? 0 : (l > S ? S : l);
      doc = tokens + (int64_t)row * S;
    }
  }
  for (int64_t x = threadIdx.x; x < len; x += CT)
    if (doc[x] < 0) bits |= SFX_ERR_NEGATIVE_TOKEN;
  raise_bits(err, bits);
}

__global__ void clear_word_kernel(uint32_t* err) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *err = 0;
}

}  // namespace

hipError_t launch_check_propose(int B, int S, int T, const int32_t* ntns, const int32_t* tok,
                                const int32_t* samp, const int32_t* counts, uint32_t* err,
                                hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_propose_kernel, dim3(B), dim3(CT), 0, st, S, T, ntns, tok, samp, counts,
                     err);
  return hipGetLastError();
}

hipError_t launch_check_ingest(int R, const int32_t* rows, const int32_t* lengths, int num_rows,
                               int S, const int64_t* doc_offsets, const int32_t* tokens,
                               uint32_t* err, hipStream_t st) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_ingest_kernel, dim3(R), dim3(CT), 0, st, rows, lengths, num_rows, S,
                     doc_offsets, tokens, err);
  return hipGetLastError();
}

hipError_t launch_clear_word(uint32_t* err, hipStream_t st) {
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(64), 0, st, err);
  return hipGetLastError();
}

}  // namespace sfx
