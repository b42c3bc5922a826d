// masked.hip -- the masked form of the drafter step.
//
// PyPI page "suffix-gpu 0.1.1", Quickstart: propose(num_tokens_no_spec, token_ids,
// combined_mask) serves callers that keep token_ids up to date themselves.  Row b's context is
// then token_ids[b, 0:n_b] alone, and rows whose mask entry is 0 get no draft.  That is the
// ordinary step with the row's last token as its sampled id: this kernel writes, per row, the
// prefix length n_b - 1 and that token (-1, no sampled id, for a masked-off or empty row), and
// the propose kernel runs on them unchanged.
#include "masked.h"

namespace sfx {

namespace {

__global__ void masked_prep_kernel(int B, int S, const int32_t* ntns, const int32_t* tok,
                                   const int32_t* mask, int32_t* n_out, int32_t* s_out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int n = ntns[b];
  n = n < 0 ? 0 : (n > S ? S : n);
  if (mask[b] != 0 && n > 0) {
    n_out[b] = n - 1;
    s_out[b] = tok[(int64_t)b * S + n - 1];
  } else {
    n_out[b] = n;
    s_out[b] = -1;
  }
}

}  // namespace

hipError_t launch_masked_prep(int B, int S, const int32_t* ntns, const int32_t* tok,
                              const int32_t* mask, int32_t* n_out, int32_t* s_out,
                              hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(masked_prep_kernel, dim3((B + 255) / 256), dim3(256), 0, st, B, S, ntns, tok,
                     mask, n_out, s_out);
  return hipGetLastError();
}

}  // namespace sfx
