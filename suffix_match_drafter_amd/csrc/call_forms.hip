// call_forms.hip -- the other call forms of the drafter step, each turned into the ordinary
// form by a preparation kernel so that the propose kernel runs on them unchanged.
//
// Masked form.  PyPI page "suffix-gpu 0.1.1", Quickstart: propose(num_tokens_no_spec, token_ids,
// combined_mask) serves callers that keep token_ids up to date themselves.  Row b's context is
// then token_ids[b, 0:n_b] alone, and rows whose mask entry is 0 get no draft.  That is the
// ordinary step with the row's last token as its sampled id: this kernel writes, per row, the
// prefix length n_b - 1 and that token (-1, no sampled id, for a masked-off or empty row), and
// the propose kernel runs on them unchanged.
#include "call_forms.h"

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

// Counted form.  vLLM issue "[RFC]: Suffix decoding on GPU (suffix_gpu)", Design: the ngram_gpu
// contract propose(k, num_tokens_no_spec, token_ids, sampled, counts), where counts[b] is the
// number of valid entries of sampled[b] instead of a -1 padding.
__global__ void counts_prep_kernel(int B, int T, const int32_t* sampled, const int32_t* counts,
                                   int32_t* s_out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)B * T) return;
  const int b = (int)(i / T), x = (int)(i % T);
  int c = counts[b];
  c = c < 0 ? 0 : (c > T ? T : c);
  s_out[i] = x < c ? sampled[i] : -1;
}

}  // namespace

hipError_t launch_counts_prep(int B, int T, const int32_t* sampled, const int32_t* counts,
                              int32_t* s_out, hipStream_t st) {
  const int64_t n = (int64_t)B * T;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(counts_prep_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, B,
                     T, sampled, counts, s_out);
  return hipGetLastError();
}

hipError_t launch_masked_prep(int B, int S, const int32_t* ntns, const int32_t* tok,
                              const int32_t* mask, int32_t* n_out, int32_t* s_out,
                              hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(masked_prep_kernel, dim3((B + 255) / 256), dim3(256), 0, st, B, S, ntns, tok,
                     mask, n_out, s_out);
  return hipGetLastError();
}

}  // namespace sfx
