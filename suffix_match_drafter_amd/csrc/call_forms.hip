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

// Padding of a batch bucket (RFC page, Design, Proposer: the draft chain is captured per batch
// size bucket).  Rows [from, to) become empty rows, no prefix and no sampled id, so a step
// captured for `to` rows reads nothing of them and proposes nothing for them.  One thread per
// row entry: entry 0 is the length, entries 1 .. T the sampled ids.  The grid covers `to` rows,
// the most any `from` >= 0 leaves, so only the arguments change between calls.
__global__ void pad_rows_kernel(int32_t* ntns, int32_t* samp, int T, int from, int to) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int w = T + 1;
  if (from < 0 || i >= (int64_t)(to - from) * w) return;
  const int64_t r = from + i / w;
  const int c = (int)(i % w);
  if (c == 0)
    ntns[r] = 0;
  else
    samp[r * T + c - 1] = -1;
}

constexpr int kPadThreads = 256;

hipKernelNodeParams pad_params(void** args, int T, int to) {
  hipKernelNodeParams p{};
  const int64_t n = (int64_t)to * (T + 1);
  p.func = reinterpret_cast<void*>(pad_rows_kernel);
  p.gridDim = dim3((unsigned)((n + kPadThreads - 1) / kPadThreads > 0
                                  ? (n + kPadThreads - 1) / kPadThreads : 1));
  p.blockDim = dim3(kPadThreads);
  p.sharedMemBytes = 0;
  p.kernelParams = args;
  p.extra = nullptr;
  return p;
}

}  // namespace

hipError_t launch_pad_rows(int32_t* ntns, int32_t* samp, int T, int from, int to,
                          hipStream_t st) {
  void* args[] = {&ntns, &samp, &T, &from, &to};
  const hipKernelNodeParams p = pad_params(args, T, to);
  return hipLaunchKernel(p.func, p.gridDim, p.blockDim, args, 0, st);
}

hipError_t set_pad_rows(hipGraphExec_t exec, hipGraphNode_t node, int32_t* ntns, int32_t* samp,
                        int T, int from, int to) {
  void* args[] = {&ntns, &samp, &T, &from, &to};
  const hipKernelNodeParams p = pad_params(args, T, to);
  return hipGraphExecKernelNodeSetParams(exec, node, &p);
}

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
