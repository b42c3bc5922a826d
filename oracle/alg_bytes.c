/*
 * alg_bytes.c -- instrumented count of the 4-byte words one drafter call must touch (the
 * algorithmic bytes of the measurement), by category.
 *
 * TEST INFRASTRUCTURE ONLY (part of the oracle library): written to a stored file by a
 * committed script, which the benchmark reads; never called by the GPU product path.
 *
 * The categories and their definitions follow the method's steps as the pages give them
 * (SuffixGPU page, How it works steps 1-3 and Highlights; vLLM docs "Suffix Decoding", Model
 * Runner V2), with the corpus searched by binary search over its suffix array (SuffixGPU page,
 * How it works step 2: a fixed-iteration binary search, all pattern lengths as one batch):
 *   [0] context: every context word once (row prefix and sampled ids): L per request;
 *   [1] per-request inputs and outputs: the length, the T sampled ids read to find t, the
 *       draft (k) and its valid count: 2 + T + k + 1 per request (the length counted as read
 *       and the count as written);
 *   [2] suffix-array probes: for every pattern length l in [2, min(D, L)], a lower-bound and an
 *       upper-bound binary search of the tail's last l tokens; each step reads one
 *       suffix-array word and the text tokens its comparison reads (up to and including the
 *       first mismatch, at most l, never past the text's end);
 *   [3] interval scans: for every distinct valid corpus candidate of length g, the words of
 *       its suffix-array interval [lo(g), hi(g)) (read to find its earliest continuing sites);
 *   [4] voted continuation tokens: for every distinct valid candidate (local or corpus), at
 *       every depth it votes, one word per alive site whose position lies inside its source.
 * Candidates that repeat an earlier candidate's length (same sites, same vote) are counted
 * once.  Without a corpus categories 2 and 3 are 0.  Everything is counted in words; the
 * caller multiplies by 4.
 */
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* Word reads of one comparison of the suffix at s with the pattern P[0..l): compares token by
 * token until a mismatch (counted), the pattern's end or the text's end.  *cmp_out: <0 when
 * the suffix sorts before P (a mismatch with a smaller token, or the text ends first), >0 when
 * after, 0 when the suffix starts with P. */
static int64_t cmp_reads(const int32_t* C, int64_t N, int64_t s, const int32_t* P, int32_t l,
                         int* cmp_out) {
  int64_t reads = 0;
  for (int32_t j = 0; j < l; j++) {
    if (s + j >= N) {
      *cmp_out = -1;
      return reads;
    }
    reads++;
    if (C[s + j] != P[j]) {
      *cmp_out = C[s + j] < P[j] ? -1 : 1;
      return reads;
    }
  }
  *cmp_out = 0;
  return reads;
}

/* Bound searches of P[0..l) in the suffix array: lo = first index whose suffix does not sort
 * before P, hi = first index whose suffix sorts after every suffix starting with P.  Classic
 * halving over [0, N); returns the words read (one per step plus the comparison's). */
static int64_t bounds(const int32_t* C, const int32_t* sa, int64_t N, const int32_t* P, int32_t l,
                      int64_t* lo_out, int64_t* hi_out) {
  int64_t words = 0;
  int64_t lo = 0, hi = N;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    int c;
    words += 1 + cmp_reads(C, N, sa[mid], P, l, &c);
    if (c < 0) lo = mid + 1;
    else hi = mid;
  }
  const int64_t first = lo;
  lo = first;
  hi = N;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    int c;
    words += 1 + cmp_reads(C, N, sa[mid], P, l, &c);
    if (c <= 0) lo = mid + 1;
    else hi = mid;
  }
  *lo_out = first;
  *hi_out = lo;
  return words;
}

/* The vote of orc_expand, counting its reads: at depth n, one word per alive site with p+n
 * inside the source. */
static int64_t vote_reads(const int32_t* X, int64_t lenX, const int32_t* sites, int32_t c0,
                          int32_t cap, int32_t scored, int64_t min_prob_ppm) {
  int32_t* alive = (int32_t*)malloc((size_t)(c0 > 0 ? c0 : 1) * sizeof(int32_t));
  int32_t* tok = (int32_t*)malloc((size_t)(c0 > 0 ? c0 : 1) * sizeof(int32_t));
  for (int32_t i = 0; i < c0; i++) alive[i] = 1;
  int64_t reads = 0;
  for (int32_t n = 0; n < cap; n++) {
    int32_t any = 0;
    for (int32_t i = 0; i < c0; i++) {
      const int64_t q = (int64_t)sites[i] + n;
      const int inside = alive[i] && q < lenX;
      reads += inside;
      tok[i] = (inside && X[q] >= 0) ? X[q] : -1;
      if (tok[i] >= 0) any = 1;
    }
    if (!any) break;
    int32_t best = -1, bestc = 0;
    for (int32_t i = 0; i < c0; i++) {
      if (tok[i] < 0) continue;
      int32_t c = 0;
      for (int32_t j = 0; j < c0; j++) c += tok[j] == tok[i];
      if (c > bestc || (c == bestc && tok[i] < best)) { best = tok[i]; bestc = c; }
    }
    if (scored && (int64_t)bestc * 1000000 < min_prob_ppm * (int64_t)c0) break;
    for (int32_t i = 0; i < c0; i++) alive[i] = alive[i] && tok[i] == best;
  }
  free(alive);
  free(tok);
  return reads;
}

/* Category 4 for the nb candidates of one source (local or corpus), distinct lengths once;
 * lens_out receives the candidate lengths (0 when invalid). */
static int64_t source_votes(const orc_params* p, const int32_t* vals, int64_t nvals,
                            int32_t min_len, const int32_t* X, int64_t lenX, int32_t* sites,
                            int32_t* lens_out) {
  int64_t reads = 0;
  int32_t prev = -1;
  for (int32_t t = 1; t <= p->num_backoff; t++) {
    const int32_t l = orc_kth_largest(vals, nvals, t);
    const int valid = l >= min_len && l >= 1;
    lens_out[t - 1] = valid ? l : 0;
    if (!valid || l == prev) {
      prev = l;
      continue;
    }
    prev = l;
    const int32_t c0 = orc_first_sites(vals, nvals, l, p->max_occurrences, sites);
    reads += vote_reads(X, lenX, sites, c0, orc_spec_cap(p, l), p->mode == ORC_MODE_SCORED,
                        p->min_token_prob_ppm);
  }
  return reads;
}

int orc_alg_words(const orc_params* p, int32_t B, int32_t S, int32_t T,
                  const int32_t* num_tokens_no_spec, const int32_t* token_ids,
                  const int32_t* sampled, const int32_t* C, int64_t N, const int32_t* sa,
                  int64_t* words_out /* [5] */, int32_t num_threads) {
  if (!p || B < 0 || S < 0 || T < 0 || (N > 0 && (!C || !sa))) return -1;
  for (int i = 0; i < 5; i++) words_out[i] = 0;
  int64_t w0 = 0, w1 = 0, w2 = 0, w3 = 0, w4 = 0;
  if (num_threads < 1) num_threads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads) \
    reduction(+ : w0, w1, w2, w3, w4)
  for (int32_t b = 0; b < B; b++) {
    const int32_t D = p->max_tree_depth;
    int32_t* ctx = (int32_t*)malloc((size_t)(S + T + 1) * sizeof(int32_t));
    int32_t t = 0;
    const int32_t L = orc_context(S, T, num_tokens_no_spec[b], token_ids + (int64_t)b * S,
                                  sampled + (int64_t)b * T, ctx, &t);
    w1 += 2 + T + p->k + 1;
    if (t == 0) {  // no draft: only the inputs that decide it (and the outputs) are touched
      free(ctx);
      continue;
    }
    w0 += L;
    int32_t* sites = (int32_t*)malloc((size_t)p->max_occurrences * sizeof(int32_t));
    int32_t lens[ORC_MAX_NB];
    int32_t* mb = (int32_t*)malloc((size_t)(L > 1 ? L - 1 : 1) * sizeof(int32_t));
    orc_match_back(ctx, L, D, mb);
    w4 += source_votes(p, mb, L - 1, p->min_self_match, ctx, L, sites, lens);
    free(mb);
    if (C && N > 0) {
      const int32_t lmax = D < L ? D : L;
      int64_t lo[65], hi[65];
      for (int32_t l = 2; l <= lmax; l++) w2 += bounds(C, sa, N, ctx + L - l, l, &lo[l], &hi[l]);
      int32_t* m = (int32_t*)malloc((size_t)N * sizeof(int32_t));
      orc_corpus_match(C, N, ctx, L, D, m);
      w4 += source_votes(p, m, N, p->min_corpus_match, C, N, sites, lens);
      free(m);
      int32_t prev = -1;
      for (int32_t i = 0; i < p->num_backoff; i++) {
        const int32_t g = lens[i];
        if (g >= 2 && g <= lmax && g != prev) w3 += hi[g] - lo[g];
        prev = g;
      }
    }
    free(sites);
    free(ctx);
  }
  words_out[0] = w0;
  words_out[1] = w1;
  words_out[2] = w2;
  words_out[3] = w3;
  words_out[4] = w4;
  return 0;
}
