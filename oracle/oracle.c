/*
 * oracle.c -- plain, slow, obviously correct CPU oracle of the suffix-match drafter.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the package smoke check and the benchmark's
 * CPU-baseline leg.  The GPU product path never includes, links or calls it, and the two share
 * no code.  Everything here is integer arithmetic; probabilities are compared as exact ratios
 * of counts by cross-multiplication.
 *
 * The drafter is a heuristic, so this file runs its steps in the order the pages give them
 * (SuffixGPU page, "How it works": local matching, global matching, expansion & selection), in
 * the simplest loops that express each definition.  Where the pages leave a detail open the
 * reading taken is stated at the function.
 */
#define _GNU_SOURCE
#include "oracle.h"

#include <stdlib.h>
#include <string.h>

/* Context of one request.
 * SuffixGPU page, Quickstart: the resident state is token_ids[B,S], num_tokens_no_spec[B] and the
 * last verifier output sampled_token_ids[B,T], -1 padded.  The RFC page (Summary, Design) has
 * the draft built from the sampled ids of the step before, as they sit on the device.
 * Reading: the context is the row
 * prefix of length n (clamped to [0,S]) followed by the leading non-negative sampled ids. */
int32_t orc_context(int32_t S, int32_t T, int32_t n_raw, const int32_t* row, const int32_t* samp,
                    int32_t* ctx, int32_t* t_out) {
  int32_t n = n_raw < 0 ? 0 : (n_raw > S ? S : n_raw);
  int32_t t = 0;
  while (t < T && samp[t] >= 0) t++;
  for (int32_t i = 0; i < n; i++) ctx[i] = row[i];
  for (int32_t i = 0; i < t; i++) ctx[n + i] = samp[i];
  *t_out = t;
  return n + t;
}

/* Local match lengths.  vLLM docs "Suffix Decoding", Model Runner V2: each request is matched
 * against its own prompt and output by the longest matching suffix, up to max_tree_depth
 * tokens.  SuffixGPU page, How it works step 1: one match_back pass over the context.
 * mb[j] (j = 0..L-2) = number of tokens, at most min(D, j+1), for which the text ending at j
 * equals the text ending at L-1.  j = L-1 (the tail itself) is excluded: every counted
 * occurrence has at least one continuation token. */
void orc_match_back(const int32_t* ctx, int32_t L, int32_t D, int32_t* mb) {
  for (int32_t j = 0; j + 1 < L; j++) {
    int32_t lim = D < j + 1 ? D : j + 1;
    int32_t m = 0;
    while (m < lim && ctx[j - m] == ctx[L - 1 - m]) m++;
    mb[j] = m;
  }
}

/* Corpus match lengths.  vLLM docs "Suffix Decoding", Model Runner V2: the corpus positions
 * that share the request's final two and final four tokens are found first and then grown
 * backwards as far as the match goes; SuffixGPU page, How it works step 2: the same tail is
 * searched in the shared corpus.
 * Reading: the corpus is the live documents in ingest order, each followed by one -1; a match
 * never covers a -1 and must be followed by a real token (C[e+1] >= 0), so it has a
 * continuation.  m[e] (e = 0..N-1) = that backward match length at end e, capped at
 * min(D, L), or 0 when e is not followed by a real token. */
void orc_corpus_match(const int32_t* C, int64_t N, const int32_t* ctx, int32_t L, int32_t D,
                      int32_t* m) {
  int32_t cap = D < L ? D : L;
  for (int64_t e = 0; e < N; e++) {
    m[e] = 0;
    if (e + 1 >= N || C[e + 1] < 0) continue;
    int32_t len = 0;
    while (len < cap && (int64_t)len <= e && C[e - len] >= 0 && C[e - len] == ctx[L - 1 - len])
      len++;
    m[e] = len;
  }
}

/* Backoff ladder.  SuffixGPU page, How it works step 1: for support threshold t the candidate
 * length is the largest length occurring at least t times, i.e. the t-th largest match_back
 * value (counted with multiplicity).  Values are non-negative match lengths; a histogram is
 * walked from the top until t values have been passed.  Returns 0 when fewer than t values
 * exist. */
int32_t orc_kth_largest(const int32_t* vals, int64_t n, int32_t t) {
  if (t < 1 || n < t) return 0;
  int32_t maxv = 0;
  for (int64_t i = 0; i < n; i++)
    if (vals[i] > maxv) maxv = vals[i];
  int64_t* hist = (int64_t*)calloc((size_t)maxv + 1, sizeof(int64_t));
  for (int64_t i = 0; i < n; i++)
    if (vals[i] >= 0) hist[vals[i]]++;
  int64_t seen = 0;
  int32_t r = 0;
  for (int32_t v = maxv; v >= 0; v--) {
    seen += hist[v];
    if (seen >= t) { r = v; break; }
  }
  free(hist);
  return r;
}

/* Support of a length: how many occurrences match at least l tokens. */
int64_t orc_count_at_least(const int32_t* vals, int64_t n, int32_t l) {
  int64_t c = 0;
  for (int64_t i = 0; i < n; i++) c += vals[i] >= l;
  return c;
}

/* Continuation sites.  SuffixGPU page, How it works step 1: each candidate keeps up to
 * max_occurrences earliest continuation sites.  A value at index i that reaches l marks the
 * site i+1 (the token right after the match); the first M sites in ascending order are kept. */
int32_t orc_first_sites(const int32_t* vals, int64_t n, int32_t l, int32_t M, int32_t* sites) {
  int32_t c = 0;
  for (int64_t i = 0; i < n && c < M; i++)
    if (vals[i] >= l) sites[c++] = (int32_t)(i + 1);
  return c;
}

/* Adaptive speculation cap.  SuffixGPU page, Quickstart: cap = factor * match_len + offset;
 * gitcode blog section 4: max_spec_tokens = max_spec_factor * prefix_match_length.  The factor
 * and offset are exact rationals in millionths, so the cap is a floor of an integer ratio,
 * never more than k.  The Model Runner V2 selection does not use it (the draft may be k long).
 * With tree_depth_cap (either mode), the gitcode blog's parameter table in section 4 is read
 * literally: max_tree_depth bounds the match length plus the draft length, so the cap is also
 * at most D - l (and not below 0). */
int32_t orc_spec_cap(const orc_params* p, int32_t l) {
  int32_t cap = p->k;
  if (p->mode == ORC_MODE_SCORED) {
    int64_t c = (p->spec_factor_ppm * (int64_t)l + p->spec_offset_ppm) / 1000000;
    if (c < 0) c = 0;
    if (c < cap) cap = (int32_t)c;
  }
  if (p->tree_depth_cap) {
    const int32_t room = p->max_tree_depth - l;
    if (room < cap) cap = room < 0 ? 0 : room;
  }
  return cap;
}

/* Depth-wise vote.  SuffixGPU page, How it works step 3 and Highlights: continuations are
 * extended depth by depth by majority vote, tracking the empirical chain probability for the
 * stop rule and summing it into the score (expected accepted tokens); gitcode blog section 4:
 * a token whose count-based probability is below min_token_prob is not proposed.
 * Readings: at depth d the vote is over the still-alive sites whose token X[p+d] exists and is
 * not -1; the winner has the highest count and, among equal counts, the smallest token id; the
 * chain probability at depth d is counts[d] / c0 where c0 is the number of sites; it is kept
 * iff counts[d] * 1e6 >= min_prob_ppm * c0; the score is snum / c0 with snum = sum of counts.
 * Returns the number of tokens written to out. */
int32_t orc_expand(const int32_t* X, int64_t lenX, const int32_t* sites, int32_t c0, int32_t cap,
                   int32_t scored, int64_t min_prob_ppm, int32_t* out, int32_t* counts,
                   int64_t* snum_out) {
  int32_t* alive = (int32_t*)malloc((size_t)(c0 > 0 ? c0 : 1) * sizeof(int32_t));
  int32_t* tok = (int32_t*)malloc((size_t)(c0 > 0 ? c0 : 1) * sizeof(int32_t));
  for (int32_t i = 0; i < c0; i++) alive[i] = 1;
  int32_t n = 0;
  int64_t snum = 0;
  while (n < cap) {
    int32_t any = 0;
    for (int32_t i = 0; i < c0; i++) {
      int64_t q = (int64_t)sites[i] + n;
      tok[i] = (alive[i] && q < lenX && X[q] >= 0) ? X[q] : -1;
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
    out[n] = best;
    if (counts) counts[n] = bestc;
    n++;
    snum += bestc;
    for (int32_t i = 0; i < c0; i++) alive[i] = alive[i] && tok[i] == best;
  }
  free(alive);
  free(tok);
  *snum_out = snum;
  return n;
}

typedef struct {
  int32_t valid, len, c0, n;
  int64_t snum;
  int32_t out[64];
} cand_t;

static void run_candidate(const orc_params* p, const int32_t* vals, int64_t nvals, int32_t t,
                          int32_t min_len, const int32_t* X, int64_t lenX, int32_t* sites,
                          cand_t* c, int32_t* len_out, int32_t* sup_out) {
  int32_t l = orc_kth_largest(vals, nvals, t);
  *len_out = l;
  *sup_out = l >= 1 ? (int32_t)orc_count_at_least(vals, nvals, l) : 0;
  c->valid = l >= min_len && l >= 1;
  c->len = l;
  c->n = 0;
  c->snum = 0;
  c->c0 = 0;
  if (!c->valid) return;
  c->c0 = orc_first_sites(vals, nvals, l, p->max_occurrences, sites);
  c->n = orc_expand(X, lenX, sites, c->c0, orc_spec_cap(p, l), p->mode == ORC_MODE_SCORED,
                    p->min_token_prob_ppm, c->out, NULL, &c->snum);
}

/* One row.  Selection and output follow:
 *  - vLLM docs "Suffix Decoding", Model Runner V2 (mode LONGEST_FILL): the longer match wins;
 *    the draft always has k tokens, slots without a match get the last sampled token; factor
 *    and min-prob are not used.  Reading: equal lengths go to the request's own context.
 *  - SuffixGPU page, How it works step 3 (mode SCORED): the best-scored candidate wins per path
 *    and the local and global winners compete by the same score; the draft is -1 padded.
 *    Reading: candidates in the order local t=1..nb, global t=1..nb; the first of equal
 *    scores wins, so a strictly better score is needed to displace an earlier candidate.
 *  - gitcode blog section 5, step 1: a request with no sampled token this step (partial
 *    prefill) gets no draft: all -1, num_valid 0, in both modes. */
static void propose_row(const orc_params* p, int32_t S, int32_t T, int32_t n_raw,
                        const int32_t* row, const int32_t* samp, const int32_t* C, int64_t N,
                        int32_t* draft, int32_t* num_valid, orc_row_info* info) {
  const int32_t k = p->k, nb = p->num_backoff, D = p->max_tree_depth;
  int32_t* ctx = (int32_t*)malloc((size_t)(S + T + 1) * sizeof(int32_t));
  int32_t t = 0;
  int32_t L = orc_context(S, T, n_raw, row, samp, ctx, &t);
  orc_row_info inf;
  memset(&inf, 0, sizeof(inf));
  inf.L = L;
  inf.t = t;
  inf.chosen = -1;
  for (int32_t i = 0; i < k; i++) draft[i] = -1;
  *num_valid = 0;
  if (t == 0) {
    if (info) *info = inf;
    free(ctx);
    return;
  }
  int32_t fill = p->mode == ORC_MODE_LONGEST_FILL ? ctx[L - 1] : -1;

  cand_t cand[2 * ORC_MAX_NB];
  int32_t* sites = (int32_t*)malloc((size_t)p->max_occurrences * sizeof(int32_t));
  int32_t* mb = (int32_t*)malloc((size_t)(L > 1 ? L - 1 : 1) * sizeof(int32_t));
  orc_match_back(ctx, L, D, mb);
  for (int32_t i = 0; i < nb; i++)
    run_candidate(p, mb, L - 1, i + 1, p->min_self_match, ctx, L, sites, &cand[i],
                  &inf.local_len[i], &inf.local_support[i]);
  free(mb);
  for (int32_t i = 0; i < nb; i++) cand[nb + i].valid = 0;
  if (C && N > 0) {
    int32_t* m = (int32_t*)malloc((size_t)N * sizeof(int32_t));
    orc_corpus_match(C, N, ctx, L, D, m);
    for (int32_t i = 0; i < nb; i++)
      run_candidate(p, m, N, i + 1, p->min_corpus_match, C, N, sites, &cand[nb + i],
                    &inf.global_len[i], &inf.global_support[i]);
    free(m);
  }
  free(sites);

  int32_t win = -1;
  if (p->mode == ORC_MODE_LONGEST_FILL) {
    int32_t lv = cand[0].valid, gv = cand[nb].valid;
    if (lv && (!gv || cand[0].len >= cand[nb].len)) win = 0;
    else if (gv) win = nb;
  } else {
    for (int32_t i = 0; i < 2 * nb; i++) {
      if (!cand[i].valid) continue;
      if (win < 0 || cand[i].snum * (int64_t)cand[win].c0 > cand[win].snum * (int64_t)cand[i].c0)
        win = i;
    }
  }
  int32_t n = 0;
  if (win >= 0) {
    n = cand[win].n;
    for (int32_t i = 0; i < n; i++) draft[i] = cand[win].out[i];
    inf.chosen_len = cand[win].len;
    inf.c0 = cand[win].c0;
    inf.n = n;
    inf.snum = cand[win].snum;
  }
  inf.chosen = win;
  for (int32_t i = n; i < k; i++) draft[i] = fill;
  *num_valid = n;
  if (info) *info = inf;
  free(ctx);
}

/* The drafter call.  RFC page, Design: propose(k, num_tokens_no_spec, token_ids, sampled,
 * counts) -> (drafts [B,k], valid counts [B]).  Rows are independent; num_threads > 1 only
 * spreads whole rows over OpenMP threads (the per-row arithmetic is unchanged). */
int orc_propose(const orc_params* p, int32_t B, int32_t S, int32_t T,
                const int32_t* num_tokens_no_spec, const int32_t* token_ids, const int32_t* sampled,
                const int32_t* corpus, int64_t N, int32_t* draft, int32_t* num_valid,
                orc_row_info* info, int32_t num_threads) {
  if (!p || p->k < 1 || p->k > 64 || p->num_backoff < 1 || p->num_backoff > ORC_MAX_NB ||
      p->max_occurrences < 1 || p->max_tree_depth < 1 || p->min_self_match < 1 ||
      p->min_corpus_match < 2 || B < 0 || S < 0 || T < 0)
    return -1;
  if (num_threads < 1) num_threads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads)
  for (int32_t b = 0; b < B; b++)
    propose_row(p, S, T, num_tokens_no_spec[b], token_ids + (int64_t)b * S,
                sampled + (int64_t)b * T, corpus, N, draft + (int64_t)b * p->k, num_valid + b,
                info ? info + b : NULL);
  return 0;
}

/* State update.  SuffixGPU page, Quickstart: propose_with_update appends the verifier output to
 * the resident rows and returns the new lengths (RFC page, Design: the same device bookkeeping
 * as ngram_gpu).  Reading: the leading non-negative sampled ids are written after the row
 * prefix, as many as fit in S; the new length is the old (clamped) length plus that number. */
void orc_update_state(int32_t B, int32_t S, int32_t T, int32_t* token_ids,
                      const int32_t* num_tokens_no_spec, const int32_t* sampled,
                      int32_t* num_tokens_out) {
  for (int32_t b = 0; b < B; b++) {
    int32_t n = num_tokens_no_spec[b];
    n = n < 0 ? 0 : (n > S ? S : n);
    int32_t i = 0;
    while (i < T && sampled[(int64_t)b * T + i] >= 0 && n + i < S) {
      token_ids[(int64_t)b * S + n + i] = sampled[(int64_t)b * T + i];
      i++;
    }
    num_tokens_out[b] = n + i;
  }
}

/* Suffix array.  SuffixGPU page, Highlights: the cross-request memory is backed by a suffix
 * array (References: Manber & Myers).  Definition used: the start positions 0..n-1 ordered by
 * the suffixes they start, tokens compared as signed int32, a proper prefix before any longer
 * suffix it prefixes.  All suffixes differ in length, so the order is unique.  Built here by a
 * plain comparison sort. */
static int cmp_suffix(const void* a, const void* b, void* arg) {
  const int64_t* ctx = (const int64_t*)arg;
  const int32_t* text = (const int32_t*)(intptr_t)ctx[0];
  int64_t n = ctx[1];
  int64_t i = *(const int32_t*)a, j = *(const int32_t*)b;
  while (i < n && j < n) {
    if (text[i] != text[j]) return text[i] < text[j] ? -1 : 1;
    i++;
    j++;
  }
  if (i == n && j == n) return 0;
  return i == n ? -1 : 1;
}

int orc_suffix_array(const int32_t* text, int64_t n, int32_t* sa) {
  if (n < 0 || n > 0x7fffffff) return -1;
  for (int64_t i = 0; i < n; i++) sa[i] = (int32_t)i;
  int64_t ctx[2] = {(int64_t)(intptr_t)text, n};
  qsort_r(sa, (size_t)n, sizeof(int32_t), cmp_suffix, ctx);
  return 0;
}
