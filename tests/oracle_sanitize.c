/* Drives every entry point of the CPU oracle on many small random inputs (random shapes,
 * knobs, -1 padding, out-of-range lengths, corpora with separators, the tree-depth cap), for a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer: any out-of-bounds access, leak or
 * undefined operation in the oracle ends the run with an error.  It also checks the invariants
 * every draft must hold (num_valid within [0, k]; drafts filled as the mode says). */
#include <stdio.h>
#include <stdlib.h>

#include "../oracle/oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) { /* xorshift64* */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 2685821657736338717ull) >> 32);
}
static int uni(int lo, int hi) { return lo + (int)(rnd() % (uint32_t)(hi - lo + 1)); }

#define FAIL(...) do { fprintf(stderr, __VA_ARGS__); exit(1); } while (0)

int main(void) {
  for (int it = 0; it < 3000; ++it) {
    const int V = uni(1, 6), B = uni(1, 4), S = uni(0, 40), T = uni(0, 4);
    orc_params p = {0};
    p.mode = uni(0, 1);
    p.k = uni(1, 32);
    p.max_tree_depth = uni(2, 64);
    p.num_backoff = p.mode == ORC_MODE_LONGEST_FILL ? 1 : uni(1, ORC_MAX_NB);
    p.max_occurrences = uni(1, 128);
    p.min_self_match = uni(1, 3);
    p.min_corpus_match = uni(2, p.max_tree_depth);
    p.tree_depth_cap = uni(0, 1);
    p.spec_factor_ppm = (int64_t)uni(0, 4) * 500000;
    p.spec_offset_ppm = (int64_t)uni(0, 2) * 500000;
    p.min_token_prob_ppm = (int64_t)uni(0, 10) * 100000;
    int32_t* n = malloc(sizeof(int32_t) * B);
    int32_t* tok = malloc(sizeof(int32_t) * (B * S + 1));
    int32_t* samp = malloc(sizeof(int32_t) * (B * T + 1));
    int32_t* draft = malloc(sizeof(int32_t) * B * p.k);
    int32_t* nv = malloc(sizeof(int32_t) * B);
    int32_t* nout = malloc(sizeof(int32_t) * B);
    orc_row_info* info = malloc(sizeof(orc_row_info) * B);
    for (int b = 0; b < B; ++b) n[b] = uni(-2, S + 2);
    for (int i = 0; i < B * S; ++i) tok[i] = uni(0, V - 1);
    for (int b = 0; b < B; ++b) {
      const int lead = uni(0, T);
      for (int x = 0; x < T; ++x) samp[b * T + x] = x < lead ? uni(0, V - 1) : (uni(0, 1) ? -1 : uni(0, V - 1));
    }
    /* corpus: documents joined by -1, or none */
    int64_t N = 0;
    int32_t* corpus = NULL;
    if (uni(0, 2)) {
      const int ndoc = uni(1, 8);
      corpus = malloc(sizeof(int32_t) * ndoc * 41);
      for (int d = 0; d < ndoc; ++d) {
        const int len = uni(0, 40);
        for (int x = 0; x < len; ++x) corpus[N++] = uni(0, V - 1);
        corpus[N++] = -1;
      }
    }
    if (orc_propose(&p, B, S, T, n, tok, samp, corpus, N, draft, nv, info, 1) != 0)
      FAIL("orc_propose failed at iteration %d\n", it);
    for (int b = 0; b < B; ++b) {
      if (nv[b] < 0 || nv[b] > p.k) FAIL("num_valid %d outside [0, %d]\n", nv[b], p.k);
      for (int x = nv[b]; x < p.k; ++x) {
        const int32_t d = draft[b * p.k + x];
        if (p.mode == ORC_MODE_SCORED && d != -1) FAIL("SCORED fill is not -1\n");
      }
    }
    /* the building blocks on the same rows */
    for (int b = 0; b < B; ++b) {
      int32_t* ctx = malloc(sizeof(int32_t) * (S + T + 1));
      int32_t tused = 0;
      const int32_t L = orc_context(S, T, n[b], tok + b * S, samp + b * T, ctx, &tused);
      if (L < 0 || L > S + T) FAIL("context length %d\n", L);
      int32_t* mb = malloc(sizeof(int32_t) * (L + 1));
      orc_match_back(ctx, L, p.max_tree_depth, mb);
      const int64_t nm = L > 0 ? L - 1 : 0;
      const int32_t l1 = orc_kth_largest(mb, nm, 1);
      if (nm > 0 && orc_count_at_least(mb, nm, l1) < 1 && l1 > 0) FAIL("kth/count disagree\n");
      int32_t* sites = malloc(sizeof(int32_t) * 128);
      const int32_t c0 = orc_first_sites(mb, nm, l1 > 0 ? l1 : 1, p.max_occurrences, sites);
      int32_t out[64], counts[64];
      int64_t snum = 0;
      const int32_t cap = orc_spec_cap(&p, l1);
      if (cap < 0 || cap > p.k) FAIL("spec cap %d\n", cap);
      (void)orc_expand(ctx, L, sites, c0, cap, p.mode, p.min_token_prob_ppm, out, counts, &snum);
      if (N > 0 && L > 0) {
        int32_t* gm = malloc(sizeof(int32_t) * (N + 1));
        orc_corpus_match(corpus, N, ctx, L, p.max_tree_depth, gm);
        free(gm);
      }
      free(sites);
      free(mb);
      free(ctx);
    }
    orc_update_state(B, S, T, tok, n, samp, nout);
    for (int b = 0; b < B; ++b)
      if (nout[b] < 0 || nout[b] > S) FAIL("updated length %d outside [0, %d]\n", nout[b], S);
    /* suffix arrays of the corpus and of random texts with repeats */
    if (N > 0) {
      int32_t* sa = malloc(sizeof(int32_t) * N);
      if (orc_suffix_array(corpus, N, sa) != 0) FAIL("suffix array failed\n");
      free(sa);
    }
    free(corpus);
    free(info);
    free(nout);
    free(nv);
    free(draft);
    free(samp);
    free(tok);
    free(n);
  }
  for (int it = 0; it < 300; ++it) {
    const int64_t len = uni(0, 300);
    const int V = uni(1, 4);
    int32_t* t = malloc(sizeof(int32_t) * (len + 1));
    int32_t* sa = malloc(sizeof(int32_t) * (len + 1));
    for (int64_t i = 0; i < len; ++i) t[i] = uni(-1, V - 1);
    if (orc_suffix_array(t, len, sa) != 0) FAIL("suffix array failed\n");
    char* seen = calloc((size_t)len + 1, 1);
    for (int64_t i = 0; i < len; ++i) {
      if (sa[i] < 0 || sa[i] >= len || seen[sa[i]]) FAIL("suffix array not a permutation\n");
      seen[sa[i]] = 1;
    }
    free(seen);
    free(sa);
    free(t);
  }
  printf("oracle sanitizer run: ok\n");
  return 0;
}
