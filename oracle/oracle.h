/*
 * oracle.h -- interface of the plain CPU oracle of the suffix-match drafter.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the package smoke check and the CPU-baseline leg
 * of the benchmark are the only users.  Nothing on the GPU product path includes this header,
 * links this library or shares code with it.
 *
 * Sources (each function in oracle.c names the passage it follows):
 *   [GPU-RFC]  vLLM issue "[RFC]: Suffix decoding on GPU (suffix_gpu)", sections Design, Correctness.
 *   [SGPU]     PyPI page "suffix-gpu 0.1.1" (SuffixGPU), sections Highlights, Quickstart,
 *              How it works (steps 1-4), References.
 *   [MRV2]     vLLM docs page "Suffix Decoding", section Model Runner V2.
 *   [BLOG]     gitcode blog "vLLM Suffix Decoding 投机解码实战", section 4 (knob table) and
 *              section 5 (propose flow).
 */
#ifndef SFX_ORACLE_H
#define SFX_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_MODE_LONGEST_FILL = 0, ORC_MODE_SCORED = 1 };
enum { ORC_MAX_NB = 8 };

typedef struct {
  int32_t k;                 /* draft width */
  int32_t max_tree_depth;    /* D: longest suffix considered */
  int32_t num_backoff;       /* nb: ladder candidates per source */
  int32_t max_occurrences;   /* M: earliest continuation sites kept per candidate */
  int32_t mode;              /* ORC_MODE_* */
  int32_t min_self_match;    /* shortest valid self match (>= 1) */
  int32_t min_corpus_match;  /* shortest valid corpus match (>= 2: last-2 probe) */
  int32_t tree_depth_cap;    /* nonzero: match length plus draft length at most D */
  int64_t spec_factor_ppm;   /* max_spec_factor * 1e6 */
  int64_t spec_offset_ppm;   /* max_spec_offset * 1e6 */
  int64_t min_token_prob_ppm;/* min_token_prob * 1e6 */
} orc_params;

typedef struct {
  int32_t L, t;                                   /* context length, sampled tokens used */
  int32_t local_len[ORC_MAX_NB], local_support[ORC_MAX_NB];
  int32_t global_len[ORC_MAX_NB], global_support[ORC_MAX_NB];
  int32_t chosen;                                 /* -1 none, [0,nb) local t, [nb,2nb) global t */
  int32_t chosen_len, c0, n;
  int64_t snum;                                   /* sum of per-depth counts of the winner */
} orc_row_info;

/* building blocks, exported for the pin tests */
int32_t orc_context(int32_t S, int32_t T, int32_t n_raw, const int32_t* row, const int32_t* samp,
                    int32_t* ctx, int32_t* t_out);
void    orc_match_back(const int32_t* ctx, int32_t L, int32_t D, int32_t* mb);
void    orc_corpus_match(const int32_t* C, int64_t N, const int32_t* ctx, int32_t L, int32_t D,
                         int32_t* m);
int32_t orc_kth_largest(const int32_t* vals, int64_t n, int32_t t);
int64_t orc_count_at_least(const int32_t* vals, int64_t n, int32_t l);
int32_t orc_first_sites(const int32_t* vals, int64_t n, int32_t l, int32_t M, int32_t* sites);
int32_t orc_spec_cap(const orc_params* p, int32_t l);
int32_t orc_expand(const int32_t* X, int64_t lenX, const int32_t* sites, int32_t c0, int32_t cap,
                   int32_t scored, int64_t min_prob_ppm, int32_t* out, int32_t* counts,
                   int64_t* snum_out);

/* one drafter call over B rows; corpus may be NULL with N = 0 */
int orc_propose(const orc_params* p, int32_t B, int32_t S, int32_t T,
                const int32_t* num_tokens_no_spec, const int32_t* token_ids, const int32_t* sampled,
                const int32_t* corpus, int64_t N, int32_t* draft, int32_t* num_valid,
                orc_row_info* info, int32_t num_threads);

/* append the leading valid sampled ids to each row, clamped at S */
void orc_update_state(int32_t B, int32_t S, int32_t T, int32_t* token_ids,
                      const int32_t* num_tokens_no_spec, const int32_t* sampled,
                      int32_t* num_tokens_out);

/* suffix array of text[0,n): starts sorted by suffix, signed compare, proper prefix first */
int orc_suffix_array(const int32_t* text, int64_t n, int32_t* sa);

/* alg_bytes.c: the words one call must touch, by category (context, per-request I/O,
 * suffix-array probes, interval scans, voted continuation tokens); sa is the corpus's suffix
 * array (ignored without a corpus). */
int orc_alg_words(const orc_params* p, int32_t B, int32_t S, int32_t T,
                  const int32_t* num_tokens_no_spec, const int32_t* token_ids,
                  const int32_t* sampled, const int32_t* C, int64_t N, const int32_t* sa,
                  int64_t* words_out, int32_t num_threads);

#ifdef __cplusplus
}
#endif
#endif
