/*
 * sfx.h -- C-ABI of libsfx, the MI355X (gfx950) suffix-match drafter.
 *
 * The drafter proposes, for every request of a decode batch, a draft of up to k next tokens by
 * matching the request's last tokens against (a) its own prompt+output and (b) a shared corpus
 * of finished responses, then expanding the best match by depth-wise frequency vote.
 *
 * Passages this interface follows (cited by page title and section):
 *   - vLLM issue "[RFC]: Suffix decoding on GPU (suffix_gpu)", Design: the proposer contract
 *     propose(k, num_tokens_no_spec, token_ids, sampled, counts) -> (drafts [B,k],
 *     valid counts [B]); finished requests are ingested into a cross-request index.
 *   - PyPI page "suffix-gpu 0.1.1", Highlights and Quickstart: device tensors in and out, no
 *     per-step host synchronisation, static shapes; int32 state token_ids [B,S],
 *     num_tokens_no_spec [B], sampled [B,T] (-1 padded); draft [B,k] (-1 padded) and
 *     num_valid [B]; harvest_finished(row_indices, lengths, token_ids) and poll().
 *   - same page, How it works steps 1-4: local match_back ladder, global suffix-array match,
 *     fused vote + score, corpus ring + delta with a side-stream suffix-array rebuild that is
 *     swapped without moving buffers.
 *   - vLLM docs "Suffix Decoding", Model Runner V2: longest suffix up to max_tree_depth,
 *     corpus probed by the last 2 and last 4 tokens, longer match wins, fill with the last
 *     sampled token, corpus budget with oldest-first eviction.
 *   - gitcode blog "vLLM Suffix Decoding 投机解码实战", section 4: knob ranges
 *     (max_tree_depth >= 1, max_spec_factor >= 0, min_token_prob in [0,1]).
 *
 * Conventions (all entry points):
 *   - Every array argument is a DEVICE pointer owned by the caller unless stated otherwise; the
 *     library never frees it and never keeps it past the call.  Arrays are dense row-major.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is enqueued on
 *     it; entry points on the propose path neither synchronise the host nor allocate.
 *   - Return value: SFX_OK (0) or a negative SFX_E* code; on error nothing was enqueued and
 *     sfx_last_error() returns a thread-local message.  Values the host cannot see without a
 *     synchronisation (lengths stored in device memory) are clamped on the device instead of
 *     being rejected.
 *   - A context is used from one host thread at a time and its work is ordered by the streams
 *     given; two calls that overlap on different streams without ordering race.
 */
#ifndef SFX_H
#define SFX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SFX_OK = 0,
  SFX_EINVAL = -1,     /* bad argument or configuration */
  SFX_ENOMEM = -2,     /* device allocation failed (only sfx_create allocates) */
  SFX_ECAPACITY = -3,  /* shape above what the context was created for */
  SFX_EHIP = -4,       /* a HIP runtime call failed */
  SFX_ESTATE = -5,     /* call not valid in the context's current state */
  SFX_EIO = -6         /* a corpus file could not be written or read, or is not valid */
};

enum {
  SFX_MODE_LONGEST_FILL = 0, /* vLLM docs, Model Runner V2: longer match wins, fill with the
                                last sampled token, no stop rule (requires num_backoff == 1) */
  SFX_MODE_SCORED = 1        /* suffix-gpu page, How it works step 3: adaptive stop rule and
                                score; best score wins; -1 padding */
};

enum {
  SFX_FLAG_STREAM_CONTEXT = 1, /* sfx_propose reads each context from device memory instead of
                                  staging it in the workgroup's LDS (same results).  Without it
                                  a row is staged when it fits (max_seq up to about 19K tokens)
                                  and streamed otherwise. */
  SFX_FLAG_CHECK_INPUTS = 2,   /* the propose and ingest calls also launch a check of their
                                  device-resident inputs that sets SFX_ERR_* bits in the
                                  context's error word (sfx_debug_errors); results do not
                                  change */
  SFX_FLAG_TREE_DEPTH_CAP = 4  /* gitcode blog section 4, parameter table: max_tree_depth bounds
                                  the match length plus the draft length, so a candidate of
                                  match length l drafts at most max(0, max_tree_depth - l)
                                  tokens (both modes; off by default, where only the match
                                  length is bounded) */
};

/* Bits of the sticky device error word.  Each names an input that the device clamps or ignores
 * because the host cannot see it without a synchronisation; the calls' results follow the
 * documented clamping either way. */
enum {
  SFX_ERR_LENGTH = 1,            /* a length outside [0, S] (num_tokens_no_spec, lengths,
                                    counts outside [0, T]) or a decreasing document offset */
  SFX_ERR_NEGATIVE_TOKEN = 2,    /* a negative id inside a row prefix or a document */
  SFX_ERR_SAMPLED_AFTER_PAD = 4, /* a non-negative sampled id after a negative one (ignored) */
  SFX_ERR_ROW_INDEX = 8,         /* an ingest row index outside the rows (ignored) */
  SFX_ERR_SYNC_TIMEOUT = 16      /* a propose workgroup's bounded wait for its other wavefronts
                                    ran out (raised with or without SFX_FLAG_CHECK_INPUTS; the
                                    drafts of that call are unreliable) */
};

typedef struct sfx_config {
  int32_t k;                /* draft width, 1..32 */
  int32_t max_tree_depth;   /* D: longest suffix matched, 1..64 (>= 2 when a corpus is used) */
  int32_t num_backoff;      /* nb: ladder candidates per source, 1..8 */
  int32_t max_occurrences;  /* M: earliest continuation sites kept per candidate, 1..128 */
  int32_t mode;             /* SFX_MODE_* */
  int32_t min_self_match;   /* shortest self match that makes a candidate, >= 1 */
  int32_t min_corpus_match; /* shortest corpus match that makes a candidate, 2..max_tree_depth */
  int32_t max_batch;        /* largest B accepted by sfx_propose */
  int32_t max_seq;          /* largest S accepted by sfx_propose (row capacity), 0..32768 */
  int32_t max_sampled;      /* largest T accepted by sfx_propose, 0..16 */
  int64_t spec_factor_ppm;  /* max_spec_factor * 1e6, >= 0 (SCORED) */
  int64_t spec_offset_ppm;  /* max_spec_offset * 1e6, >= 0 (SCORED) */
  int64_t min_token_prob_ppm; /* min_token_prob * 1e6, 0..1e6 (SCORED) */
  int64_t corpus_capacity;  /* ring size in tokens, separators included; 0 = no corpus;
                               at most 2^30 */
  int32_t flags;            /* SFX_FLAG_* (0 = defaults) */
  int32_t reserved;         /* must be 0 */
} sfx_config;

typedef struct sfx_ctx sfx_ctx;

/* Validates *cfg and allocates every device buffer the context will ever use (rows scratch,
 * corpus ring, double-buffered corpus index, control block and, for max_batch <= 1024, the
 * per-call pair index of the delta) on the current HIP device.
 * Returns SFX_EINVAL for a configuration outside the ranges above, SFX_ENOMEM when device
 * memory runs out.  *out receives the context. */
int sfx_create(const sfx_config* cfg, sfx_ctx** out);

/* Waits for the context's own side-stream work, then frees everything it allocated. */
void sfx_destroy(sfx_ctx* ctx);

/* Thread-local text of the last error (never NULL). */
const char* sfx_last_error(void);

/* One drafter step for B requests (RFC page, Design; suffix-gpu page, How it works 1-3).
 *   num_tokens_no_spec [B]   row prefix length n_b; clamped to [0,S] on the device
 *   token_ids          [B,S] resident rows; only token_ids[b, 0:n_b] is read
 *   sampled            [B,T] last verifier output, -1 padded; the leading non-negative
 *                            entries are appended (virtually) to the row prefix
 *   draft              [B,k] out: proposed ids; the rest of the row is the last sampled token
 *                            (LONGEST_FILL) or -1 (SCORED); all -1 when a row has no sampled id
 *   num_valid          [B]   out: number of proposed ids
 * Token ids must be >= 0.  Requires B <= max_batch, S <= max_seq, T <= max_sampled
 * (else SFX_ECAPACITY).  Reads the corpus index that is live when the kernel runs.  While some
 * ingest since the context's last swapped-in rebuild is pending (and B <= 1024), the call first
 * groups the delta's positions by the batch's tail pairs (four small passes on `stream`,
 * no allocation); otherwise, or in a graph captured without them, each request scans the
 * delta itself.  Both give the same result. */
int sfx_propose(sfx_ctx* ctx, int32_t B, int32_t S, int32_t T, const int32_t* num_tokens_no_spec,
                const int32_t* token_ids, const int32_t* sampled, int32_t* draft,
                int32_t* num_valid, void* stream);

/* The masked form (suffix-gpu page, Quickstart: propose(num_tokens_no_spec, token_ids,
 * combined_mask), for callers that keep token_ids up to date themselves).  Row b's context is
 * token_ids[b, 0:clamp(n_b, 0, S)] alone; mask [B] (device int32) selects the rows to draft:
 * a row with mask[b] == 0, or an empty row, gets no draft (num_valid 0, all -1).  Otherwise as
 * sfx_propose, with the context's last token in the role of the last sampled id (LONGEST_FILL
 * fills with it).  Needs max_sampled >= 1 (else SFX_ECAPACITY); uses context-owned scratch,
 * so it neither synchronises nor allocates. */
int sfx_propose_masked(sfx_ctx* ctx, int32_t B, int32_t S, const int32_t* num_tokens_no_spec,
                       const int32_t* token_ids, const int32_t* mask, int32_t* draft,
                       int32_t* num_valid, void* stream);

/* The counted form (RFC page, Design: the ngram_gpu contract propose(k, num_tokens_no_spec,
 * token_ids, sampled, counts) -> (drafts [B,k], valid counts [B])).  counts [B] (device int32)
 * is the number of valid entries of sampled[b], clamped to [0, T], in place of the -1 padding:
 * the context appends sampled[b, 0:counts[b]] up to its first negative entry.  k is this
 * call's draft width, 1 .. the configured k (else SFX_EINVAL / SFX_ECAPACITY): draft is [B, k]
 * and the SCORED cap is taken against it.  Otherwise as sfx_propose; uses context-owned
 * scratch, so it neither synchronises nor allocates. */
int sfx_propose_counts(sfx_ctx* ctx, int32_t k, int32_t B, int32_t S, int32_t T,
                       const int32_t* num_tokens_no_spec, const int32_t* token_ids,
                       const int32_t* sampled, const int32_t* counts, int32_t* draft,
                       int32_t* num_valid, void* stream);

/* State update (suffix-gpu page, Quickstart: propose_with_update).  Writes the leading
 * non-negative sampled ids of row b after its clamped prefix, as many as fit in S, and stores
 * the new length in num_tokens_out[b].  token_ids is modified in place.  Needs no context. */
int sfx_update_state(int32_t B, int32_t S, int32_t T, int32_t* token_ids,
                     const int32_t* num_tokens_no_spec, const int32_t* sampled,
                     int32_t* num_tokens_out, void* stream);

/* Ingest finished rows into the corpus (suffix-gpu page, Quickstart: harvest_finished; How it
 * works step 4).  Document r is token_ids[row_indices[r], 0:clamp(lengths[r], 0, S)], appended
 * in r order and followed by one -1 separator; afterwards the oldest documents are evicted
 * while the live total exceeds corpus_capacity.  token_ids is [num_rows, S]; a row index
 * outside [0, num_rows) makes an empty document.  New documents become visible to
 * sfx_propose at once (matched in the delta until the next rebuild is swapped in).
 * SFX_ESTATE when the context has no corpus. */
int sfx_harvest_finished(sfx_ctx* ctx, int32_t R, const int32_t* row_indices,
                         const int32_t* lengths, const int32_t* token_ids, int32_t num_rows,
                         int32_t S, void* stream);

/* In-flight ingest (RFC page "[RFC]: Suffix decoding on GPU (suffix_gpu)", Design: in-flight
 * responses are ingested off the critical path, finished requests are final-flushed before
 * their batch rows are reused; the suffix_gpu_ingest_chunk knob).  The context keeps an ingest
 * cursor for every batch row in [0, max_batch), 0 at creation.  For entry r, with
 * row = row_indices[r] and n = clamp(lengths[r], 0, S): the chunk token_ids[row, cursor:n] is
 * appended as one document (followed by -1) when it holds at least max(min_chunk, 1) tokens, or
 * when final_flags[r] != 0 and it is not empty; the cursor then moves to n.  After a final
 * flush the cursor is 0, so the row can start a new request.  n below the cursor (a row reused
 * without a flush) restarts the row at 0.  Chunks are separate documents: matches and
 * continuations do not cross from one chunk to the next.  Entries append in r order; an entry
 * that appends nothing adds no document; a row listed again in the same call, or outside
 * [0, min(num_rows, max_batch)), is ignored.  final_flags may be NULL (no flush).  Documents and
 * eviction otherwise as sfx_harvest_finished; all decisions are taken on the device, so the
 * call neither synchronises nor allocates.  R at most 65536 (else SFX_ECAPACITY). */
int sfx_ingest_inflight(sfx_ctx* ctx, int32_t R, const int32_t* row_indices,
                        const int32_t* lengths, const int32_t* final_flags,
                        const int32_t* token_ids, int32_t num_rows, int32_t S, int32_t min_chunk,
                        void* stream);

/* Ingest packed documents: document d is tokens[doc_offsets[d] : doc_offsets[d+1]] (offsets
 * int64, non-decreasing, device memory); otherwise as sfx_harvest_finished. */
int sfx_ingest(sfx_ctx* ctx, int32_t num_docs, const int64_t* doc_offsets, const int32_t* tokens,
               void* stream);

/* Rebuild the corpus index over the live corpus and make it live, in stream order on `stream`
 * (snapshot copy, suffix array by prefix doubling, n-gram interval tables).  The host thread
 * waits for the stream while it drives the doubling rounds. */
int sfx_rebuild(sfx_ctx* ctx, void* stream);

/* Same rebuild, off the critical path: the snapshot is copied in order on `stream`, the
 * suffix array and tables are built into the idle buffer by the library's worker thread on the
 * context's own side stream, and sfx_poll swaps them in.  SFX_ESTATE if a rebuild is already
 * in flight. */
int sfx_rebuild_async(sfx_ctx* ctx, void* stream);

/* Non-blocking: if an asynchronous rebuild has finished, enqueue on `stream` the swap that makes
 * it live (buffers never move, so captured work keeps its pointers) and set *swapped = 1;
 * otherwise *swapped = 0.  `swapped` is a host pointer. */
int sfx_poll(sfx_ctx* ctx, int32_t* swapped, void* stream);

/* Block until an in-flight asynchronous rebuild has finished, then swap it in on `stream`.
 * No-op when none is in flight. */
int sfx_wait_rebuild(sfx_ctx* ctx, void* stream);

/* Copy the live corpus text (documents in ingest order, each followed by -1) into text_out
 * (device, capacity `cap` ints) and its length into *n_out (host pointer).  Synchronises the
 * stream.  SFX_ECAPACITY if cap is too small. */
int sfx_corpus_snapshot(sfx_ctx* ctx, int32_t* text_out, int64_t cap, int64_t* n_out,
                        void* stream);

/* Per-slot acceptance estimate (vLLM docs "Suffix Decoding", Use adaptive verification at
 * higher concurrency: a running estimate of each draft position's chance of acceptance, keyed
 * by the draft's source, its match length and the position, lets the scheduler skip verifying
 * positions that are unlikely to pay off).  Every sfx_propose records, per row b < B, its winning candidate: source (0 the
 * request's own context, 1 the corpus), match length, and num_valid (no winner: nothing).
 * The context keeps a table of counts per (source, length 0..64, slot 0..31): proposed and
 * accepted.
 *
 * sfx_accept_estimate: est_ppm [B, k] (device, int32) receives, for every slot d < num_valid of
 *   row b's last propose, floor(10^6 * (accepted + 1) / (proposed + 2)) of its cell (Laplace's
 *   rule: 500000 for an unseen cell), and 0 for the other slots.
 * sfx_accept_feedback: num_accepted [B] (device) is the number of draft tokens the verifier
 *   accepted for each row of the last propose (a prefix of the draft; clamped to
 *   [0, num_valid]).  Every drafted slot d of the row adds one proposal to its cell, and one
 *   acceptance when d < num_accepted.  The row's record is consumed, so feedback counts each
 *   propose once.
 * sfx_accept_reset: clears the table and the records.
 * sfx_accept_counts: copies the table to `counts` (device, 2*65*32*2 uint64, index
 *   ((source * 65 + length) * 32 + slot) * 2 + {0 proposed, 1 accepted}).
 * All four enqueue on `stream` and neither synchronise nor allocate.  B at most max_batch
 * (else SFX_ECAPACITY). */
int sfx_accept_estimate(sfx_ctx* ctx, int32_t B, int32_t* est_ppm, void* stream);
int sfx_accept_feedback(sfx_ctx* ctx, int32_t B, const int32_t* num_accepted, void* stream);
int sfx_accept_reset(sfx_ctx* ctx, void* stream);
int sfx_accept_counts(sfx_ctx* ctx, uint64_t* counts, void* stream);

/* Batch-bucketed graphs of the drafter step (RFC page "[RFC]: Suffix decoding on GPU
 * (suffix_gpu)", Design, Proposer bullet: the draft chain is captured per batch-size bucket at
 * engine warm-up, so no serving step pays for a capture, and runs eagerly when capture fails or
 * graphs are disabled).
 *
 * sfx_graphs_create captures, for every bucket size Bp of `buckets` (nbuckets entries, host
 * array, strictly ascending, 1 <= Bp <= max_batch, at most 64 buckets), the step over the first
 * Bp rows of the caller's persistent device buffers:
 *   num_tokens   [max bucket]     row prefix lengths (rows past B are overwritten, see below)
 *   token_ids    [max bucket, S]  resident rows (written only with SFX_GRAPHS_UPDATE_STATE)
 *   sampled      [max bucket, T]  sampled ids, -1 padded (rows past B are overwritten)
 *   draft        [max bucket, k]  out, as for sfx_propose
 *   num_valid    [max bucket]     out, as for sfx_propose
 *   num_tokens_out [max bucket]   out, new lengths (SFX_GRAPHS_UPDATE_STATE only, else NULL;
 *                                 may be num_tokens itself)
 * The chain of a bucket is sfx_propose(Bp rows), then with SFX_GRAPHS_UPDATE_STATE
 * sfx_update_state(Bp rows).  Each bucket gets two graphs: one for B == Bp, and one that first
 * empties rows B .. Bp-1 (num_tokens 0, sampled -1: such a row reads nothing, proposes nothing,
 * gets draft -1 and num_valid 0, and with the update keeps its token_ids row).  Capture happens
 * on a stream of the library's own, so `stream` is only used to upload the graphs; no kernel
 * runs during creation.  A bucket whose capture or instantiation fails is run eagerly
 * instead (sfx_graphs_stats reports which).  The buffers must stay allocated, and the context
 * alive, until sfx_graphs_destroy.  The graphs read the corpus index and delta that are live
 * when they run (swaps keep every buffer in place).
 *
 * sfx_graphs_propose(g, B, stream) runs the step for the first B rows: the graph of the
 * smallest bucket >= B, replayed on `stream` (B == 0 does nothing).  With B above the largest
 * bucket, with a bucket that was not captured, or with SFX_GRAPHS_EAGER, the same chain runs
 * eagerly for exactly B rows (sfx_propose's errors apply).  Replays neither allocate nor wait.
 * Not thread-safe for one object: calls on one object must be serialised by the caller. */
enum {
  SFX_GRAPHS_EAGER = 1,         /* capture nothing: every call runs eagerly */
  SFX_GRAPHS_UPDATE_STATE = 2,  /* the chain ends with sfx_update_state */
  SFX_GRAPHS_DELTA_INDEX = 4,   /* every chain groups the delta by tail pair first (as
                                   sfx_propose does while an ingest is pending), for engines that
                                   ingest every step; without it the replays scan the delta */
  SFX_GRAPHS_DEBUG_BREAK_ODD = 8 /* test hook: a call that is not allowed under capture is made
                                   inside the capture of every odd-indexed bucket, so those
                                   captures fail and those buckets run eagerly */
};
typedef struct sfx_graphs sfx_graphs;
int sfx_graphs_create(sfx_ctx* ctx, int32_t nbuckets, const int32_t* buckets, int32_t S,
                      int32_t T, int32_t* num_tokens, int32_t* token_ids, int32_t* sampled,
                      int32_t* draft, int32_t* num_valid, int32_t* num_tokens_out,
                      int32_t flags, void* stream, sfx_graphs** out);
int sfx_graphs_propose(sfx_graphs* g, int32_t B, void* stream);
/* Bit i of *exact_mask / *padded_mask: bucket i's graph for B == Bp / B < Bp was captured.
 * *replays and *eager_calls count the calls of sfx_graphs_propose so far.  NULL outputs are
 * skipped. */
int sfx_graphs_stats(sfx_graphs* g, int32_t* nbuckets, uint64_t* exact_mask,
                     uint64_t* padded_mask, int64_t* replays, int64_t* eager_calls);
/* Frees the graphs (not the buffers).  Work already launched may still be running. */
void sfx_graphs_destroy(sfx_graphs* g);

/* Persist the corpus (suffix-gpu page, TODO: the cross-request global memory -- corpus ring,
 * suffix array and delta -- is saved to disk and restored across sessions, so the accumulated
 * statistics survive a restart instead of being rebuilt).  Writes the host file `path`: the
 * live documents (indexed and delta alike, in ingest order), their start positions, the ring
 * counters, and the live index as its snapshot text and suffix array.  The n-gram tables are
 * not written: sfx_load derives them from the suffix array.  Synchronises `stream` and copies
 * through host memory.  An asynchronous rebuild still in flight keeps running and is not saved;
 * what it covers is in the saved delta.  SFX_ESTATE without a corpus, SFX_EIO when the file
 * cannot be written.
 *
 * File layout, little-endian:
 *   bytes  0..7   magic "SFXCORP1"
 *   bytes  8..71  int64 capacity, head, tail, doc_head, doc_tail, snap_start, snap_end,
 *                 then uint64 checksum.  Live tokens are logical positions [tail, head); live
 *                 documents are numbers [doc_tail, doc_head); the index covers logical
 *                 positions [snap_start, snap_end) (empty when no index is live).
 *   then          int32 tokens[head - tail]                (each document ends with -1)
 *                 int64 doc_start[doc_head - doc_tail]      (logical start of each document)
 *                 int32 index_text[snap_end - snap_start]
 *                 int32 suffix_array[snap_end - snap_start]
 *   checksum      FNV-1a over the payload's 32-bit words: h = 14695981039346656037, then for
 *                 every word w: h = (h xor w) * 1099511628211 (mod 2^64). */
int sfx_save(sfx_ctx* ctx, const char* path, void* stream);

/* Restore a file written by sfx_save into a context created with the same corpus_capacity,
 * replacing its whole corpus state; the n-gram tables are built from the saved suffix array on
 * `stream`, and the restored index is live when the call returns.  Every counter, the document
 * structure and the suffix array (a permutation) are checked on the host before anything is
 * copied.  SFX_EIO for a file that cannot be read, is truncated, has trailing bytes, a wrong
 * magic or checksum, or inconsistent contents (the context is then unchanged); SFX_EINVAL for a
 * capacity mismatch; SFX_ESTATE without a corpus or with an asynchronous rebuild in flight or
 * finished but not yet swapped in (sfx_wait_rebuild first).  The in-flight ingest cursors and
 * the acceptance counts belong to the serving batch, not to the corpus: they are neither
 * saved nor replaced.  Synchronises `stream`. */
int sfx_load(sfx_ctx* ctx, const char* path, void* stream);

/* The optional debug call for the clamping convention of the device-resident inputs: waits for
 * `stream`, stores the context's sticky error word (SFX_ERR_* bits raised since the last read)
 * in *bits_out (host memory) and clears it.  The word is only written by calls of a context
 * created with SFX_FLAG_CHECK_INPUTS; otherwise it reads 0.  Synchronises `stream`. */
int sfx_debug_errors(sfx_ctx* ctx, uint32_t* bits_out, void* stream);

/* Statistics of the last index build (sfx_rebuild, or an asynchronous rebuild that has
 * finished): *rounds_out = prefix-doubling rounds of its suffix array (the first sort plus
 * every doubling round that had suffixes left to sort), *tokens_out = its snapshot tokens.
 * Host values; waits for the build's last round if it is still running.  SFX_ESTATE while an
 * asynchronous rebuild is in flight or without a corpus. */
int sfx_rebuild_stats(sfx_ctx* ctx, int32_t* rounds_out, int64_t* tokens_out);

/* Debug export of the live corpus index (suffix-gpu page, How it works step 4: the snapshot
 * text and its suffix array, rebuilt on a side stream and swapped in): copies the live buffer's
 * snapshot text into text_out and its suffix array into sa_out (device, capacity `cap` ints
 * each) and the snapshot length into *n_out (host; 0, with nothing copied, before the first
 * rebuild).  The snapshot is the live corpus of the rebuild that produced the index; documents
 * evicted since then stay in it (proposes skip them).  Synchronises `stream`.  SFX_ECAPACITY if
 * cap is too small, SFX_ESTATE without a corpus. */
int sfx_debug_index(sfx_ctx* ctx, int32_t* text_out, int32_t* sa_out, int64_t cap,
                    int64_t* n_out, void* stream);

/* Test hook for the failure path of the rebuild (suffix-gpu page, How it works step 4: the
 * index is rebuilt on a side stream and double-buffered, so a rebuild that does not finish must
 * leave the live one in place).  The next rebuild of ctx -- sfx_rebuild, or the worker started
 * by sfx_rebuild_async -- fails with SFX_EHIP after building into the inactive buffer and
 * before the swap: sfx_rebuild returns the error; sfx_poll then reports it with *swapped = 0 and
 * sfx_wait_rebuild returns it.  The live index, the corpus and its delta are unchanged, so
 * proposes keep their results, and the rebuild after that works as usual.  SFX_ESTATE without a
 * corpus. */
int sfx_debug_fail_next_rebuild(sfx_ctx* ctx);

/* Suffix array (suffix-gpu page, Highlights and References: Manber & Myers prefix doubling):
 * sa[r] = start of the r-th smallest suffix of text[0:n], tokens compared as signed int32, a
 * proper prefix before the longer suffix.  text and sa are device arrays; workspace is a
 * device buffer of at least sfx_suffix_array_workspace_bytes(n) bytes.  The doubling rounds
 * count the suffixes left to sort on the device; the host reads those counts two rounds late
 * through pinned memory, with no wait per round, and stops enqueueing once one is 0.  Returns
 * after `stream` has finished the build.  n at most 2^30. */
size_t sfx_suffix_array_workspace_bytes(int64_t n);
int sfx_build_suffix_array(const int32_t* text, int64_t n, int32_t* sa, void* workspace,
                           size_t workspace_bytes, void* stream);

/* For callers that cannot allocate (code under graph capture, tight serving loops, harnesses
 * that forbid allocation): sfx_build_suffix_array without a workspace argument and without
 * any allocation.  Same result in sa.  Its workspace is a device array held by the library on
 * each device it runs on, until the process ends: n is at most 2^20 (SFX_ECAPACITY above
 * that), for about 40 MiB per device.  It calls no allocator, creates no event, uses no host
 * memory and does not wait: every doubling round is enqueued on `stream` (the rounds after
 * convergence do nothing) and the call returns; sa is ready once `stream` reaches that point.
 * Every call on one device shares that array, so calls that overlap on one device (on
 * different streams, or from several threads) race: order them, for example on one stream. */
int sfx_build_suffix_array_noalloc(const int32_t* text, int64_t n, int32_t* sa, void* stream);

#ifdef __cplusplus
}
#endif
#endif
