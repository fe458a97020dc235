/*
 * svdraft.h - C ABI of the n-gram self-drafter (in libsvattn.so and in the
 * HIP-free libsvattn_core.so).
 *
 * The drafter proposes the k draft tokens a decode step verifies (AX Engine
 * page, "Core Technical Architecture & Methods": bigram and trigram tables
 * built at run time from the tokens seen, up to 4 drafts per step, an
 * exponential moving average of the acceptance rate with tau = 0.1 that
 * switches speculation off below 0.5; no second model).  Host only: a few
 * hash-table look-ups per drafted token.
 *
 * Rules (the page leaves them open; these are the readings taken):
 *  - Tables count continuations over every token a sequence has observed:
 *    trigram (a, b) -> t and bigram b -> t.
 *  - A draft continues the context with the trigram of its last two tokens
 *    when that pair was seen, else the bigram of its last token, else it
 *    stops; the continuation is the most frequent one, ties going to the one
 *    seen most recently; each drafted token extends the context for the
 *    next, up to max_drafts; drafted tokens never enter the tables.
 *  - The average starts at 1.  Observing tokens after a prediction of m > 0
 *    tokens sets rate = (1 - tau) * rate + tau * matched / m (matched = the
 *    common prefix of the prediction and the observed tokens, in double
 *    precision).  Drafts are returned while rate >= threshold; predictions
 *    are still made and scored while the gate is closed, so it reopens when
 *    the text turns repetitive.
 *
 * Conventions as in svattn.h: int status (0 or a negative KV_E* code),
 * host arrays read during the call, one thread per handle.
 */
#ifndef SVDRAFT_H
#define SVDRAFT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ngram_drafter ngram_drafter; /* opaque */

typedef struct {
  int32_t max_seqs;     /* sequence ids are 0 .. max_seqs-1 */
  int32_t max_drafts;   /* 1 .. 7 (a verify call takes at most 8 rows); the page uses 4 */
  double ema_tau;       /* in (0, 1]; the page uses 0.1 */
  double ema_threshold; /* in [0, 1]; the page uses 0.5 */
} ngram_params;

/* Errors: -1 (KV_EINVAL) for parameters out of range. */
int ngram_create(const ngram_params* p, ngram_drafter** out);
int ngram_destroy(ngram_drafter* d);

/* Tokens sequence seq has accepted (its prompt, then each step's accepted
 * drafts and the token after them), in order; tokens >= 0.  Scores the
 * pending prediction (if any) against them first.  Errors: KV_ENOSEQ,
 * KV_EINVAL (n < 0, null tokens with n > 0, a negative token). */
int ngram_observe(ngram_drafter* d, int32_t seq, const int32_t* tokens, int32_t n);

/* Predict up to max_drafts tokens for seq and keep the prediction for
 * scoring; out (cap >= max_drafts entries) receives the drafts to verify,
 * *n_out of them: 0 while the gate is closed or when the tables have no
 * continuation.  Errors: KV_ENOSEQ, KV_EINVAL (cap < max_drafts). */
int ngram_draft(ngram_drafter* d, int32_t seq, int32_t* out, int32_t cap, int32_t* n_out);

/* ngram_draft for n_seqs sequences: out[i * max_drafts + j], n_out[i]. */
int ngram_draft_batch(ngram_drafter* d, int32_t n_seqs, const int32_t* seq_ids, int32_t* out, int32_t* n_out);

/* ngram_observe for n_seqs sequences: counts[i] tokens each, concatenated. */
int ngram_observe_batch(ngram_drafter* d, int32_t n_seqs, const int32_t* seq_ids, const int32_t* counts,
                        const int32_t* tokens);

/* The gate's state: the average, whether drafts are offered, tokens seen. */
int ngram_state(const ngram_drafter* d, int32_t seq, double* ema, int32_t* enabled, int64_t* observed);

/* Forget a sequence (tables, average, pending prediction). */
int ngram_reset(ngram_drafter* d, int32_t seq);

/* Message of the handle's last failure. */
const char* ngram_last_error(const ngram_drafter* d);

#ifdef __cplusplus
}
#endif

#endif /* SVDRAFT_H */
