/*
 * pa_sched.h - continuous-batching scheduler of libpa.so over a pa_mgr
 * (pa_host.h).  Host-only; no call here touches a GPU.
 *
 * [engine] "Building a paged inference engine from scratch, and measuring it
 * honestly", "02 The engine": requests are admitted roughly in order, but the
 * scheduler may look a few requests ahead and admit whichever fit; after too
 * many requests are skipped in a row it falls back to blocking mode until
 * memory frees up; new requests join the running batch; every call runs four
 * phases (release finished sequences, grow the running ones, admit waiting
 * requests, assemble the batch), and prefill versus decode follows from the
 * token counts.
 *
 * Policy (the readings where the page is silent):
 * - A request has a prompt of P tokens and generates N tokens.  Its first
 *   step reserves its P prompt positions (one row block of q_len P) and yields
 *   token 1; each later step reserves one position (the previous token) and
 *   yields the next; after N tokens it is finished and its blocks are released
 *   at the start of the next step.  Lifetime: P + N - 1 positions.
 * - A request fits when its lifetime blocks ceil((P + N - 1) / block_size)
 *   fit in the free blocks minus those still owed to running requests (their
 *   lifetime blocks minus the blocks they hold), its P rows fit in the step's
 *   row budget (max_batch_tokens minus one row per running request), and
 *   fewer than max_seqs sequences would run.  Admission reserves the
 *   lifetime, so a running request never runs out of blocks.
 * - The first `lookahead` waiting requests are considered in arrival order;
 *   each that fits is admitted.  When the oldest waiting request is passed
 *   over while a later one is admitted, its skip count grows; beyond
 *   `max_skips` the scheduler blocks: only the oldest may be admitted, once
 *   it fits, which ends blocking mode.
 * - A batch lists the running requests (admission order), then the requests
 *   admitted in this step (admission order).
 *
 * Conventions as in pa_host.h: host pointers owned by the caller, int32
 * arrays, pa_host_status results, one thread per scheduler.  The scheduler
 * keeps a pointer to its manager, which must outlive it; the manager must
 * not be used for other sequences meanwhile (its free count is the
 * scheduler's budget).
 */
#ifndef PA_SCHED_H
#define PA_SCHED_H

#include <stdint.h>

#include "pa_host.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_sched pa_sched;

/* NULL for invalid arguments (any size < 1, max_skips < 0). */
pa_sched* pa_sched_create(pa_mgr* m, int32_t max_batch_tokens, int32_t max_seqs, int32_t lookahead,
                          int32_t max_skips);
void pa_sched_destroy(pa_sched* s);

/* Queue a request; *rid = its id (counting up from 0).  PA_HOST_ERR_ARG when
 * it could never be admitted (P or N < 1, P > max_batch_tokens, or more
 * lifetime blocks than the pool holds). */
int32_t pa_sched_add(pa_sched* s, int32_t prompt_len, int32_t new_tokens, int32_t* rid);

/* A request with token ids (prompt = tokens[0 .. n-1]): on admission its
 * prompt is matched against the manager's prefix cache (pa_host.h), its first
 * step reserves only the positions after the cached ones, and after that step
 * its full prompt blocks are published.  Admission still reserves the whole
 * lifetime (cached blocks count among the available ones). */
int32_t pa_sched_add_tokens(pa_sched* s, const int32_t* tokens, int32_t n, int32_t new_tokens, int32_t* rid);

/* Prompt tokens served from the prefix cache so far. */
int64_t pa_sched_cached_tokens(const pa_sched* s);

/* Widest block table any step can need: the largest lifetime in blocks of
 * the requests added so far (at least 1). */
int32_t pa_sched_max_width(const pa_sched* s);

/*
 * pa_sched_step - one step: the four phases, then pa_mgr_step for the batch.
 *   rids, sids, q_lens [max_seqs]  the batch's requests, their manager
 *                      sequence ids and rows (1 for a decode, P for a prefill);
 *                      *num_rows = how many.
 *   finished [cap_finished]  requests released in phase 1; *num_finished.
 *   width, slot_mapping [max_batch_tokens], block_tables [max_seqs][width],
 *   seq_lens [max_seqs]  as for pa_mgr_step (width >= pa_sched_max_width).
 * An empty batch (nothing running, nothing admissible) is not an error.
 */
int32_t pa_sched_step(pa_sched* s, int32_t* rids, int32_t* sids, int32_t* q_lens, int32_t* num_rows,
                      int32_t* finished, int32_t cap_finished, int32_t* num_finished, int32_t width,
                      int32_t* slot_mapping, int32_t* block_tables, int32_t* seq_lens);

/* Queue sizes, blocking mode and tokens generated so far (any pointer may be NULL). */
int32_t pa_sched_counts(const pa_sched* s, int32_t* waiting, int32_t* running, int32_t* finished,
                        int32_t* blocking, int64_t* generated);

#ifdef __cplusplus
}
#endif

#endif /* PA_SCHED_H */
