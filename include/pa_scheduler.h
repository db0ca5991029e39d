/*
 * pa_scheduler.h -- iteration-level (continuous) batching decisions on the
 * host: which requests run their prompt's prefill, which yield a token and
 * which wait, one generation boundary at a time.
 *
 * What it follows:
 *   - "What problem does PagedAttention solve, and what is continuous
 *     batching?" (datarekha), section "What continuous batching changes":
 *     the active set is revisited at every generation boundary; a finished
 *     request leaves at once and a queued one takes its place once its
 *     prompt's prefill is scheduled.  Section "How the two fit together in
 *     production": queue -> prefill and block allocation -> decode pool ->
 *     release on finish -> admit waiting requests when capacity allows;
 *     long prompts are processed in chunks under a per-step token cap.
 *     Section "A concrete memory example": a conventional design reserves
 *     4,096 tokens per request; paged allocation hands out blocks as they
 *     fill.  Section "The senior-level nuance": when the pool is full the
 *     server must queue, preempt and recompute, offload or reject.
 *
 * The pages fix no policy; this scheduler takes the same readings as the
 * Python model in paged_kv_cache_400_amd/scheduler.py, and decides exactly
 * as it does (the tests compare the two plan by plan):
 *   - an iteration is one generation boundary; a request's prefill (its
 *     whole prompt, or the chunks of it that fit under the step's token cap,
 *     in admission order) runs in the iterations after its admission; the
 *     iteration that completes its prompt also yields its first token; every
 *     other running request yields one token per iteration; a request that
 *     reaches its generation length leaves at the end of that iteration;
 *   - admission is first come, first served: the head of the queue waits
 *     until it fits, and nothing behind it is admitted first;
 *   - PA_SCHED_STATIC: a batch of up to max_batch requests is formed when no
 *     batch is running and holds its slots until its last member finishes,
 *     each member reserving reserve_tokens; PA_SCHED_RESERVED: iteration-
 *     level batching, each request reserving reserve_tokens tokens of the
 *     pool for its whole life; PA_SCHED_PAGED: iteration-level batching over
 *     blocks: a request is admitted when the free blocks cover its prompt
 *     plus one token, takes a block whenever its last one fills, and if the
 *     pool cannot supply one the most recently admitted running request is
 *     preempted (its progress dropped, back to the front of the queue) until
 *     the growth fits.
 *
 * Host memory only.  A scheduler is not safe to use from several threads at
 * once.
 */
#ifndef PA_SCHEDULER_H
#define PA_SCHEDULER_H

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_sched pa_sched;

enum { PA_SCHED_STATIC = 0, PA_SCHED_RESERVED = 1, PA_SCHED_PAGED = 2 };

/*
 * Creates a scheduler over a pool of num_blocks blocks of block_size tokens.
 * mode: PA_SCHED_STATIC, PA_SCHED_RESERVED or PA_SCHED_PAGED.  max_batch:
 * running requests at most; max_step_tokens: prefill tokens per iteration
 * at most; reserve_tokens: a reservation (static and reserved modes).
 * Errors: PA_ERR_NULL (out), PA_ERR_SHAPE (unknown mode, a size < 1).
 */
pa_status pa_sched_create(int32_t mode, int32_t num_blocks, int32_t block_size,
                          int32_t max_batch, int32_t max_step_tokens, int32_t reserve_tokens,
                          pa_sched** out);

/* Frees a scheduler (NULL is ignored). */
void pa_sched_destroy(pa_sched* s);

/*
 * Adds n requests: rids[i] (distinct, not seen before), arriving at
 * iteration arrivals[i] (admitted no earlier), prompt_lens[i] >= 1 prompt
 * tokens, gen_lens[i] >= 1 tokens to generate.  Pending requests are taken
 * in order of (arrival, rid).  Errors: PA_ERR_NULL, PA_ERR_SHAPE (a repeated
 * rid, a length < 1, n < 0); nothing is added then.
 */
pa_status pa_sched_add(pa_sched* s, const int64_t* rids, const int64_t* arrivals,
                       const int32_t* prompt_lens, const int32_t* gen_lens, int32_t n);

/*
 * One iteration's decisions.  The arrays point into the scheduler and stay
 * valid until its next pa_sched_step or pa_sched_destroy.  Rids are listed
 * in admission order unless noted.
 */
typedef struct pa_sched_plan {
  int64_t iteration;        /* 1 for the first step */
  int32_t n_prefill;
  const int64_t* prefill;   /* n_prefill x 3: rid, first prompt token, count */
  int32_t n_decode;
  const int64_t* decode;    /* requests yielding a token */
  int32_t n_padded;
  const int64_t* padded;    /* static: finished rows still in the batch */
  int32_t n_admitted;
  const int64_t* admitted;
  int32_t n_finished;
  const int64_t* finished;  /* yielded their last token */
  int32_t n_preempted;
  const int64_t* preempted; /* in the order they were preempted */
  int32_t n_released;
  const int64_t* released;  /* left the running set at the end of the step */
  int32_t running;          /* running requests after the step */
  int32_t queued;           /* waiting in the queue after the step */
  int64_t blocks_used;      /* paged: blocks the running requests hold; else reserved */
} pa_sched_plan;

/*
 * Runs one iteration and describes it in *plan.  Errors: PA_ERR_NULL,
 * PA_ERR_SHAPE (static or reserved mode: the queue's head needs more than
 * a reservation; the iteration is then not run).
 */
pa_status pa_sched_step(pa_sched* s, pa_sched_plan* plan);

/* Requests pending, queued or running (0: nothing left to do); -1 for NULL. */
int64_t pa_sched_active(const pa_sched* s);

/*
 * Progress of request rid: state[0] iteration admitted (-1 if never), [1]
 * prompt tokens prefilled, [2] tokens generated, [3] iteration of its last
 * token (-1), [4] iteration it was released (-1), [5] times preempted.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (unknown rid).
 */
pa_status pa_sched_request(const pa_sched* s, int64_t rid, int64_t* state);

#ifdef __cplusplus
}
#endif

#endif /* PA_SCHEDULER_H */
