/*
 * pa_sched.h - page-budget admission and lazy page assignment for the paged KV
 * cache (host C++, no GPU calls).
 *
 * ([README] "6 Hours of YouTube and 85 handtyped pages of notes on LLM
 * Inference - Start here", paragraphs on admission, FIFO waiting and --stats;
 * news-factory.app article, section "How does the engine manage KV cache
 * memory?"; roxreport.com article, paragraph on admission credits.)
 *
 * The policy:
 *   - a request reserves credits for its longest processed prefix,
 *     prompt_tokens + allowed_new - 1 tokens with allowed_new =
 *     min(max_new_tokens, context - prompt_tokens), rounded up to 16-token
 *     pages in each layer;
 *   - credits are separate from physical pages: a page is assigned to a
 *     (request, layer, block) only when a position first needs it, lowest free
 *     page id first;
 *   - waiting requests are admitted in strict first-in, first-out order when
 *     their credits fit beside the active requests' (static mode: only when no
 *     request is active); a budget above the whole pool is rejected;
 *   - finishing, also early, returns the request's pages and credits.
 * Because every active request holds credits for all the pages it can reach,
 * growth within the budget never fails: the pool cannot be exhausted or
 * deadlocked by page-boundary growth.
 *
 * The page ids are those of the shared pool that pa_fill, pa_append and
 * pa_decode address through the block tables; this object only computes
 * them (the caller copies pa_sched_block_table rows into the device tables).
 * A pa_sched object is not thread-safe; distinct objects are independent.
 */
#ifndef PA_SCHED_H_
#define PA_SCHED_H_

#include <stdint.h>

#include "pa.h" /* status codes */

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_sched pa_sched;

typedef struct {
  int64_t pool_pages;           /* physical pages in the pool */
  int64_t free_pages;           /* pages not assigned now */
  int64_t assigned_pages;
  int64_t peak_assigned_pages;
  int64_t credits_free;         /* pages of credit not reserved by active requests */
  int32_t active;               /* admitted, not finished */
  int32_t waiting;
  int32_t peak_active;
  int32_t largest_decode_batch; /* largest value passed to pa_sched_decode_batch */
  int64_t admission_waits;      /* requests not admitted by the first pass after submission */
  int64_t rejected;
  int64_t completed;
} pa_sched_stats;

/* Credits in pages (all layers) for a request; PA_ERR_SHAPE unless
 * 1 <= prompt_tokens < context_tokens, max_new_tokens >= 1, n_layers >= 1. */
int pa_sched_budget_pages(int32_t prompt_tokens, int32_t max_new_tokens, int32_t context_tokens,
                          int32_t n_layers, int64_t* pages);

/* A scheduler over pool_pages physical pages (ids 0..pool_pages-1) for
 * n_layers layers and a context of context_tokens (a multiple of 16, at most
 * 16 * PA_MAX_BLOCKS_LIMIT); static_batching != 0 selects static mode.
 * *out receives the object (NULL on error).  PA_OK, PA_ERR_NULL or PA_ERR_SHAPE. */
int pa_sched_create(int64_t pool_pages, int32_t n_layers, int32_t context_tokens, int32_t static_batching,
                    pa_sched** out);
void pa_sched_destroy(pa_sched* s);

/* Queue a request.  PA_OK with its id in *request_id (ids count up from 0),
 * PA_ERR_REJECTED when its credits exceed the whole pool (nothing is queued),
 * PA_ERR_SHAPE for sizes outside pa_sched_budget_pages' range. */
int pa_sched_submit(pa_sched* s, int32_t prompt_tokens, int32_t max_new_tokens, int64_t* request_id);

/* Admit waiting requests by the mode's rule, at most `capacity` of them, and
 * write their ids in admission order to ids[0 .. *n_admitted-1]. */
int pa_sched_admit(pa_sched* s, int64_t* ids, int32_t capacity, int32_t* n_admitted);

/* Make positions 0..new_length-1 of an active request backed by pages in
 * every layer (assigning pages for blocks it reaches the first time).
 * PA_OK; PA_ERR_BUDGET when new_length exceeds the request's longest
 * processed prefix (nothing assigned); PA_ERR_STATE for an id that is not
 * active. */
int pa_sched_grow(pa_sched* s, int64_t request_id, int32_t new_length);

/* Copy block-table row `layer` of an active request into row[0..max_blocks-1]:
 * assigned page ids, then -1.  PA_ERR_SHAPE when max_blocks is smaller than
 * the request's assigned blocks; PA_ERR_STATE for an id that is not active. */
int pa_sched_block_table(const pa_sched* s, int64_t request_id, int32_t layer, int32_t* row, int32_t max_blocks);

/* Finish an active request (at any length): its pages return to the pool and
 * its credits to the free credits.  PA_ERR_STATE for an id that is not active. */
int pa_sched_finish(pa_sched* s, int64_t request_id);

/* Record the size of a decode batch (for the largest-batch statistic). */
int pa_sched_decode_batch(pa_sched* s, int32_t n);

int pa_sched_get_stats(const pa_sched* s, pa_sched_stats* out);

#ifdef __cplusplus
}
#endif

#endif /* PA_SCHED_H_ */
