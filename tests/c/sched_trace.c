/*
 * Random traces through the admission scheduler's C ABI (include/pa_sched.h),
 * for a host build with AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * Each trace creates a scheduler with a random pool, layer count, context and
 * mode, then applies random submit / admit / grow / block_table / finish /
 * decode_batch calls, and after every call checks what the header promises:
 *   - assigned + free pages = pool, and credits never go negative;
 *   - every active request's block-table rows hold ceil(length / 16) distinct
 *     page ids in [0, pool) followed by -1, and no page id appears in two rows
 *     (two layers or two requests);
 *   - growth up to the request's longest processed prefix never fails, and one
 *     token beyond it returns PA_ERR_BUDGET;
 *   - calls on requests that are not active return PA_ERR_STATE.
 * Exit status 0 when every check held; the first failure is printed.
 * Usage: sched_trace [traces] [steps] [seed]
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pa_sched.h"

#define MAX_REQ 256
#define MAX_LAYERS 4
#define MAX_BLOCKS 128

static uint64_t rng_state;
static uint32_t rnd(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 2685821657736338717ull) >> 32);
}
static int32_t uniform(int32_t lo, int32_t hi) { return lo + (int32_t)(rnd() % (uint32_t)(hi - lo + 1)); }

#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      fprintf(stderr, "trace %d step %d: ", trace, step); \
      fprintf(stderr, __VA_ARGS__);                        \
      fprintf(stderr, "\n");                               \
      return 1;                                            \
    }                                                      \
  } while (0)

typedef struct {
  int64_t id;
  int32_t prompt, max_new, length, limit; /* limit: longest processed prefix */
  int active;
} Req;

static int32_t longest_prefix(int32_t prompt, int32_t max_new, int32_t context) {
  const int32_t allowed = max_new < context - prompt ? max_new : context - prompt;
  return prompt + allowed - 1;
}

static int run_trace(int trace, int steps) {
  int step = -1;
  const int32_t layers = uniform(1, MAX_LAYERS);
  const int32_t context = 16 * uniform(2, MAX_BLOCKS);
  const int64_t pool = uniform(1, 400);
  const int32_t is_static = uniform(0, 1);
  pa_sched* s = NULL;
  CHECK(pa_sched_create(pool, layers, context, is_static, &s) == PA_OK && s, "create");
  static Req req[MAX_REQ];
  int nreq = 0;
  static unsigned char owner[1 << 12];
  for (step = 0; step < steps; ++step) {
    const int op = uniform(0, 9);
    if (op <= 1 && nreq < MAX_REQ) { /* submit */
      const int32_t prompt = uniform(1, context - 1);
      const int32_t max_new = uniform(1, 3 * MAX_BLOCKS);
      int64_t id = -1;
      const int st = pa_sched_submit(s, prompt, max_new, &id);
      int64_t budget = 0;
      CHECK(pa_sched_budget_pages(prompt, max_new, context, layers, &budget) == PA_OK, "budget");
      if (budget > pool) {
        CHECK(st == PA_ERR_REJECTED, "over-pool request not rejected (%d)", st);
      } else {
        CHECK(st == PA_OK && id == nreq, "submit returned %d, id %lld", st, (long long)id);
        req[nreq].id = id;
        req[nreq].prompt = prompt;
        req[nreq].max_new = max_new;
        req[nreq].length = 0;
        req[nreq].limit = longest_prefix(prompt, max_new, context);
        req[nreq].active = 0;
        ++nreq;
      }
    } else if (op == 2) { /* admit */
      int64_t ids[MAX_REQ];
      int32_t n = -1;
      const int32_t cap = uniform(0, 8);
      CHECK(pa_sched_admit(s, ids, cap, &n) == PA_OK && n >= 0 && n <= cap, "admit");
      for (int i = 0; i < n; ++i) {
        CHECK(ids[i] >= 0 && ids[i] < nreq && !req[ids[i]].active, "admitted id %lld", (long long)ids[i]);
        req[ids[i]].active = 1;
      }
    } else if (op <= 6) { /* grow an active request, to its prompt or by one token */
      const int r = uniform(0, nreq > 0 ? nreq - 1 : 0);
      if (nreq == 0) continue;
      Req* q = &req[r];
      const int32_t target = q->length == 0 ? q->prompt : q->length + uniform(1, 3);
      const int st = pa_sched_grow(s, q->id, target);
      if (!q->active) {
        CHECK(st == PA_ERR_STATE, "grow on an inactive request returned %d", st);
      } else if (target > q->limit) {
        CHECK(st == PA_ERR_BUDGET, "growth past the budget returned %d", st);
      } else {
        CHECK(st == PA_OK, "growth within the budget failed (%d): length %d of %d", st, target, q->limit);
        if (target > q->length) q->length = target;
      }
    } else if (op == 7) { /* finish */
      if (nreq == 0) continue;
      Req* q = &req[uniform(0, nreq - 1)];
      const int st = pa_sched_finish(s, q->id);
      CHECK(st == (q->active ? PA_OK : PA_ERR_STATE), "finish returned %d", st);
      q->active = 0;
      q->length = -1; /* finished for good */
    } else if (op == 8) {
      CHECK(pa_sched_decode_batch(s, uniform(0, 64)) == PA_OK, "decode_batch");
    } else { /* a call on an unknown id */
      CHECK(pa_sched_grow(s, nreq + 7, 1) == PA_ERR_STATE, "grow on an unknown id");
      int32_t row[1];
      CHECK(pa_sched_block_table(s, -3, 0, row, 1) == PA_ERR_STATE, "table of an unknown id");
    }

    /* invariants */
    pa_sched_stats st;
    CHECK(pa_sched_get_stats(s, &st) == PA_OK, "stats");
    CHECK(st.pool_pages == pool && st.free_pages + st.assigned_pages == pool && st.free_pages >= 0,
          "page accounting: pool %lld free %lld assigned %lld", (long long)pool, (long long)st.free_pages,
          (long long)st.assigned_pages);
    CHECK(st.credits_free >= 0 && st.credits_free <= pool, "credits %lld", (long long)st.credits_free);
    memset(owner, 0, sizeof owner);
    int64_t seen = 0;
    int active = 0;
    for (int r = 0; r < nreq; ++r) {
      if (!req[r].active) continue;
      ++active;
      const int32_t nb = req[r].length > 0 ? (req[r].length + 15) / 16 : 0;
      for (int32_t l = 0; l < layers; ++l) {
        int32_t row[MAX_BLOCKS + 1];
        CHECK(pa_sched_block_table(s, req[r].id, l, row, MAX_BLOCKS + 1) == PA_OK, "block table");
        for (int32_t j = 0; j <= MAX_BLOCKS; ++j) {
          if (j < nb) {
            CHECK(row[j] >= 0 && row[j] < pool, "request %d layer %d block %d: page %d", r, l, j, row[j]);
            CHECK(!owner[row[j]], "page %d owned twice", row[j]);
            owner[row[j]] = 1;
            ++seen;
          } else {
            CHECK(row[j] == -1, "request %d layer %d entry %d past its blocks holds %d", r, l, j, row[j]);
          }
        }
        if (nb > 0) {
          int32_t small[1];
          CHECK(nb <= 1 || pa_sched_block_table(s, req[r].id, l, small, 1) == PA_ERR_SHAPE, "short row");
        }
      }
    }
    CHECK(seen == st.assigned_pages, "rows hold %lld pages, stats say %lld", (long long)seen,
          (long long)st.assigned_pages);
    CHECK(st.active == active, "stats active %d, trace %d", st.active, active);
  }
  pa_sched_destroy(s);
  return 0;
}

int main(int argc, char** argv) {
  const int traces = argc > 1 ? atoi(argv[1]) : 200;
  const int steps = argc > 2 ? atoi(argv[2]) : 400;
  rng_state = argc > 3 ? strtoull(argv[3], NULL, 10) : 205;
  if (rng_state == 0) rng_state = 1;
  for (int t = 0; t < traces; ++t)
    if (run_trace(t, steps)) return 1;
  printf("%d traces of %d steps: all checks held\n", traces, steps);
  return 0;
}
