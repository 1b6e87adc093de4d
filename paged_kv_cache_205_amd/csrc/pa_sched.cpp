// Page-budget admission and lazy page assignment (host C++; declarations and
// the policy in include/pa_sched.h).
//
// Sources: [README] "6 Hours of YouTube and 85 handtyped pages of notes on LLM
// Inference - Start here", admission / FIFO / --stats paragraphs;
// news-factory.app article, "How does the engine manage KV cache memory?";
// roxreport.com article, admission-credit paragraph.

#include "pa_sched.h"

#include <deque>
#include <functional>
#include <new>
#include <queue>
#include <unordered_map>
#include <vector>

namespace {

constexpr int32_t kPageTokens = 16;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool valid_request(int32_t prompt, int32_t max_new, int32_t context, int32_t layers) {
  return prompt >= 1 && prompt < context && max_new >= 1 && layers >= 1;
}

// Longest processed prefix: the prompt plus the allowed output, less the last
// predicted token, which is returned without being processed.
int32_t longest_prefix(int32_t prompt, int32_t max_new, int32_t context) {
  const int32_t allowed_new = max_new < context - prompt ? max_new : context - prompt;
  return prompt + allowed_new - 1;
}

struct Request {
  int64_t credits = 0;  // pages, all layers
  int32_t limit = 0;    // longest processed prefix, tokens
  int32_t blocks = 0;   // blocks backed by pages in every layer
  bool active = false;
  bool waited = false;
  std::vector<int32_t> pages;  // [layer][block], blocks <= limit / 16 + 1 per layer
};

}  // namespace

struct pa_sched {
  int64_t pool = 0;
  int32_t layers = 0;
  int32_t context = 0;
  int32_t max_blocks = 0;
  bool is_static = false;
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free;  // lowest id first
  int64_t credits_free = 0;
  std::deque<int64_t> waiting;
  std::unordered_map<int64_t, Request> reqs;  // waiting and active
  int32_t active = 0;
  int64_t next_id = 0;
  int64_t peak_assigned = 0;
  int32_t peak_active = 0;
  int32_t largest_batch = 0;
  int64_t admission_waits = 0, rejected = 0, completed = 0;
};

extern "C" {

int pa_sched_budget_pages(int32_t prompt_tokens, int32_t max_new_tokens, int32_t context_tokens,
                          int32_t n_layers, int64_t* pages) {
  if (!pages) return PA_ERR_NULL;
  if (!valid_request(prompt_tokens, max_new_tokens, context_tokens, n_layers)) return PA_ERR_SHAPE;
  *pages = ceil_div(longest_prefix(prompt_tokens, max_new_tokens, context_tokens), kPageTokens) * n_layers;
  return PA_OK;
}

int pa_sched_create(int64_t pool_pages, int32_t n_layers, int32_t context_tokens, int32_t static_batching,
                    pa_sched** out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (pool_pages <= 0 || pool_pages > INT32_MAX || n_layers <= 0 || context_tokens <= kPageTokens ||
      context_tokens % kPageTokens != 0 || context_tokens / kPageTokens > PA_MAX_BLOCKS_LIMIT)
    return PA_ERR_SHAPE;
  pa_sched* s = new (std::nothrow) pa_sched;
  if (!s) return PA_ERR_NULL;
  s->pool = pool_pages;
  s->layers = n_layers;
  s->context = context_tokens;
  s->max_blocks = context_tokens / kPageTokens;
  s->is_static = static_batching != 0;
  std::vector<int32_t> ids((size_t)pool_pages);
  for (int64_t i = 0; i < pool_pages; ++i) ids[(size_t)i] = (int32_t)i;
  s->free = decltype(s->free)(std::greater<int32_t>(), std::move(ids));
  s->credits_free = pool_pages;
  *out = s;
  return PA_OK;
}

void pa_sched_destroy(pa_sched* s) { delete s; }

int pa_sched_submit(pa_sched* s, int32_t prompt_tokens, int32_t max_new_tokens, int64_t* request_id) {
  if (!s || !request_id) return PA_ERR_NULL;
  int64_t credits = 0;
  const int st = pa_sched_budget_pages(prompt_tokens, max_new_tokens, s->context, s->layers, &credits);
  if (st != PA_OK) return st;
  if (credits > s->pool) {
    ++s->rejected;
    return PA_ERR_REJECTED;
  }
  Request r;
  r.credits = credits;
  r.limit = longest_prefix(prompt_tokens, max_new_tokens, s->context);
  const int64_t id = s->next_id++;
  s->reqs.emplace(id, std::move(r));
  s->waiting.push_back(id);
  *request_id = id;
  return PA_OK;
}

int pa_sched_admit(pa_sched* s, int64_t* ids, int32_t capacity, int32_t* n_admitted) {
  if (!s || !n_admitted || (capacity > 0 && !ids)) return PA_ERR_NULL;
  if (capacity < 0) return PA_ERR_SHAPE;
  int32_t n = 0;
  if (!(s->is_static && s->active > 0)) {
    while (n < capacity && !s->waiting.empty()) {
      Request& r = s->reqs.at(s->waiting.front());
      if (r.credits > s->credits_free) break;  // strict FIFO: nobody passes the oldest
      s->credits_free -= r.credits;
      r.active = true;
      r.pages.assign((size_t)s->layers * (size_t)(r.limit / kPageTokens + 1), -1);
      ids[n++] = s->waiting.front();
      s->waiting.pop_front();
      ++s->active;
    }
  }
  for (int64_t id : s->waiting) {
    Request& r = s->reqs.at(id);
    if (!r.waited) {
      r.waited = true;
      ++s->admission_waits;
    }
  }
  if (s->active > s->peak_active) s->peak_active = s->active;
  *n_admitted = n;
  return PA_OK;
}

int pa_sched_grow(pa_sched* s, int64_t request_id, int32_t new_length) {
  if (!s) return PA_ERR_NULL;
  auto it = s->reqs.find(request_id);
  if (it == s->reqs.end() || !it->second.active) return PA_ERR_STATE;
  Request& r = it->second;
  if (new_length < 0 || new_length > r.limit) return PA_ERR_BUDGET;
  const int32_t need = (int32_t)ceil_div(new_length, kPageTokens);
  const size_t row = (size_t)(r.limit / kPageTokens + 1);
  // The credits cover every block up to the limit, so the free list cannot run
  // dry here; checked all the same, before anything is assigned.
  if (need > r.blocks && (int64_t)s->free.size() < (int64_t)(need - r.blocks) * s->layers) return PA_ERR_STATE;
  for (int32_t l = 0; l < s->layers; ++l)
    for (int32_t blk = r.blocks; blk < need; ++blk) {
      r.pages[(size_t)l * row + (size_t)blk] = s->free.top();
      s->free.pop();
    }
  if (need > r.blocks) r.blocks = need;
  const int64_t assigned = s->pool - (int64_t)s->free.size();
  if (assigned > s->peak_assigned) s->peak_assigned = assigned;
  return PA_OK;
}

int pa_sched_block_table(const pa_sched* s, int64_t request_id, int32_t layer, int32_t* row, int32_t max_blocks) {
  if (!s || !row) return PA_ERR_NULL;
  auto it = s->reqs.find(request_id);
  if (it == s->reqs.end() || !it->second.active) return PA_ERR_STATE;
  const Request& r = it->second;
  if (layer < 0 || layer >= s->layers || max_blocks < r.blocks) return PA_ERR_SHAPE;
  const size_t stride = (size_t)(r.limit / kPageTokens + 1);
  for (int32_t b = 0; b < max_blocks; ++b)
    row[b] = b < r.blocks ? r.pages[(size_t)layer * stride + (size_t)b] : -1;
  return PA_OK;
}

int pa_sched_finish(pa_sched* s, int64_t request_id) {
  if (!s) return PA_ERR_NULL;
  auto it = s->reqs.find(request_id);
  if (it == s->reqs.end() || !it->second.active) return PA_ERR_STATE;
  Request& r = it->second;
  const size_t stride = (size_t)(r.limit / kPageTokens + 1);
  for (int32_t l = 0; l < s->layers; ++l)
    for (int32_t b = 0; b < r.blocks; ++b) s->free.push(r.pages[(size_t)l * stride + (size_t)b]);
  s->credits_free += r.credits;
  --s->active;
  ++s->completed;
  s->reqs.erase(it);
  return PA_OK;
}

int pa_sched_decode_batch(pa_sched* s, int32_t n) {
  if (!s) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (n > s->largest_batch) s->largest_batch = n;
  return PA_OK;
}

int pa_sched_get_stats(const pa_sched* s, pa_sched_stats* out) {
  if (!s || !out) return PA_ERR_NULL;
  out->pool_pages = s->pool;
  out->free_pages = (int64_t)s->free.size();
  out->assigned_pages = s->pool - (int64_t)s->free.size();
  out->peak_assigned_pages = s->peak_assigned;
  out->credits_free = s->credits_free;
  out->active = s->active;
  out->waiting = (int32_t)s->waiting.size();
  out->peak_active = s->peak_active;
  out->largest_decode_batch = s->largest_batch;
  out->admission_waits = s->admission_waits;
  out->rejected = s->rejected;
  out->completed = s->completed;
  return PA_OK;
}

}  // extern "C"
