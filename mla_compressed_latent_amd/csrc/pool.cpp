// A stack of MLA layers on one GPU: capacity planning and the page pool that
// every layer's paged cache shares (host code; the C ABI is in include/mla.h).
//
// "Multi-head Latent Attention: the KV cache, compressed" (paperfordummies.in):
// section "The one formula" -- a token costs num_layers x (d_c + d_rope)
// elements of cache, whatever the head count; section "Where the saving
// actually lands" -- the number that matters is how many whole sequences of a
// given context one cache budget holds.
//
// Every layer holds the same tokens of the same sequences, so one page table
// serves all of them: page p of a sequence is page p of each layer's cache.
#include <stdint.h>
#include <string.h>

#include <new>
#include <vector>

#include "../../include/mla.h"

// Sets the thread's error message (api.hip).
namespace mla_api {
mla_status fail_msg(mla_status s, const char* msg);
size_t row_bytes(const mla_config* cfg);   // 0 if cfg is invalid
}

struct mla_page_pool {
  int64_t num_pages;
  int32_t page_size;
  int32_t max_seqs;
  int32_t max_pages_per_seq;
  std::vector<int32_t> free_stack;          // top = next page handed out
  std::vector<std::vector<int32_t>> pages;  // per sequence, in token order
  std::vector<int64_t> length;              // tokens reserved per sequence
};

namespace {

mla_status plan_checks(const mla_config* cfg, int32_t num_layers, size_t* page_bytes) {
  const size_t row = mla_api::row_bytes(cfg);
  if (row == 0) return MLA_ERR_INVALID_ARG;   // message set by the config check
  if (num_layers < 1) return mla_api::fail_msg(MLA_ERR_INVALID_ARG, "num_layers must be >= 1");
  *page_bytes = row * (size_t)cfg->page_size;
  return MLA_OK;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

mla_status mla_plan_cache(const mla_config* cfg, int32_t num_layers, size_t budget_bytes,
                          mla_cache_plan* out) {
  if (!out) return mla_api::fail_msg(MLA_ERR_INVALID_ARG, "mla_plan_cache: out is null");
  size_t page_bytes = 0;
  const mla_status st = plan_checks(cfg, num_layers, &page_bytes);
  if (st != MLA_OK) return st;
  const size_t per_page_all_layers = page_bytes * (size_t)num_layers;
  int64_t pages = (int64_t)(budget_bytes / per_page_all_layers);
  if (pages > INT32_MAX) pages = INT32_MAX;   // page ids are int32
  if (pages < 1)
    return mla_api::fail_msg(MLA_ERR_INSUFFICIENT_WORKSPACE,
                             "mla_plan_cache: the budget holds no page of every layer");
  out->num_layers = num_layers;
  out->page_size = cfg->page_size;
  out->num_pages = pages;
  out->page_bytes = page_bytes;
  out->layer_bytes = page_bytes * (size_t)pages;
  out->total_bytes = out->layer_bytes * (size_t)num_layers;
  out->bytes_per_token = page_bytes / (size_t)cfg->page_size * (size_t)num_layers;
  return MLA_OK;
}

int64_t mla_plan_max_sequences(const mla_config* cfg, int32_t num_layers, size_t budget_bytes,
                               int64_t context) {
  size_t page_bytes = 0;
  if (context < 1 || plan_checks(cfg, num_layers, &page_bytes) != MLA_OK) return -1;
  const uint64_t pages = (uint64_t)((context + cfg->page_size - 1) / cfg->page_size);
  const uint64_t per_seq = pages * (uint64_t)page_bytes * (uint64_t)num_layers;
  return (int64_t)(budget_bytes / per_seq);
}

mla_status mla_pool_create(int64_t num_pages, int32_t page_size, int32_t max_seqs,
                           int32_t max_pages_per_seq, mla_page_pool** out) {
  if (!out) return mla_api::fail_msg(MLA_ERR_INVALID_ARG, "mla_pool_create: out is null");
  if (num_pages < 1 || num_pages > INT32_MAX || page_size < 1 || max_seqs < 1 ||
      max_pages_per_seq < 1)
    return mla_api::fail_msg(MLA_ERR_INVALID_ARG, "mla_pool_create: sizes must be positive "
                                                  "(and num_pages < 2^31)");
  mla_page_pool* p = new (std::nothrow) mla_page_pool;
  if (!p) return mla_api::fail_msg(MLA_ERR_INVALID_ARG, "mla_pool_create: out of host memory");
  p->num_pages = num_pages;
  p->page_size = page_size;
  p->max_seqs = max_seqs;
  p->max_pages_per_seq = max_pages_per_seq;
  try {   // no exception crosses the C boundary
    p->free_stack.resize((size_t)num_pages);
    for (int64_t i = 0; i < num_pages; ++i) p->free_stack[(size_t)i] = (int32_t)(num_pages - 1 - i);
    p->pages.resize((size_t)max_seqs);
    p->length.assign((size_t)max_seqs, 0);
  } catch (const std::bad_alloc&) {
    delete p;
    return mla_api::fail_msg(MLA_ERR_INVALID_ARG, "mla_pool_create: out of host memory");
  }
  *out = p;
  return MLA_OK;
}

void mla_pool_destroy(mla_page_pool* pool) { delete pool; }

mla_status mla_pool_reserve(mla_page_pool* p, int32_t seq, int64_t length) {
  if (!p) return mla_api::fail_msg(MLA_ERR_INVALID_ARG, "pool is null");
  if (seq < 0 || seq >= p->max_seqs)
    return mla_api::fail_msg(MLA_ERR_INVALID_ARG, "mla_pool_reserve: sequence id out of range");
  if (length < 0 || length > (int64_t)p->max_pages_per_seq * p->page_size)
    return mla_api::fail_msg(MLA_ERR_INVALID_ARG,
                             "mla_pool_reserve: length beyond max_pages_per_seq * page_size");
  std::vector<int32_t>& mine = p->pages[(size_t)seq];
  const size_t need = (size_t)((length + p->page_size - 1) / p->page_size);
  if (need > mine.size()) {
    const size_t more = need - mine.size();
    if (more > p->free_stack.size())
      return mla_api::fail_msg(MLA_ERR_INSUFFICIENT_WORKSPACE,
                               "mla_pool_reserve: not enough free pages");
    try {   // grow first, so that a failure leaves the pool unchanged
      mine.reserve(need);
    } catch (const std::bad_alloc&) {
      return mla_api::fail_msg(MLA_ERR_INVALID_ARG, "mla_pool_reserve: out of host memory");
    }
    for (size_t i = 0; i < more; ++i) {
      mine.push_back(p->free_stack.back());
      p->free_stack.pop_back();
    }
  }
  if (length > p->length[(size_t)seq]) p->length[(size_t)seq] = length;
  return MLA_OK;
}

mla_status mla_pool_release(mla_page_pool* p, int32_t seq) {
  if (!p) return mla_api::fail_msg(MLA_ERR_INVALID_ARG, "pool is null");
  if (seq < 0 || seq >= p->max_seqs)
    return mla_api::fail_msg(MLA_ERR_INVALID_ARG, "mla_pool_release: sequence id out of range");
  std::vector<int32_t>& mine = p->pages[(size_t)seq];
  // last page first, so that the next reservation gets them back in order
  // (the stack's capacity is num_pages from creation: no reallocation here)
  for (size_t i = mine.size(); i-- > 0;) p->free_stack.push_back(mine[i]);
  mine.clear();
  p->length[(size_t)seq] = 0;
  return MLA_OK;
}

int64_t mla_pool_free_pages(const mla_page_pool* p) {
  return p ? (int64_t)p->free_stack.size() : -1;
}

int64_t mla_pool_length(const mla_page_pool* p, int32_t seq) {
  if (!p || seq < 0 || seq >= p->max_seqs) return -1;
  return p->length[(size_t)seq];
}

mla_status mla_pool_page_table(const mla_page_pool* p, const int32_t* seqs, int32_t n,
                               int32_t* table) {
  if (!p || !seqs || !table || n < 1)
    return mla_api::fail_msg(MLA_ERR_INVALID_ARG, "mla_pool_page_table: null pointer or n < 1");
  for (int32_t i = 0; i < n; ++i)
    if (seqs[i] < 0 || seqs[i] >= p->max_seqs)
      return mla_api::fail_msg(MLA_ERR_INVALID_ARG, "mla_pool_page_table: sequence id out of range");
  const size_t w = (size_t)p->max_pages_per_seq;
  for (int32_t i = 0; i < n; ++i) {
    const std::vector<int32_t>& mine = p->pages[(size_t)seqs[i]];
    int32_t* row = table + (size_t)i * w;
    for (size_t j = 0; j < w; ++j) row[j] = j < mine.size() ? mine[j] : -1;
  }
  return MLA_OK;
}

}  // extern "C"
#pragma GCC visibility pop
