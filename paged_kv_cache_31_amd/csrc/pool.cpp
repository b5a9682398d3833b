// Host-side block pool of the paged cache: reference counts, a free list, and the slot
// bookkeeping of a growing sequence with copy-on-write (kasblo.com vLLM explainer, sections
// "blockはrequestの成長に合わせて割り当てる" and "block共有とAutomatic Prefix Caching").
//
// A physical block is free when its count is 0.  Allocation takes blocks from a LIFO free list
// (the most recently freed block is reused first; its lines are the likeliest to still be in
// the last-level cache).  Every operation validates all of its arguments before it changes
// anything, so a refused call leaves the pool as it was.  One mutex per pool makes calls from
// several host threads safe.
#include <stdint.h>

#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

#define PA_EXPORT extern "C" __attribute__((visibility("default")))

struct pa_block_pool {
  std::vector<int32_t> ref;    // per block: sequences referring to it
  std::vector<int32_t> free;   // stack of free blocks
  std::mutex mu;
};

namespace {

constexpr int kBlockTokens = 16;

bool in_pool(const pa_block_pool* p, int32_t b) { return b >= 0 && b < (int32_t)p->ref.size(); }

int32_t pop_free(pa_block_pool* p) {
  const int32_t b = p->free.back();
  p->free.pop_back();
  p->ref[b] = 1;
  return b;
}

}  // namespace

PA_EXPORT pa_status pa_pool_create(int32_t num_blocks, pa_block_pool** pool) {
  if (!pool) return PA_ERR_INVALID_ARG;
  *pool = nullptr;
  if (num_blocks <= 0) return PA_ERR_INVALID_ARG;
  pa_block_pool* p = new (std::nothrow) pa_block_pool;
  if (!p) return PA_ERR_INVALID_ARG;
  p->ref.assign(num_blocks, 0);
  p->free.resize(num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) p->free[i] = num_blocks - 1 - i;   // pops 0, 1, ...
  *pool = p;
  return PA_OK;
}

PA_EXPORT pa_status pa_pool_destroy(pa_block_pool* pool) {
  delete pool;
  return PA_OK;
}

PA_EXPORT int32_t pa_pool_free_blocks(pa_block_pool* pool) {
  if (!pool) return -1;
  std::lock_guard<std::mutex> lock(pool->mu);
  return (int32_t)pool->free.size();
}

PA_EXPORT int32_t pa_pool_refcount(pa_block_pool* pool, int32_t block) {
  if (!pool) return -1;
  std::lock_guard<std::mutex> lock(pool->mu);
  return in_pool(pool, block) ? pool->ref[block] : -1;
}

PA_EXPORT pa_status pa_pool_alloc(pa_block_pool* pool, int32_t n, int32_t* blocks) {
  if (!pool || n < 0 || (n > 0 && !blocks)) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(pool->mu);
  if ((size_t)n > pool->free.size()) return PA_ERR_OUT_OF_BLOCKS;
  for (int32_t i = 0; i < n; ++i) blocks[i] = pop_free(pool);
  return PA_OK;
}

PA_EXPORT pa_status pa_pool_share(pa_block_pool* pool, int32_t n, const int32_t* blocks) {
  if (!pool || n < 0 || (n > 0 && !blocks)) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(pool->mu);
  for (int32_t i = 0; i < n; ++i)
    if (!in_pool(pool, blocks[i]) || pool->ref[blocks[i]] < 1) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) ++pool->ref[blocks[i]];
  return PA_OK;
}

PA_EXPORT pa_status pa_pool_release(pa_block_pool* pool, int32_t n, const int32_t* blocks) {
  if (!pool || n < 0 || (n > 0 && !blocks)) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(pool->mu);
  std::unordered_map<int32_t, int32_t> times;
  for (int32_t i = 0; i < n; ++i) {
    if (!in_pool(pool, blocks[i])) return PA_ERR_INVALID_ARG;
    if (++times[blocks[i]] > pool->ref[blocks[i]]) return PA_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i)
    if (--pool->ref[blocks[i]] == 0) pool->free.push_back(blocks[i]);
  return PA_OK;
}

PA_EXPORT pa_status pa_pool_write(pa_block_pool* pool, int32_t block, int32_t* target,
                                  int32_t* needs_copy) {
  if (!pool || !target || !needs_copy) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(pool->mu);
  if (!in_pool(pool, block) || pool->ref[block] < 1) return PA_ERR_INVALID_ARG;
  if (pool->ref[block] == 1) {
    *target = block;
    *needs_copy = 0;
    return PA_OK;
  }
  if (pool->free.empty()) return PA_ERR_OUT_OF_BLOCKS;
  --pool->ref[block];
  *target = pop_free(pool);
  *needs_copy = 1;
  return PA_OK;
}

PA_EXPORT pa_status pa_pool_slot_for(pa_block_pool* pool, int32_t* table, int32_t* num_blocks,
                                     int32_t max_blocks, int32_t pos, int64_t* slot,
                                     int32_t* copy_src, int32_t* copy_dst) {
  if (!pool || !table || !num_blocks || !slot || !copy_src || !copy_dst) return PA_ERR_INVALID_ARG;
  const int32_t nb = *num_blocks;
  if (pos < 0 || nb < 0 || nb > max_blocks) return PA_ERR_INVALID_ARG;
  const int32_t j = pos / kBlockTokens;
  if (j > nb || j >= max_blocks) return PA_ERR_INVALID_ARG;   // tokens are written in order
  std::lock_guard<std::mutex> lock(pool->mu);
  for (int32_t i = 0; i < nb; ++i)
    if (!in_pool(pool, table[i]) || pool->ref[table[i]] < 1) return PA_ERR_INVALID_ARG;
  *copy_src = *copy_dst = -1;
  if (j == nb) {                                              // the token opens a new block
    if (pool->free.empty()) return PA_ERR_OUT_OF_BLOCKS;
    table[nb] = pop_free(pool);
    *num_blocks = nb + 1;
  } else if (pool->ref[table[j]] > 1) {                       // shared: write into a copy
    if (pool->free.empty()) return PA_ERR_OUT_OF_BLOCKS;
    --pool->ref[table[j]];
    *copy_src = table[j];
    table[j] = pop_free(pool);
    *copy_dst = table[j];
  }
  *slot = (int64_t)table[j] * kBlockTokens + pos % kBlockTokens;
  return PA_OK;
}
