// Paged block pool: host-side bookkeeping of fixed-size KV blocks.
//
// Follows the PagedAttention manager of the "KV Cache optimization techniques"
// tutorial, section 3.2: a pool of equal blocks, a block list per sequence, a
// reference count per block and a set of free blocks. Allocation is all or
// nothing, freeing an unknown sequence is a no-op, and asking for the blocks
// of an unknown sequence is an error. Unlike the tutorial, the number of
// tokens a sequence holds is not derived from its block count: the device
// tracks lengths, and the pool only answers how many blocks a length needs.
//
// The free list starts as a seeded Fisher-Yates shuffle of the block ids
// (splitmix64 generator), so blocks land at a seeded random permutation of
// the pool, the placement a long-running server ends up with.
#include <stdarg.h>
#include <stdint.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "kvc.h"

namespace kvc {
int32_t fail(int32_t status, const char* fmt, ...);
void clear_error();
}  // namespace kvc

struct kvc_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_list;  // back = next block handed out
  std::vector<int32_t> refcount;
  std::unordered_map<int32_t, std::vector<int32_t>> seqs;
};

namespace {

uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace

extern "C" {

kvc_pool_t* kvc_pool_create(int32_t num_blocks, int32_t block_size, uint64_t shuffle_seed) {
  kvc::clear_error();
  if (num_blocks < 1 || block_size < 1) {
    kvc::fail(KVC_ERR_INVALID_ARG, "num_blocks and block_size must be >= 1");
    return nullptr;
  }
  kvc_pool* p = new (std::nothrow) kvc_pool;
  if (!p) return nullptr;
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  std::vector<int32_t> order(num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) order[i] = i;
  if (shuffle_seed) {
    uint64_t s = shuffle_seed;
    for (int32_t i = num_blocks - 1; i > 0; --i) {
      const int32_t j = (int32_t)(splitmix64(s) % (uint64_t)(i + 1));
      const int32_t t = order[i];
      order[i] = order[j];
      order[j] = t;
    }
  }
  // Hand blocks out in `order`: the back of the free list is order[0].
  p->free_list.assign(order.rbegin(), order.rend());
  p->refcount.assign(num_blocks, 0);
  return p;
}

void kvc_pool_destroy(kvc_pool_t* pool) { delete pool; }

int32_t kvc_pool_reserve(kvc_pool_t* pool, int32_t seq_id, int32_t num_tokens) {
  kvc::clear_error();
  if (!pool) return kvc::fail(KVC_ERR_INVALID_ARG, "pool is NULL");
  if (seq_id < 0 || num_tokens < 0) return kvc::fail(KVC_ERR_INVALID_ARG, "seq_id and num_tokens must be >= 0");
  const int64_t need_total = ((int64_t)num_tokens + pool->block_size - 1) / pool->block_size;
  auto it = pool->seqs.find(seq_id);
  const int64_t have = it == pool->seqs.end() ? 0 : (int64_t)it->second.size();
  const int64_t extra = need_total > have ? need_total - have : 0;
  if (extra > (int64_t)pool->free_list.size())
    return kvc::fail(KVC_ERR_CAPACITY, "sequence %d needs %lld more blocks, %zu free", seq_id, (long long)extra,
                     pool->free_list.size());
  std::vector<int32_t>& blocks = pool->seqs[seq_id];
  for (int64_t i = 0; i < extra; ++i) {
    const int32_t b = pool->free_list.back();
    pool->free_list.pop_back();
    pool->refcount[b] = 1;
    blocks.push_back(b);
  }
  return KVC_OK;
}

int32_t kvc_pool_free(kvc_pool_t* pool, int32_t seq_id) {
  kvc::clear_error();
  if (!pool) return kvc::fail(KVC_ERR_INVALID_ARG, "pool is NULL");
  auto it = pool->seqs.find(seq_id);
  if (it == pool->seqs.end()) return KVC_OK;
  for (int32_t b : it->second) {
    if (--pool->refcount[b] == 0) pool->free_list.push_back(b);
  }
  pool->seqs.erase(it);
  return KVC_OK;
}

int32_t kvc_pool_release(kvc_pool_t* pool, int32_t seq_id, const int32_t* blocks_host, int32_t n) {
  kvc::clear_error();
  if (!pool) return kvc::fail(KVC_ERR_INVALID_ARG, "pool is NULL");
  if (n < 0 || (n > 0 && !blocks_host)) return kvc::fail(KVC_ERR_INVALID_ARG, "bad block list");
  auto it = pool->seqs.find(seq_id);
  if (it == pool->seqs.end()) return kvc::fail(KVC_ERR_INVALID_ARG, "unknown sequence %d", seq_id);
  std::vector<int32_t>& blocks = it->second;
  // All or nothing: every listed block must be one of the sequence's, once.
  std::vector<char> drop(blocks.size(), 0);
  for (int32_t i = 0; i < n; ++i) {
    size_t k = 0;
    while (k < blocks.size() && (blocks[k] != blocks_host[i] || drop[k])) ++k;
    if (k == blocks.size())
      return kvc::fail(KVC_ERR_INVALID_ARG, "block %d is not held by sequence %d", blocks_host[i], seq_id);
    drop[k] = 1;
  }
  std::vector<int32_t> kept;
  kept.reserve(blocks.size() - (size_t)n);
  for (size_t k = 0; k < blocks.size(); ++k) {
    if (!drop[k]) {
      kept.push_back(blocks[k]);
    } else if (--pool->refcount[blocks[k]] == 0) {
      pool->free_list.push_back(blocks[k]);
    }
  }
  blocks.swap(kept);
  return KVC_OK;
}

int32_t kvc_pool_num_free(const kvc_pool_t* pool) { return pool ? (int32_t)pool->free_list.size() : -1; }

int32_t kvc_pool_num_blocks(const kvc_pool_t* pool, int32_t seq_id) {
  if (!pool) return -1;
  auto it = pool->seqs.find(seq_id);
  return it == pool->seqs.end() ? -1 : (int32_t)it->second.size();
}

int32_t kvc_pool_block_table(const kvc_pool_t* pool, const int32_t* seq_ids_host, int32_t batch, int32_t max_blocks,
                             int32_t* table_host) {
  kvc::clear_error();
  if (!pool || !seq_ids_host || !table_host) return kvc::fail(KVC_ERR_INVALID_ARG, "NULL argument");
  if (batch < 1 || max_blocks < 1) return kvc::fail(KVC_ERR_INVALID_ARG, "batch and max_blocks must be >= 1");
  for (int32_t b = 0; b < batch; ++b) {
    auto it = pool->seqs.find(seq_ids_host[b]);
    if (it == pool->seqs.end()) return kvc::fail(KVC_ERR_INVALID_ARG, "unknown sequence %d", seq_ids_host[b]);
    if ((int64_t)it->second.size() > max_blocks)
      return kvc::fail(KVC_ERR_CAPACITY, "sequence %d holds %zu blocks > max_blocks %d", seq_ids_host[b],
                       it->second.size(), max_blocks);
  }
  for (int32_t b = 0; b < batch; ++b) {
    const std::vector<int32_t>& blocks = pool->seqs.find(seq_ids_host[b])->second;
    int32_t* row = table_host + (int64_t)b * max_blocks;
    for (int32_t i = 0; i < max_blocks; ++i) row[i] = i < (int32_t)blocks.size() ? blocks[i] : -1;
  }
  return KVC_OK;
}

}  // extern "C"
