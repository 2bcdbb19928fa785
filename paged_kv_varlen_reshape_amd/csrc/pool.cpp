// Host block allocator: pa_pool_*.
//
// Allocation procedure of the Inside vLLM summary (techfeed.io), section
// "PagedAttentionの仕組み": a request that will hold T tokens needs
// ceil(T / block_size) blocks; the blocks it lacks are taken from the head of
// the free-block queue and appended to its list in req_to_blocks.  When the
// queue is too short the page's engine preempts a lower-priority request;
// picking that request is scheduler policy, so this allocator reports
// PA_ERR_NO_BLOCKS and changes nothing.  Blocks go back to the pool when
// tokens no longer need them (engr-sng explainer of the same article,
// paragraph on Paging Attention): release drops one reference from each block
// of the request, in list order, and appends blocks that reach zero references
// to the tail of the queue.  Prefix caching (Inside vLLM summary, "高度な機能群")
// shares already cached blocks between requests with one reference each.
//
// Prefix cache index (Inside vLLM summary, "高度な機能群", Prefix Caching: a
// request that starts with the same prompt reuses the cached KV blocks; the
// architecture overview places that index in the block pool).  A full block
// can be registered under a caller-computed 64-bit key (for instance a hash
// of its tokens chained with the key of the block before it); a new request
// takes over the longest run of leading blocks whose keys hit, one reference
// each.  A block whose references drop to zero keeps its contents and its key:
// it waits in the free queue like any free block and stays findable until the
// queue hands it out again, which removes its key (a hit on such a block
// takes it out of the queue).
//
// The free queue is an intrusive doubly-linked list over block ids (sentinel
// num_blocks), so allocation, release and taking a cached block out of the
// queue are O(1) per block.
#include <cstring>
#include <unordered_map>
#include <vector>

#include "errors.h"

struct pa_pool {
  int64_t num_blocks;
  int32_t block_size;
  std::vector<int32_t> next, prev;  // free queue links, [num_blocks + 1]
  int64_t count = 0;                // blocks in the queue
  std::vector<int32_t> refcount;
  std::unordered_map<int64_t, std::vector<int32_t>> req_to_blocks;
  std::unordered_map<uint64_t, int32_t> cache;  // key -> block
  std::vector<uint64_t> block_key;
  std::vector<char> has_key;

  int32_t sentinel() const { return int32_t(num_blocks); }
  void push_back(int32_t b) {
    const int32_t s = sentinel(), t = prev[s];
    next[t] = b;
    prev[b] = t;
    next[b] = s;
    prev[s] = b;
    ++count;
  }
  void unlink(int32_t b) {
    next[prev[b]] = next[b];
    prev[next[b]] = prev[b];
    --count;
  }
  int32_t pop_front() {  // the block leaves the cache index, its contents will be overwritten
    const int32_t b = next[sentinel()];
    unlink(b);
    if (has_key[b]) {
      cache.erase(block_key[b]);
      has_key[b] = 0;
    }
    return b;
  }
};

extern "C" pa_pool* pa_pool_create(int64_t num_blocks, int32_t block_size, const int32_t* initial_order) {
  pa::clear_error();
  if (num_blocks <= 0 || num_blocks > (int64_t(1) << 31) - 1) {
    pa::fail(PA_ERR_INVALID, "pa_pool_create: num_blocks %lld out of range", (long long)num_blocks);
    return nullptr;
  }
  if (block_size <= 0 || num_blocks * int64_t(block_size) > (int64_t(1) << 31) - 1) {
    pa::fail(PA_ERR_INVALID, "pa_pool_create: block_size must be positive and slots must fit in int32");
    return nullptr;
  }
  pa_pool* p = new pa_pool;
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->next.assign(num_blocks + 1, 0);
  p->prev.assign(num_blocks + 1, 0);
  p->next[num_blocks] = p->prev[num_blocks] = int32_t(num_blocks);  // empty queue
  p->refcount.assign(num_blocks, 0);
  p->block_key.assign(num_blocks, 0);
  p->has_key.assign(num_blocks, 0);
  if (initial_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int64_t i = 0; i < num_blocks; ++i) {
      int32_t b = initial_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        pa::fail(PA_ERR_INVALID, "pa_pool_create: initial_order is not a permutation (entry %lld)",
                 (long long)i);
        return nullptr;
      }
      seen[b] = 1;
    }
    for (int64_t i = 0; i < num_blocks; ++i) p->push_back(initial_order[i]);
  } else {
    for (int64_t i = 0; i < num_blocks; ++i) p->push_back(int32_t(i));
  }
  return p;
}

extern "C" void pa_pool_destroy(pa_pool* pool) { delete pool; }

extern "C" int pa_allocate_slots(pa_pool* pool, int64_t req, int64_t num_computed, int64_t num_new,
                                 int32_t* new_ids_out, int32_t cap, int32_t* n_out) {
  pa::clear_error();
  if (n_out) *n_out = 0;
  if (!pool) return pa::fail(PA_ERR_INVALID, "pa_allocate_slots: null pool");
  if (num_computed < 0 || num_new < 0) return pa::fail(PA_ERR_INVALID, "pa_allocate_slots: negative token count");
  const int64_t total = num_computed + num_new;
  const int64_t want = (total + pool->block_size - 1) / pool->block_size;
  auto it = pool->req_to_blocks.find(req);
  const int64_t have = it == pool->req_to_blocks.end() ? 0 : int64_t(it->second.size());
  const int64_t need = want > have ? want - have : 0;
  if (need > pool->count)
    return pa::fail(PA_ERR_NO_BLOCKS, "pa_allocate_slots: request %lld needs %lld blocks, %lld free",
                    (long long)req, (long long)need, (long long)pool->count);
  if (new_ids_out && need > cap)
    return pa::fail(PA_ERR_INVALID, "pa_allocate_slots: output capacity %d < %lld new blocks", cap, (long long)need);
  std::vector<int32_t>& list = pool->req_to_blocks[req];
  for (int64_t i = 0; i < need; ++i) {
    int32_t b = pool->pop_front();
    pool->refcount[b] = 1;
    list.push_back(b);
    if (new_ids_out) new_ids_out[i] = b;
  }
  if (n_out) *n_out = int32_t(need);
  return PA_OK;
}

extern "C" int pa_share_prefix(pa_pool* pool, int64_t req, const int32_t* ids, int32_t n) {
  pa::clear_error();
  if (!pool) return pa::fail(PA_ERR_INVALID, "pa_share_prefix: null pool");
  if (n < 0 || (n > 0 && !ids)) return pa::fail(PA_ERR_INVALID, "pa_share_prefix: bad id list");
  for (int32_t i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= pool->num_blocks || pool->refcount[ids[i]] <= 0)
      return pa::fail(PA_ERR_INVALID, "pa_share_prefix: block %d is not allocated", ids[i]);
  }
  std::vector<int32_t>& list = pool->req_to_blocks[req];
  for (int32_t i = 0; i < n; ++i) {
    pool->refcount[ids[i]] += 1;
    list.push_back(ids[i]);
  }
  return PA_OK;
}

extern "C" int pa_free(pa_pool* pool, int64_t req) {
  pa::clear_error();
  if (!pool) return pa::fail(PA_ERR_INVALID, "pa_free: null pool");
  auto it = pool->req_to_blocks.find(req);
  if (it == pool->req_to_blocks.end()) return PA_OK;
  for (int32_t b : it->second) {
    if (--pool->refcount[b] == 0) pool->push_back(b);
  }
  pool->req_to_blocks.erase(it);
  return PA_OK;
}

extern "C" int pa_prefix_match(pa_pool* pool, int64_t req, const uint64_t* keys, int32_t n, int32_t* n_hit) {
  pa::clear_error();
  if (n_hit) *n_hit = 0;
  if (!pool) return pa::fail(PA_ERR_INVALID, "pa_prefix_match: null pool");
  if (n < 0 || (n > 0 && !keys)) return pa::fail(PA_ERR_INVALID, "pa_prefix_match: bad key list");
  auto it = pool->req_to_blocks.find(req);
  if (it != pool->req_to_blocks.end() && !it->second.empty())
    return pa::fail(PA_ERR_INVALID, "pa_prefix_match: request %lld already holds blocks", (long long)req);
  int32_t hits = 0;
  for (; hits < n; ++hits) {
    auto c = pool->cache.find(keys[hits]);
    if (c == pool->cache.end()) break;
    const int32_t b = c->second;
    if (pool->refcount[b] == 0) pool->unlink(b);  // a released block waiting in the queue
    pool->refcount[b] += 1;
    pool->req_to_blocks[req].push_back(b);
  }
  if (n_hit) *n_hit = hits;
  return PA_OK;
}

extern "C" int pa_prefix_register(pa_pool* pool, int64_t req, const uint64_t* keys, int32_t n) {
  pa::clear_error();
  if (!pool) return pa::fail(PA_ERR_INVALID, "pa_prefix_register: null pool");
  if (n < 0 || (n > 0 && !keys)) return pa::fail(PA_ERR_INVALID, "pa_prefix_register: bad key list");
  auto it = pool->req_to_blocks.find(req);
  const int64_t have = it == pool->req_to_blocks.end() ? 0 : int64_t(it->second.size());
  if (n > have)
    return pa::fail(PA_ERR_INVALID, "pa_prefix_register: request %lld holds %lld blocks < %d", (long long)req,
                    (long long)have, n);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = it->second[i];
    if (pool->has_key[b] && pool->block_key[b] != keys[i])
      return pa::fail(PA_ERR_INVALID, "pa_prefix_register: block %d is cached under another key", b);
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = it->second[i];
    if (pool->has_key[b] || pool->cache.count(keys[i])) continue;  // already there, or an equal block is
    pool->cache.emplace(keys[i], b);
    pool->block_key[b] = keys[i];
    pool->has_key[b] = 1;
  }
  return PA_OK;
}

extern "C" int64_t pa_prefix_cached(const pa_pool* pool) { return pool ? int64_t(pool->cache.size()) : -1; }

extern "C" int64_t pa_num_free(const pa_pool* pool) { return pool ? pool->count : -1; }

extern "C" int32_t pa_num_req_blocks(const pa_pool* pool, int64_t req) {
  if (!pool) return -1;
  auto it = pool->req_to_blocks.find(req);
  return it == pool->req_to_blocks.end() ? 0 : int32_t(it->second.size());
}

extern "C" int32_t pa_refcount(const pa_pool* pool, int32_t block) {
  if (!pool || block < 0 || block >= pool->num_blocks) return -1;
  return pool->refcount[block];
}

extern "C" int pa_block_table_row(const pa_pool* pool, int64_t req, int32_t* out, int32_t width,
                                  int32_t pad_value) {
  pa::clear_error();
  if (!pool || (!out && width > 0) || width < 0) return pa::fail(PA_ERR_INVALID, "pa_block_table_row: bad arguments");
  auto it = pool->req_to_blocks.find(req);
  const int64_t n = it == pool->req_to_blocks.end() ? 0 : int64_t(it->second.size());
  if (n > width)
    return pa::fail(PA_ERR_INVALID, "pa_block_table_row: request %lld holds %lld blocks > width %d",
                    (long long)req, (long long)n, width);
  if (n) std::memcpy(out, it->second.data(), size_t(n) * sizeof(int32_t));
  for (int64_t i = n; i < width; ++i) out[i] = pad_value;
  return PA_OK;
}

extern "C" int pa_slot_mapping(const pa_pool* pool, int64_t req, int64_t start_pos, int32_t n, int32_t* out) {
  pa::clear_error();
  if (!pool || n < 0 || (n > 0 && !out) || start_pos < 0) return pa::fail(PA_ERR_INVALID, "pa_slot_mapping: bad arguments");
  auto it = pool->req_to_blocks.find(req);
  const int64_t have = it == pool->req_to_blocks.end() ? 0 : int64_t(it->second.size());
  const int64_t bs = pool->block_size;
  if (n > 0 && (start_pos + n - 1) / bs >= have)
    return pa::fail(PA_ERR_INVALID, "pa_slot_mapping: position %lld of request %lld has no block",
                    (long long)(start_pos + n - 1), (long long)req);
  for (int32_t j = 0; j < n; ++j) {
    const int64_t pos = start_pos + j;
    out[j] = int32_t(int64_t(it->second[pos / bs]) * bs + pos % bs);
  }
  return PA_OK;
}
