// Host block pool of the paged KV cache: the control plane on either side of
// the attention step.
//
// What it does ("vLLM 推理流程分析" §4.2-4.3, §8.1, §10; "vLLM 源码完全拆解（十六）",
// second walk-through path):
//  - allocate_slots gives a request enough physical blocks for the tokens it
//    will hold after the step; a request that starts with a prefix-cache hit
//    first takes the hit blocks (touch: reference count + 1);
//  - free drops the request's references; a block whose count reaches zero
//    joins the free queue, where its contents stay valid for prefix hits
//    until the block is handed out again (free means "may be overwritten",
//    not "cleared");
//  - full blocks of computed tokens are entered into a map from a chained
//    block hash (parent hash, extra identity, the block's token ids) to the
//    block, and get_computed_blocks looks a token sequence up in it.
//
// Policy (the plainest reading where the pages leave it open): the free queue
// starts in ascending block order and hands out from its head (least recently
// freed first); a freed request returns its blocks last-first, so its later
// blocks, which fewer requests share, are reused before its prefix.  A block
// taken from the queue while it is in the hash map leaves the map.
//
// Hash: FNV-1a 64 (Fowler-Noll-Vo; offset basis 0xcbf29ce484222325, prime
// 0x100000001b3) over the little-endian bytes of the parent block's hash (0
// for the first block), the extra key, and the block's S token ids (int32).
// A lookup also compares the stored key itself, so a hash collision cannot
// produce a false hit.
//
// Every function is host-only and runs in O(blocks touched) time.
#include <stdint.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

namespace pa {

struct BlockKey {
  uint64_t parent = 0;
  uint64_t extra = 0;
  std::vector<int32_t> tokens;
};

}  // namespace pa

struct pa_kv_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ref;                 // reference count per block
  std::vector<int32_t> prev, next;          // free queue (doubly linked, sentinel = num_blocks)
  std::vector<uint8_t> queued;              // block is in the free queue
  int32_t num_queued = 0;
  std::vector<uint8_t> hashed;              // block holds a valid hash entry
  std::vector<uint64_t> hash;
  std::vector<pa::BlockKey> key;
  std::unordered_map<uint64_t, int32_t> cached;   // block hash -> block
  std::unordered_map<int64_t, std::vector<int32_t>> req_blocks;
  std::mutex mu;
};

namespace pa {

static uint64_t fnv1a(uint64_t h, const void *p, size_t n) {
  const uint8_t *b = (const uint8_t *)p;
  for (size_t i = 0; i < n; ++i) {
    h ^= b[i];
    h *= 0x100000001b3ULL;
  }
  return h;
}

static uint64_t block_hash(uint64_t parent, uint64_t extra, const int32_t *tokens, int32_t S) {
  uint64_t h = 0xcbf29ce484222325ULL;
  uint8_t buf[8];
  for (int i = 0; i < 8; ++i) buf[i] = (uint8_t)(parent >> (8 * i));
  h = fnv1a(h, buf, 8);
  for (int i = 0; i < 8; ++i) buf[i] = (uint8_t)(extra >> (8 * i));
  h = fnv1a(h, buf, 8);
  for (int32_t t = 0; t < S; ++t) {
    const uint32_t v = (uint32_t)tokens[t];
    for (int i = 0; i < 4; ++i) buf[i] = (uint8_t)(v >> (8 * i));
    h = fnv1a(h, buf, 4);
  }
  return h;
}

static void queue_remove(pa_kv_manager &m, int32_t b) {
  const int32_t p = m.prev[b], n = m.next[b];
  m.next[p] = n;
  m.prev[n] = p;
  m.queued[b] = 0;
  --m.num_queued;
}

static void queue_push_back(pa_kv_manager &m, int32_t b) {
  const int32_t s = m.num_blocks, last = m.prev[s];
  m.next[last] = b;
  m.prev[b] = last;
  m.next[b] = s;
  m.prev[s] = b;
  m.queued[b] = 1;
  ++m.num_queued;
}

// Head of the free queue, taken out; its hash entry (if any) is dropped
// because the block is about to be overwritten.
static int32_t queue_pop_front(pa_kv_manager &m) {
  const int32_t b = m.next[m.num_blocks];
  queue_remove(m, b);
  if (m.hashed[b]) {
    auto it = m.cached.find(m.hash[b]);
    if (it != m.cached.end() && it->second == b) m.cached.erase(it);
    m.hashed[b] = 0;
  }
  return b;
}

static int32_t blocks_for(int64_t tokens, int32_t S) { return (int32_t)((tokens + S - 1) / S); }

}  // namespace pa

using namespace pa;

extern "C" {

pa_status pa_kv_manager_create(int32_t num_blocks, int32_t block_size, pa_kv_manager **out) {
  if (!out) return pa_set_error(PA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0) return pa_set_error(PA_ERR_INVALID_ARG, "num_blocks and block_size must be positive");
  pa_kv_manager *m = new pa_kv_manager;
  m->num_blocks = num_blocks;
  m->block_size = block_size;
  m->ref.assign(num_blocks, 0);
  m->prev.assign(num_blocks + 1, num_blocks);
  m->next.assign(num_blocks + 1, num_blocks);
  m->queued.assign(num_blocks, 0);
  m->hashed.assign(num_blocks, 0);
  m->hash.assign(num_blocks, 0);
  m->key.resize(num_blocks);
  for (int32_t b = 0; b < num_blocks; ++b) queue_push_back(*m, b);
  *out = m;
  return PA_OK;
}

void pa_kv_manager_destroy(pa_kv_manager *m) { delete m; }

int32_t pa_kv_manager_num_free_blocks(pa_kv_manager *m) {
  if (!m) return -1;
  std::lock_guard<std::mutex> lk(m->mu);
  return m->num_queued;
}

pa_status pa_kv_manager_get_computed_blocks(pa_kv_manager *m, const int32_t *token_ids,
                                            int32_t num_tokens, uint64_t extra_key, int32_t *blocks,
                                            int32_t max_blocks, int32_t *num_blocks) {
  if (!m || !num_blocks || num_tokens < 0 || max_blocks < 0 || (num_tokens > 0 && !token_ids) ||
      (max_blocks > 0 && !blocks))
    return pa_set_error(PA_ERR_INVALID_ARG, "invalid argument");
  std::lock_guard<std::mutex> lk(m->mu);
  const int32_t S = m->block_size;
  // the block holding the last token is never reported: at least one token
  // of the request is computed in the step
  const int32_t full = num_tokens > 0 ? (num_tokens - 1) / S : 0;
  uint64_t parent = 0;
  int32_t n = 0;
  for (int32_t i = 0; i < full && n < max_blocks; ++i) {
    const int32_t *tok = token_ids + (int64_t)i * S;
    const uint64_t h = block_hash(parent, extra_key, tok, S);
    auto it = m->cached.find(h);
    if (it == m->cached.end()) break;
    const BlockKey &k = m->key[it->second];
    if (k.parent != parent || k.extra != extra_key || memcmp(k.tokens.data(), tok, (size_t)S * 4) != 0) break;
    blocks[n++] = it->second;
    parent = h;
  }
  *num_blocks = n;
  return PA_OK;
}

pa_status pa_kv_manager_allocate_slots(pa_kv_manager *m, int64_t request_id, int32_t num_tokens,
                                       const int32_t *computed_blocks, int32_t num_computed_blocks,
                                       int32_t *new_blocks, int32_t max_new, int32_t *num_new) {
  if (!m || !num_new || num_tokens < 0 || num_computed_blocks < 0 || max_new < 0 ||
      (num_computed_blocks > 0 && !computed_blocks) || (max_new > 0 && !new_blocks))
    return pa_set_error(PA_ERR_INVALID_ARG, "invalid argument");
  std::lock_guard<std::mutex> lk(m->mu);
  *num_new = 0;
  auto it = m->req_blocks.find(request_id);
  const int32_t have = it == m->req_blocks.end() ? 0 : (int32_t)it->second.size();
  if (have > 0 && num_computed_blocks > 0)
    return pa_set_error(PA_ERR_INVALID_ARG, "computed blocks are only taken by a request that holds none yet");
  for (int32_t i = 0; i < num_computed_blocks; ++i) {
    const int32_t b = computed_blocks[i];
    if (b < 0 || b >= m->num_blocks) return pa_set_error(PA_ERR_INVALID_ARG, "computed block %d outside the pool", b);
    if (!m->hashed[b]) return pa_set_error(PA_ERR_INVALID_ARG, "computed block %d holds no cached content", b);
  }
  const int32_t need = blocks_for(num_tokens, m->block_size);
  const int32_t fresh = need - have - num_computed_blocks;
  // hit blocks that sit in the free queue leave it when touched
  int32_t hit_queued = 0;
  for (int32_t i = 0; i < num_computed_blocks; ++i) hit_queued += m->queued[computed_blocks[i]];
  if (fresh > 0 && fresh > m->num_queued - hit_queued)
    return pa_set_error(PA_ERR_CAPACITY, "request %lld needs %d new blocks, %d free", (long long)request_id,
                        fresh, m->num_queued - hit_queued);
  if (fresh > max_new) return pa_set_error(PA_ERR_INVALID_ARG, "new_blocks holds %d ids, %d needed", max_new, fresh);
  std::vector<int32_t> &list = m->req_blocks[request_id];
  for (int32_t i = 0; i < num_computed_blocks; ++i) {      // touch
    const int32_t b = computed_blocks[i];
    if (m->queued[b]) queue_remove(*m, b);
    ++m->ref[b];
    list.push_back(b);
  }
  for (int32_t i = 0; i < fresh; ++i) {
    const int32_t b = queue_pop_front(*m);
    m->ref[b] = 1;
    list.push_back(b);
    new_blocks[i] = b;
  }
  *num_new = fresh > 0 ? fresh : 0;
  return PA_OK;
}

pa_status pa_kv_manager_cache_blocks(pa_kv_manager *m, int64_t request_id, const int32_t *token_ids,
                                     int32_t num_tokens, uint64_t extra_key) {
  if (!m || num_tokens < 0 || (num_tokens > 0 && !token_ids)) return pa_set_error(PA_ERR_INVALID_ARG, "invalid argument");
  std::lock_guard<std::mutex> lk(m->mu);
  auto it = m->req_blocks.find(request_id);
  if (it == m->req_blocks.end()) return pa_set_error(PA_ERR_INVALID_ARG, "unknown request %lld", (long long)request_id);
  const int32_t S = m->block_size;
  const std::vector<int32_t> &list = it->second;
  const int32_t full = std::min<int32_t>(num_tokens / S, (int32_t)list.size());
  uint64_t parent = 0;
  for (int32_t i = 0; i < full; ++i) {
    const int32_t b = list[i];
    const int32_t *tok = token_ids + (int64_t)i * S;
    const uint64_t h = block_hash(parent, extra_key, tok, S);
    if (!m->hashed[b] && m->cached.find(h) == m->cached.end()) {
      m->cached[h] = b;
      m->hashed[b] = 1;
      m->hash[b] = h;
      m->key[b].parent = parent;
      m->key[b].extra = extra_key;
      m->key[b].tokens.assign(tok, tok + S);
    }
    parent = h;
  }
  return PA_OK;
}

pa_status pa_kv_manager_free(pa_kv_manager *m, int64_t request_id) {
  if (!m) return pa_set_error(PA_ERR_INVALID_ARG, "manager is NULL");
  std::lock_guard<std::mutex> lk(m->mu);
  auto it = m->req_blocks.find(request_id);
  if (it == m->req_blocks.end()) return pa_set_error(PA_ERR_INVALID_ARG, "unknown request %lld", (long long)request_id);
  const std::vector<int32_t> &list = it->second;
  for (size_t i = list.size(); i-- > 0;) {
    const int32_t b = list[i];
    if (--m->ref[b] == 0) queue_push_back(*m, b);
  }
  m->req_blocks.erase(it);
  return PA_OK;
}

pa_status pa_kv_manager_block_ids(pa_kv_manager *m, int64_t request_id, int32_t *blocks,
                                  int32_t max_blocks, int32_t *num_blocks) {
  if (!m || !num_blocks || max_blocks < 0 || (max_blocks > 0 && !blocks))
    return pa_set_error(PA_ERR_INVALID_ARG, "invalid argument");
  std::lock_guard<std::mutex> lk(m->mu);
  auto it = m->req_blocks.find(request_id);
  if (it == m->req_blocks.end()) return pa_set_error(PA_ERR_INVALID_ARG, "unknown request %lld", (long long)request_id);
  const int32_t n = (int32_t)it->second.size();
  if (n > max_blocks) return pa_set_error(PA_ERR_INVALID_ARG, "blocks holds %d ids, request has %d", max_blocks, n);
  memcpy(blocks, it->second.data(), (size_t)n * 4);
  *num_blocks = n;
  return PA_OK;
}

pa_status pa_kv_manager_ref_count(pa_kv_manager *m, int32_t block, int32_t *ref_count) {
  if (!m || !ref_count || block < 0 || block >= m->num_blocks) return pa_set_error(PA_ERR_INVALID_ARG, "invalid argument");
  std::lock_guard<std::mutex> lk(m->mu);
  *ref_count = m->ref[block];
  return PA_OK;
}

}  // extern "C"
