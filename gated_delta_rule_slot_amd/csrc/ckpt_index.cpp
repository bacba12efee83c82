// ckpt_index.cpp -- the host checkpoint index declared in include/gdn_ckpt.h.
//
// Layout: checkpoints live in a fixed pool of `capacity` nodes (key, slot,
// reference count, previous / next in the recency list); an open-addressing
// table with linear probing maps a key to its node.  The table has a power of
// two buckets, at least twice the capacity, and deletes by backward shifting,
// so lookups never walk tombstones.  The recency list runs from the least
// recently used node (head) to the most recent (tail); eviction walks it from
// the head to the first unpinned node.
#include <stdint.h>
#include <string.h>

#include <new>
#include <vector>

#include "errors.hpp"
#include "gdn_ckpt.h"

#define GDN_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr uint64_t kFnvOffset = 14695981039346656037ull;
constexpr uint64_t kFnvPrime = 1099511628211ull;

inline uint64_t fnv_byte(uint64_t h, uint8_t b) { return (h ^ b) * kFnvPrime; }

// key of one chunk: FNV-1a over the previous key (8 bytes, little endian; none
// for chunk 0) and the chunk's tokens (4 bytes each, little endian)
uint64_t chunk_key(bool first, uint64_t prev, const int32_t *tok, int32_t stride) {
  uint64_t h = kFnvOffset;
  if (!first)
    for (int i = 0; i < 8; ++i) h = fnv_byte(h, uint8_t(prev >> (8 * i)));
  for (int32_t t = 0; t < stride; ++t) {
    const uint32_t v = uint32_t(tok[t]);
    h = fnv_byte(h, uint8_t(v));
    h = fnv_byte(h, uint8_t(v >> 8));
    h = fnv_byte(h, uint8_t(v >> 16));
    h = fnv_byte(h, uint8_t(v >> 24));
  }
  return h;
}

constexpr int32_t kNone = -1;

struct Node {
  uint64_t key;
  int32_t slot;
  int32_t refs;
  int32_t prev, next;  // recency list
};

}  // namespace

struct gdn_ckpt_index {
  std::vector<Node> nodes;
  std::vector<int32_t> free_nodes;
  std::vector<int32_t> table;  // node index or kNone
  uint64_t mask = 0;
  int32_t head = kNone, tail = kNone, count = 0;

  static uint64_t mix(uint64_t k) {  // spread FNV output over the bucket bits
    k ^= k >> 33;
    k *= 0xff51afd7ed558ccdull;
    k ^= k >> 33;
    return k;
  }
  int64_t bucket_of(uint64_t key) const {
    for (uint64_t b = mix(key) & mask;; b = (b + 1) & mask) {
      const int32_t n = table[b];
      if (n == kNone || nodes[n].key == key) return int64_t(b);
    }
  }
  int32_t find_node(uint64_t key) const { return table[bucket_of(key)]; }

  void unlink(int32_t n) {
    Node &x = nodes[n];
    if (x.prev != kNone) nodes[x.prev].next = x.next; else head = x.next;
    if (x.next != kNone) nodes[x.next].prev = x.prev; else tail = x.prev;
    x.prev = x.next = kNone;
  }
  void push_tail(int32_t n) {
    Node &x = nodes[n];
    x.prev = tail;
    x.next = kNone;
    if (tail != kNone) nodes[tail].next = n; else head = n;
    tail = n;
  }
  // remove the key's bucket, shifting later members of its probe run back
  void erase_bucket(uint64_t b) {
    table[b] = kNone;
    for (uint64_t j = (b + 1) & mask; table[j] != kNone; j = (j + 1) & mask) {
      const int32_t n = table[j];
      const uint64_t home = mix(nodes[n].key) & mask;
      // n may move into the hole at b if its home does not lie in (b, j]
      const bool between = b <= j ? (home > b && home <= j) : (home > b || home <= j);
      if (!between) {
        table[b] = n;
        table[j] = kNone;
        b = j;
      }
    }
  }
};

GDN_API gdn_status ckpt_chain_hashes(const int32_t *tokens, int64_t n_tokens, int32_t stride,
                                     int64_t first_chunk, uint64_t prev_key, uint64_t *keys,
                                     int64_t keys_cap, int64_t *n_keys) {
  if (!n_keys) return gdn::set_error(GDN_ERR_ARG, "n_keys is NULL");
  if (stride < 1) return gdn::set_error(GDN_ERR_ARG, "stride %d < 1", stride);
  if (n_tokens < 0 || first_chunk < 0) return gdn::set_error(GDN_ERR_RANGE, "negative count");
  const int64_t chunks = n_tokens / stride;
  const int64_t n = chunks > first_chunk ? chunks - first_chunk : 0;
  *n_keys = n;
  if (n == 0) return gdn::clear_error();
  if (!tokens || !keys) return gdn::set_error(GDN_ERR_ARG, "tokens or keys is NULL");
  if (keys_cap < n) return gdn::set_error(GDN_ERR_RANGE, "keys_cap %lld < %lld", (long long)keys_cap, (long long)n);
  uint64_t k = prev_key;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t c = first_chunk + i;
    k = chunk_key(c == 0, k, tokens + c * stride, stride);
    keys[i] = k;
  }
  return gdn::clear_error();
}

GDN_API gdn_status ckpt_index_create(int32_t capacity, gdn_ckpt_index_t *out) {
  if (!out) return gdn::set_error(GDN_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (capacity < 1 || capacity > (1 << 28)) return gdn::set_error(GDN_ERR_RANGE, "capacity %d", capacity);
  gdn_ckpt_index *x = new (std::nothrow) gdn_ckpt_index;
  if (!x) return gdn::set_error(GDN_ERR_ARG, "out of host memory");
  uint64_t buckets = 16;
  while (buckets < 2ull * uint64_t(capacity)) buckets <<= 1;
  try {
    x->nodes.resize(capacity);
    x->table.assign(buckets, kNone);
    x->free_nodes.reserve(capacity);
  } catch (...) {
    delete x;
    return gdn::set_error(GDN_ERR_ARG, "out of host memory");
  }
  for (int32_t i = capacity - 1; i >= 0; --i) x->free_nodes.push_back(i);
  x->mask = buckets - 1;
  *out = x;
  return gdn::clear_error();
}

GDN_API void ckpt_index_destroy(gdn_ckpt_index_t idx) { delete idx; }

GDN_API int32_t ckpt_index_size(gdn_ckpt_index_t idx) { return idx ? idx->count : -1; }

GDN_API int32_t ckpt_index_contains(gdn_ckpt_index_t idx, uint64_t key) {
  if (!idx) return -1;
  return idx->find_node(key) != kNone ? 1 : 0;
}

GDN_API gdn_status ckpt_index_match(gdn_ckpt_index_t idx, const uint64_t *keys, int64_t n_keys,
                                    int64_t n_tokens, int32_t stride, int64_t *reach,
                                    int32_t *slot, uint64_t *key) {
  if (!idx || !reach || !slot || !key) return gdn::set_error(GDN_ERR_ARG, "a required pointer is NULL");
  if (stride < 1 || n_keys < 0) return gdn::set_error(GDN_ERR_ARG, "stride < 1 or n_keys < 0");
  if (n_keys > 0 && !keys) return gdn::set_error(GDN_ERR_ARG, "keys is NULL");
  *reach = 0;
  *slot = -1;
  *key = 0;
  // whole chunks that end strictly below the final token
  int64_t eligible = n_tokens >= 1 ? (n_tokens - 1) / stride : 0;
  if (eligible > n_keys) eligible = n_keys;
  for (int64_t i = eligible - 1; i >= 0; --i) {  // the deepest hit is the first found from the end
    const int32_t n = idx->find_node(keys[i]);
    if (n == kNone) continue;
    Node &x = idx->nodes[n];
    x.refs += 1;
    idx->unlink(n);
    idx->push_tail(n);
    *reach = (i + 1) * int64_t(stride);
    *slot = x.slot;
    *key = x.key;
    break;
  }
  return gdn::clear_error();
}

GDN_API gdn_status ckpt_index_release(gdn_ckpt_index_t idx, uint64_t key) {
  if (!idx) return gdn::set_error(GDN_ERR_ARG, "index is NULL");
  const int32_t n = idx->find_node(key);
  if (n == kNone) return gdn::set_error(GDN_ERR_ARG, "key not held");
  if (idx->nodes[n].refs <= 0) return gdn::set_error(GDN_ERR_ARG, "release without a matching match");
  idx->nodes[n].refs -= 1;
  return gdn::clear_error();
}

GDN_API gdn_status ckpt_index_insert(gdn_ckpt_index_t idx, uint64_t key, int32_t slot,
                                     int32_t *outcome, int32_t *slot_back) {
  if (!idx || !outcome || !slot_back) return gdn::set_error(GDN_ERR_ARG, "a required pointer is NULL");
  if (idx->find_node(key) != kNone) {
    *outcome = GDN_CKPT_PRESENT;
    *slot_back = slot;
    return gdn::clear_error();
  }
  int32_t evicted = -1;
  if (idx->free_nodes.empty()) {
    int32_t v = idx->head;
    while (v != kNone && idx->nodes[v].refs > 0) v = idx->nodes[v].next;
    if (v == kNone) {
      *outcome = GDN_CKPT_FULL;
      *slot_back = slot;
      return gdn::clear_error();
    }
    evicted = idx->nodes[v].slot;
    idx->erase_bucket(uint64_t(idx->bucket_of(idx->nodes[v].key)));
    idx->unlink(v);
    idx->free_nodes.push_back(v);
    idx->count -= 1;
  }
  const int32_t n = idx->free_nodes.back();
  idx->free_nodes.pop_back();
  idx->nodes[n] = Node{key, slot, 0, kNone, kNone};
  idx->table[idx->bucket_of(key)] = n;
  idx->push_tail(n);
  idx->count += 1;
  *outcome = GDN_CKPT_STORED;
  *slot_back = evicted;
  return gdn::clear_error();
}

GDN_API gdn_status ckpt_plan_restores(gdn_ckpt_index_t idx, int32_t n_req, const int32_t *tokens,
                                      const int64_t *cu_tokens, int32_t stride,
                                      const int32_t *live_slots, gdn_restore_op *ops,
                                      int64_t *reach, uint64_t *hit_keys) {
  if (!idx) return gdn::set_error(GDN_ERR_ARG, "index is NULL");
  if (n_req < 0 || stride < 1) return gdn::set_error(GDN_ERR_ARG, "n_req < 0 or stride < 1");
  if (n_req == 0) return gdn::clear_error();
  if (!cu_tokens || !live_slots || !ops || !reach || !hit_keys)
    return gdn::set_error(GDN_ERR_ARG, "a required pointer is NULL");
  std::vector<uint64_t> keys;
  for (int32_t r = 0; r < n_req; ++r) {
    const int64_t b = cu_tokens[r], n = cu_tokens[r + 1] - cu_tokens[r];
    if (b < 0 || n < 0) return gdn::set_error(GDN_ERR_RANGE, "request %d: bad token range", r);
    const int64_t chunks = n / stride;
    try {
      keys.resize(size_t(chunks));
    } catch (...) {
      return gdn::set_error(GDN_ERR_ARG, "out of host memory");
    }
    int64_t nk = 0;
    gdn_status s = ckpt_chain_hashes(tokens + b, n, stride, 0, 0, keys.data(), chunks, &nk);
    if (s != GDN_OK) return s;
    int32_t slot = -1;
    s = ckpt_index_match(idx, keys.data(), nk, n, stride, &reach[r], &slot, &hit_keys[r]);
    if (s != GDN_OK) return s;
    ops[r].linear_state_id = live_slots[r];
    ops[r].restore_requested = 1;
    ops[r].restore_src_slot_id = slot;
  }
  return gdn::clear_error();
}

GDN_API gdn_status ckpt_finish_request(gdn_ckpt_index_t idx, int32_t has_key, uint64_t key,
                                       int32_t live_slot, const int32_t *track_slots,
                                       int32_t next_track_idx, int32_t *freed, int32_t *n_freed) {
  if (!idx || !track_slots || !freed || !n_freed)
    return gdn::set_error(GDN_ERR_ARG, "a required pointer is NULL");
  const int32_t cur = next_track_idx & 1;
  const int32_t keep = track_slots[1 - cur];
  int32_t n = 0;
  auto give = [&](int32_t s) {
    if (s > 0) freed[n++] = s;
  };
  give(live_slot);
  give(track_slots[cur]);
  if (!has_key) {
    give(keep);
  } else {
    int32_t outcome = 0, back = -1;
    const gdn_status st = ckpt_index_insert(idx, key, keep, &outcome, &back);
    if (st != GDN_OK) return st;
    give(back);  // an evicted slot, or the kept slot when the index did not take it
  }
  *n_freed = n;
  return gdn::clear_error();
}
