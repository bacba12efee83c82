/*
 * gdn_ckpt.h -- host checkpoint index of linear states (C ABI).
 *
 * A linear layer's state cannot be shared block by block the way a KV prefix
 * is; a prefix hit restores the deepest saved checkpoint into the request's
 * live slot instead (page "Qwen3.5 Linear-State Prefix Cache", sections 2.2 and
 * 5.1).  This index answers "how far can this request be restored, and from
 * which slot": it maps a chained per-chunk key to the pool slot that holds the
 * state at that chunk boundary.
 *
 *   key(i)  covers tokens [0, (i+1)*stride) and is chained from key(i-1) and the
 *           chunk's own tokens (section 4: a hash domain of its own with the
 *           prefill chunk as its step, computed once per sequence and extended
 *           as it grows).  Hash: 64-bit FNV-1a over the previous key's 8
 *           little-endian bytes, then the chunk's tokens as 4 little-endian
 *           bytes each; chunk 0 starts from the offset basis alone.
 *   match   probes every whole chunk that ends strictly below the final token
 *           ((i+1)*stride <= n_tokens - 1), gaps allowed, and takes only the
 *           deepest hit: reach = (i+1)*stride (section 6.2).  Probing leaves the
 *           recency order alone; taking the hit pins it (reference count + 1)
 *           and makes it the most recent.
 *   insert  stores a checkpoint under the key recorded at its boundary
 *           (section 5.2, insert_with_recorded_hash).
 *   evict   a full index drops its least recently used unpinned entry.
 *
 * All calls are host-only and synchronous; an index is not thread-safe (one
 * scheduler thread owns it).  Errors return a negative gdn_status with a
 * message for gdn_last_error().
 */
#ifndef GDN_CKPT_H
#define GDN_CKPT_H

#include <stddef.h>
#include <stdint.h>

#include "gdn_slot.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gdn_ckpt_index *gdn_ckpt_index_t;

/* Outcome of ckpt_index_insert. */
enum { GDN_CKPT_STORED = 0, GDN_CKPT_PRESENT = 1, GDN_CKPT_FULL = 2 };

/* Keys of the whole chunks first_chunk .. n_tokens/stride - 1 of a token
 * sequence, chained from prev_key (the key of chunk first_chunk - 1; ignored
 * when first_chunk == 0).  tokens: host int32 [n_tokens].  keys: host uint64
 * [keys_cap]; *n_keys receives the count (0 when the sequence holds no further
 * whole chunk).  GDN_ERR_RANGE if keys_cap is too small. */
gdn_status ckpt_chain_hashes(const int32_t *tokens, int64_t n_tokens, int32_t stride,
                             int64_t first_chunk, uint64_t prev_key, uint64_t *keys,
                             int64_t keys_cap, int64_t *n_keys);

/* An empty index of at most `capacity` checkpoints (>= 1). */
gdn_status ckpt_index_create(int32_t capacity, gdn_ckpt_index_t *out);

/* Free an index (not the slots it names).  NULL is ignored. */
void ckpt_index_destroy(gdn_ckpt_index_t idx);

/* Number of checkpoints held (-1 for a NULL index). */
int32_t ckpt_index_size(gdn_ckpt_index_t idx);

/* 1 if the key is held, 0 if not (-1 for a NULL index).  Does not change the
 * recency order. */
int32_t ckpt_index_contains(gdn_ckpt_index_t idx, uint64_t key);

/* Deepest checkpoint of a request: keys [n_keys] from ckpt_chain_hashes for
 * the request's n_tokens tokens.  On a hit: *reach = (i+1)*stride, *slot = the
 * checkpoint's slot, *key = its key, and the entry is pinned until
 * ckpt_index_release(*key).  On a miss: *reach = 0, *slot = -1, *key = 0. */
gdn_status ckpt_index_match(gdn_ckpt_index_t idx, const uint64_t *keys, int64_t n_keys,
                            int64_t n_tokens, int32_t stride, int64_t *reach, int32_t *slot,
                            uint64_t *key);

/* Unpin a checkpoint taken by ckpt_index_match once its restore copy is done
 * (GDN_ERR_ARG if the key is not held or not pinned). */
gdn_status ckpt_index_release(gdn_ckpt_index_t idx, uint64_t key);

/* Store `slot` as the checkpoint of `key`.  *outcome:
 *   GDN_CKPT_STORED   stored; *slot_back = the slot of an evicted entry or -1
 *                     (the caller returns it to its free list);
 *   GDN_CKPT_PRESENT  the key is already held and keeps its slot; *slot_back =
 *                     `slot` (the caller keeps or frees it);
 *   GDN_CKPT_FULL     every entry is pinned, nothing stored; *slot_back = `slot`. */
gdn_status ckpt_index_insert(gdn_ckpt_index_t idx, uint64_t key, int32_t slot, int32_t *outcome,
                             int32_t *slot_back);

/* The scheduler's step for a batch of new or resumed requests (section 5.1):
 * for request r with tokens [cu_tokens[r], cu_tokens[r+1]) of `tokens` and live
 * slot live_slots[r], hash its whole chunks, match (pinning the hit), and fill
 * ops[r] = {live_slots[r], 1, hit slot or -1} for restore_slots, which turns a
 * miss into a cold start.  reach[r] and hit_keys[r] (0 on a miss) receive the
 * match; the caller releases every non-zero hit key after the restore copies
 * have run.  n_req >= 0; all arrays host memory. */
gdn_status ckpt_plan_restores(gdn_ckpt_index_t idx, int32_t n_req, const int32_t *tokens,
                              const int64_t *cu_tokens, int32_t stride, const int32_t *live_slots,
                              gdn_restore_op *ops, int64_t *reach, uint64_t *hit_keys);

/* A request finishes (page "SGLang Mamba Radix Cache 深度解析", cache_finished_req
 * with the ping-pong track slots): the track slot other(next) =
 * track_slots[1 - (next_track_idx & 1)] holds the state of the last tracked
 * boundary and is handed to the index under that boundary's recorded key,
 * without a copy; the live slot and track_slots[next_track_idx & 1] are
 * released.  has_key = 0 means no boundary was tracked and every slot is
 * released.  freed (host int32 [4]) receives the slots the caller returns to
 * its free list, *n_freed their count: the live slot, the other track slot,
 * the kept slot when the index does not take it (key already held, or every
 * entry pinned), and a slot the insert evicted.  Ids <= 0 are left out. */
gdn_status ckpt_finish_request(gdn_ckpt_index_t idx, int32_t has_key, uint64_t key,
                               int32_t live_slot, const int32_t *track_slots,
                               int32_t next_track_idx, int32_t *freed, int32_t *n_freed);

#ifdef __cplusplus
}
#endif
#endif /* GDN_CKPT_H */
