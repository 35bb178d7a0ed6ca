/*
 * pkv_prefix.h — C ABI of libpkv's host-side prefix index: the step before the
 * attention kernels that turns token IDs into the block tables, prefix lengths
 * and slot mappings they consume (include/pkv.h). Host memory only; no GPU
 * call is made, so these entry points also work on a machine without a GPU.
 *
 * Source of the operations (pages, cited by title and section):
 *  [A] "PagedAttention과 RadixAttention으로 LLM KV 캐시 최적화" (aitrends.kr):
 *      §02 blocks are allocated only for tokens that exist, and a block table
 *      maps a request's logical blocks to physical ones; §03 the longest cached
 *      prefix is reused and only the suffix is computed, kept in a radix tree
 *      that stores common prefixes once; §04 new KV joins the tree after a
 *      request, and under memory pressure leaves go first (least recently
 *      used), sparing shared interior prefixes; §05 chain hashing: a block's
 *      hash covers its parent's hash, its own token IDs and optional extra keys
 *      (LoRA id, multimodal input hash), and a request reuses blocks up to the
 *      first miss, allocating new ones from there; §06 a per-tenant salt is
 *      part of the cache identifier.
 *  [B] "KV Cache 완전 정리 — PagedAttention vs RadixAttention" (cell-devlog):
 *      "PagedAttention" pages no longer used are reused by other requests;
 *      "RadixAttention" one shared system prompt with per-user branches, LRU.
 *
 * Conventions
 * -----------
 *  - Every call returns a pkv_status (include/pkv.h); on error nothing changes
 *    and pkv_last_error() describes it. Two more statuses are used here:
 *    PKV_ERR_NO_BLOCKS (the pool has too few free or evictable blocks) and
 *    PKV_ERR_NOT_FOUND (unknown request id; a prefix to lock is not stored;
 *    unlock without lock).
 *  - Objects are created and destroyed by the library; all other pointers are
 *    caller-owned host memory, read or written only during the call.
 *  - An object is not thread-safe: calls on one object must be serialised.
 *    Different objects are independent.
 *
 * Policies where the pages are silent (the same in the test model):
 *  - Only full blocks are published and matched; a partly filled block belongs
 *    to its request. When every token of a request is cached, its last block is
 *    still computed, so that at least one token goes through the model.
 *  - A hit needs the block's 64-bit chain hash, its parent's chain hash and its
 *    own token IDs to be equal to the stored ones (a false hit needs a 64-bit
 *    collision of the parent chain).
 *  - New blocks come from a FIFO free list, then from evicting the least
 *    recently released cached block. A request releases its blocks tail first.
 */
#ifndef PKV_PREFIX_H_
#define PKV_PREFIX_H_

#include <stdint.h>

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------- chain-hash prefix cache over a block pool ([A] §02, §05, §06) */

typedef struct pkv_prefix_cache pkv_prefix_cache;

/* A pool of num_blocks physical blocks of block_size tokens, all free.
 * num_blocks in [1, 2^31), block_size in [1, 4096]. */
int pkv_pc_create(int64_t num_blocks, int32_t block_size, pkv_prefix_cache** out);
void pkv_pc_destroy(pkv_prefix_cache* pc);

/*
 * pkv_pc_admit — a new request of n >= 1 tokens (token IDs, any int32).
 *  salt          tenant salt ([A] §06); equal token lists with different salts
 *                never share blocks.
 *  extra         further identity ([A] §05: LoRA id, multimodal hash); 0 = none.
 *  block_table   out: ceil(n / B) physical block ids, in logical order; the
 *                caller passes room for max_blocks >= ceil(n / B) entries.
 *  slot_mapping  out: the slot (block * B + offset) of tokens prefix_len .. n-1,
 *                n - prefix_len entries; room for n entries must be passed.
 *  prefix_len    out: tokens whose K, V are already cached (a multiple of B,
 *                < n): the suffix prefill starts there.
 *  request_id    out: the handle for the calls below.
 * Reused blocks gain a reference; new blocks are taken as described above.
 * PKV_ERR_NO_BLOCKS if ceil(n / B) - hits blocks cannot be found.
 */
int pkv_pc_admit(pkv_prefix_cache* pc, const int32_t* tokens, int64_t n, uint64_t salt,
                 uint64_t extra, int32_t* block_table, int64_t max_blocks, int64_t* slot_mapping,
                 int64_t* prefix_len, int64_t* request_id);

/* One more token for a running request ([C] §3 decode: the new token's K, V go
 * into the cache): its slot, taking a new block when the last one is full. */
int pkv_pc_append(pkv_prefix_cache* pc, int64_t request_id, int32_t token, int64_t* slot);

/* The request's K, V are written: its full blocks that are not yet cached
 * become matchable ([A] §04: new KV is inserted after a request). *published
 * (may be NULL) receives how many blocks were published. */
int pkv_pc_commit(pkv_prefix_cache* pc, int64_t request_id, int64_t* published);

/* The request is finished: each block loses a reference (tail first); cached
 * blocks nobody uses stay matchable until evicted, the others become free. */
int pkv_pc_release(pkv_prefix_cache* pc, int64_t request_id);

/* The request's current block table (it grows with pkv_pc_append): up to
 * max_blocks entries are written, *num_blocks receives the full count. */
int pkv_pc_block_table(const pkv_prefix_cache* pc, int64_t request_id, int32_t* block_table,
                       int64_t max_blocks, int64_t* num_blocks);

/* Pool state: free blocks, cached blocks no request uses (evictable), and all
 * cached blocks. Any pointer may be NULL. */
int pkv_pc_stats(const pkv_prefix_cache* pc, int64_t* free_blocks, int64_t* evictable,
                 int64_t* cached);

/* ---------------- radix tree ([A] §03, §04; [B] "RadixAttention") */

typedef struct pkv_radix pkv_radix;

/* An empty tree matching in whole pages of `page` tokens (1 = token level,
 * B = the block size of a paged cache). page in [1, 4096]. */
int pkv_radix_create(int32_t page, pkv_radix** out);
void pkv_radix_destroy(pkv_radix* t);

/* Longest stored prefix of tokens[0..n) in whole pages: *matched tokens, and
 * their stored values in values[0..*matched) (room for n entries). The nodes
 * on the path count as used now. */
int pkv_radix_match(pkv_radix* t, const int32_t* tokens, int64_t n, int64_t* values,
                    int64_t* matched);

/* Store tokens[0..n') with values[0..n'), n' = n rounded down to a whole
 * page; an edge matched part-way is split. *existing (may be NULL) receives
 * how many leading tokens were already stored; their old values are kept. */
int pkv_radix_insert(pkv_radix* t, const int32_t* tokens, int64_t n, const int64_t* values,
                     int64_t* existing);

/* A running request holds the first `length` stored tokens (whole pages):
 * none of their nodes can be evicted until the matching unlock. */
int pkv_radix_lock(pkv_radix* t, const int32_t* tokens, int64_t length);
int pkv_radix_unlock(pkv_radix* t, const int32_t* tokens, int64_t length);

/* Remove unlocked leaves, least recently used first (ties: older node first),
 * until at least num_tokens tokens are gone, nothing more can go, or the next
 * leaf's values would not fit in `capacity`. A node with children is never
 * removed. The removed values are written in order to values[0..*evicted). */
int pkv_radix_evict(pkv_radix* t, int64_t num_tokens, int64_t* values, int64_t capacity,
                    int64_t* evicted);

/* Tokens stored in the tree. */
int pkv_radix_total_tokens(const pkv_radix* t, int64_t* total);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PREFIX_H_ */
