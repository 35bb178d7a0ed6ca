/*
 * pkv.h — C ABI of libpkv: attention over a paged KV cache with prefix reuse,
 * hand-written HIP kernels for MI355X (gfx950).
 *
 * Source of the operations (pages, cited by title and section):
 *  [A] "PagedAttention과 RadixAttention으로 LLM KV 캐시 최적화" (aitrends.kr):
 *      §02 fixed 16/32-token blocks, a per-request block table mapping logical
 *      blocks to scattered physical blocks that the attention kernel reads as
 *      one contiguous sequence; §03 reuse of the longest cached prefix so only
 *      the suffix is computed; §05 reuse leaves the model output unchanged.
 *  [B] "KV Cache 완전 정리 — PagedAttention vs RadixAttention" (cell-devlog):
 *      "FP8 KV 캐시" — the cache may be stored as fp8 e4m3.
 *  [C] "KV Cache에 대해 알아보자 (Feat. Attention)" (chooblog): §1 the
 *      attention equation softmax(QK^T / sqrt(d_k)) V; §3 prefill processes
 *      all new tokens at once, decode appends the new token's K, V and attends
 *      over the whole cache; §4 grouped-query attention (fewer KV heads).
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  - Every tensor is described by a pkv_tensor: a DEVICE pointer owned by the
 *    caller, a dtype, and shape/strides in ELEMENTS. The library never
 *    allocates, frees or retains device memory; pointers are used only by work
 *    enqueued during the call.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without synchronising. Buffers must outlive that work.
 *  - Validation is host-side only: the library never reads device memory to
 *    validate and never synchronises. On error nothing is launched, a status
 *    other than PKV_OK is returned and pkv_last_error() describes it.
 *  - Device-side values are clamped, not trusted: a block id outside
 *    [0, num_blocks) is clamped into range, a length past a table's capacity is
 *    cut to the capacity, a negative length counts as 0, and a slot outside
 *    [0, num_blocks*B) is skipped. Results for such inputs are unspecified but
 *    every memory access stays inside the caller's buffers.
 *  - block_tables hold at most 2^24 entries per row (a capacity of at most
 *    2^29 tokens), so that every position the kernels form fits in 32 bits.
 *  - scale is the softmax scale of [C] §1 (1/sqrt(d) in the usual model). Any
 *    finite value is accepted, including negative ones and 0 (uniform weights
 *    over the visible keys); scale * k_scale * log2(e) must be finite.
 *  - Thread safety: no global mutable state other than the thread-local error
 *    string; concurrent calls on different streams are safe.
 *
 * Physical cache layout (the pages leave it open; this library's choice)
 * ----------------------------------------------------------------------
 *  A token's SLOT is physical_block * B + offset_in_block ([A] §02). The K and
 *  V caches of one layer are two contiguous tensors:
 *     k_cache: [num_blocks, H_kv, B, d]   one (block, head) = B rows of d
 *     v_cache: [num_blocks, H_kv, d, B]   one (block, head) = d rows of B tokens
 *  i.e. each (block, KV head) is one contiguous tile, and V tiles are stored
 *  transposed so that both attention products read their matrix-core operands
 *  with 16-byte loads. Element of token `slot`, head h, dim i:
 *     K: k_cache[slot / B][h][slot % B][i]     V: v_cache[slot / B][h][i][slot % B]
 *  Supported: d in {64, 128}, B in {16, 32}; cache dtype f32, f16, bf16 (same
 *  as q) or fp8 e4m3fn (q in f16 or bf16; values are code * scale).
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 6

typedef enum {
  PKV_F32 = 0,
  PKV_F16 = 1,
  PKV_BF16 = 2,
  PKV_FP8_E4M3FN = 3, /* OCP e4m3fn: bias 7, no infinities, 0x7F/0xFF NaN, max 448 */
  PKV_I32 = 4,
  PKV_I64 = 5
} pkv_dtype;

typedef struct {
  void* data;        /* device pointer */
  int32_t dtype;     /* a pkv_dtype */
  int32_t ndim;      /* 1..4 */
  int64_t shape[4];
  int64_t stride[4]; /* in elements */
} pkv_tensor;

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,        /* a required pointer is NULL */
  PKV_ERR_DTYPE = 2,       /* unsupported dtype or dtype combination */
  PKV_ERR_SHAPE = 3,       /* shapes disagree with each other */
  PKV_ERR_LAYOUT = 4,      /* strides / alignment not supported */
  PKV_ERR_UNSUPPORTED = 5, /* head_dim, block size or head grouping not supported */
  PKV_ERR_WORKSPACE = 6,   /* decode workspace missing or too small */
  PKV_ERR_HIP = 7,         /* the HIP runtime reported an error at launch */
  PKV_ERR_NO_BLOCKS = 8,   /* prefix index: too few free or evictable blocks */
  PKV_ERR_NOT_FOUND = 9    /* prefix index: unknown request or stored prefix */
} pkv_status;

/*
 * pkv_append — write new tokens' K and V rows into their cache slots.
 * [C] §3 (decode adds the new token's K, V to the cache; prefill writes the
 * K, V of every new token); [A] §02 (the slot comes from the block table).
 *
 *  k, v          [T, H_kv, d], dtype f32/f16/bf16; last dim contiguous,
 *                row starts 16-byte aligned.
 *  slot_mapping  [T] int32 or int64; row i goes to slot slot_mapping[i].
 *                Negative (or out-of-range) slots are skipped. Two rows naming
 *                the same slot in one call: which one lands is unspecified.
 *  k_cache       [num_blocks, H_kv, B, d] contiguous (layout above).
 *  v_cache       [num_blocks, H_kv, d, B] contiguous.
 *  k_scale,      used only for fp8 caches: the stored code is
 *  v_scale       e4m3fn(x / scale), the float32 quotient rounded to nearest
 *                with ties to even and saturated to +-448. Must be > 0.
 *                For other caches the row dtype must equal the cache dtype and
 *                the copy is bit-exact.
 * Bytes not named by a slot are never written.
 */
int pkv_append(const pkv_tensor* k, const pkv_tensor* v, const pkv_tensor* slot_mapping,
               const pkv_tensor* k_cache, const pkv_tensor* v_cache, float k_scale,
               float v_scale, void* stream);

/*
 * pkv_decode_workspace_bytes — bytes of device workspace pkv_decode_attn needs
 * on the CURRENT device: per-wave partial results for sequences that several
 * waves share, (waves_per_head + num_seqs) * H_q * (head_dim + 2) floats, plus
 * two ints per sequence. waves_per_head = 8 * (compute units) / (H_kv *
 * ceil(G / 16)), at least 1; the environment variable PKV_DECODE_WAVES (a
 * positive integer) replaces the 8 * (compute units) total for both calls.
 * max_blocks_per_seq and block_size do not change the size (kept for
 * callers that size by the full problem). Returns 0 on invalid sizes.
 */
size_t pkv_decode_workspace_bytes(int64_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int64_t max_blocks_per_seq,
                                  int32_t block_size);

/*
 * pkv_decode_attn — one decode step of paged attention.
 * [C] §3: the new token's query attends to every cached K, V of its sequence;
 * [C] §1: out = softmax(scale * q K^T) V; [C] §4: query head h reads KV head
 * h / G with G = H_q / H_kv; [A] §02: token t of sequence s lives in physical
 * block block_tables[s][t / B] at offset t % B.
 *
 *  q             [num_seqs, H_q, d], f32/f16/bf16; last dim contiguous, rows
 *                16-byte aligned.
 *  k_cache,      caches in the layout above.
 *  v_cache
 *  block_tables  [num_seqs, max_blocks] int32, row stride >= max_blocks; only
 *                the first ceil(context_lens[s] / B) entries are read.
 *  context_lens  [num_seqs] int32: cached tokens of each sequence, including
 *                the newest one. 0 gives a zero output row.
 *  scale         softmax scale (1/sqrt(d) in the usual model).
 *  k_scale,      dequantization scales of an fp8 cache (ignored otherwise).
 *  v_scale
 *  workspace     device buffer of at least pkv_decode_workspace_bytes(...)
 *                bytes, 16-byte aligned (the caller allocates it; it holds
 *                partial results). No initial contents are needed; calls
 *                that share one workspace must be ordered on one stream.
 *  out           [num_seqs, H_q, d], same dtype as q; last dim contiguous.
 * Results are bitwise deterministic and depend only on logical positions, so
 * permuting physical blocks or aliasing identical blocks between sequences
 * does not change a single bit.
 */
int pkv_decode_attn(const pkv_tensor* q, const pkv_tensor* k_cache, const pkv_tensor* v_cache,
                    const pkv_tensor* block_tables, const pkv_tensor* context_lens, float scale,
                    float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                    const pkv_tensor* out, void* stream);

/*
 * pkv_decode_attn_noalloc — pkv_decode_attn without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops without an allocator, harnesses that forbid allocation).
 * Same arguments, results and bits as pkv_decode_attn, minus the workspace:
 * the partial results live in a device-resident array of 32 MiB inside the
 * library, one per GPU, set up on the first call on each device and held
 * until the process ends. The call never allocates or frees memory.
 *  - A batch whose pkv_decode_workspace_bytes(...) exceeds 32 MiB is rejected
 *    with PKV_ERR_WORKSPACE before anything is launched (at 8 KV heads,
 *    d = 128 and 256 compute units: up to 1,759 sequences of 32 query heads,
 *    752 of 64).
 *  - Every call on one GPU shares that GPU's array and nothing in it needs
 *    clearing; calls that overlap on one GPU (different streams, or different
 *    threads without ordering) race on it and give wrong results. Calls
 *    ordered on one stream are safe.
 */
int pkv_decode_attn_noalloc(const pkv_tensor* q, const pkv_tensor* k_cache, const pkv_tensor* v_cache,
                            const pkv_tensor* block_tables, const pkv_tensor* context_lens, float scale,
                            float k_scale, float v_scale, const pkv_tensor* out, void* stream);

/*
 * pkv_decode_step_attn — a whole decode step in one call: pkv_append of each
 * sequence's newest token at position context_lens[s] - 1 (its slot taken
 * from the block table), then pkv_decode_attn over context_lens[s] tokens.
 * [C] §3: the new token's K, V join the cache and its query attends to all of
 * them; [A] §02: position t lives in block block_tables[s][t / B] at offset
 * t % B. The wave that reads the newest position takes its K, V from k_new /
 * v_new and also writes them to the cache, so no separate append launch runs.
 * Outputs and cache contents are bit for bit those of pkv_append (with
 * slot_mapping[s] = that slot) followed by pkv_decode_attn.
 *
 *  k_new, v_new  [num_seqs, H_kv, d]: the newest token's K and V rows. Their
 *                dtype is the cache dtype (copied bit for bit), or the q dtype
 *                for an fp8 cache (stored as e4m3fn(x / k_scale), resp.
 *                v_scale, as pkv_append stores it). Last dim contiguous, rows
 *                16-byte aligned.
 *  other args    as for pkv_decode_attn (same workspace size).
 * A sequence with context_lens[s] <= 0 appends nothing and gets a zero row.
 * The newest position's slot must not be one that another sequence of the
 * same call reads (a block shared by several sequences is never appended to).
 */
int pkv_decode_step_attn(const pkv_tensor* q, const pkv_tensor* k_new, const pkv_tensor* v_new,
                         const pkv_tensor* k_cache, const pkv_tensor* v_cache, const pkv_tensor* block_tables,
                         const pkv_tensor* context_lens, float scale, float k_scale, float v_scale,
                         void* workspace, size_t workspace_bytes, const pkv_tensor* out, void* stream);

/*
 * pkv_suffix_prefill_attn — attention for the new suffix tokens of requests
 * whose prefix is already cached.
 * [A] §03: with the longest matching prefix reused from the cache, only the
 * unmatched suffix is computed; [C] §3: prefill handles all new tokens at
 * once; [C] §1: the attention equation. Suffix row i of request r (absolute
 * position P_r + i) attends to key positions 0 .. P_r + i inclusive: the whole
 * prefix and the suffix causally. The suffix K, V must already be in the cache
 * (pkv_append them first).
 *
 *  q_suffix      [sum_r S_r, H_q, d] packed request by request; f16 or bf16
 *                (the products run on matrix cores); rows 16-byte aligned.
 *  k_cache,      caches in the layout above.
 *  v_cache
 *  block_tables  [R, max_blocks] int32; request r reads entries
 *                0 .. ceil((P_r + S_r) / B) - 1.
 *  prefix_lens   [R] int32, P_r >= 0 (cut to the table's capacity).
 *  suffix_lens   [R] int32, S_r >= 0; sum_r S_r must equal q_suffix.shape[0]
 *                (the device values are trusted only up to that total).
 *                sum_r S_r * (H_q / H_kv) must stay below 2^30.
 *  scale,        as for pkv_decode_attn.
 *  k_scale,
 *  v_scale
 *  out           [sum_r S_r, H_q, d], same dtype as q_suffix.
 */
int pkv_suffix_prefill_attn(const pkv_tensor* q_suffix, const pkv_tensor* k_cache,
                            const pkv_tensor* v_cache, const pkv_tensor* block_tables,
                            const pkv_tensor* prefix_lens, const pkv_tensor* suffix_lens,
                            float scale, float k_scale, float v_scale, const pkv_tensor* out,
                            void* stream);

/*
 * pkv_suffix_prefill_workspace_bytes — bytes of device workspace that
 * pkv_suffix_prefill_attn_split needs on the CURRENT device for a batch of
 * total_suffix_tokens rows from num_requests requests: 0 when the batch
 * needs no split, else parts * total_suffix_tokens * H_q * (head_dim + 2)
 * floats. parts (per row tile, 2..17) comes from the shapes alone: a batch
 * whose row tiles, ceil(total * G / 256) per KV head, give every compute unit
 * at least half a work-group takes no split; otherwise each tile gets enough
 * parts to fill the compute units, with prefix chunks of at least 256 keys at
 * the table's capacity. The environment variable PKV_PREFILL_SPLITS (1..17)
 * sets the count for both calls. num_requests does not change the size.
 * Returns 0 on invalid sizes as well.
 */
size_t pkv_suffix_prefill_workspace_bytes(int64_t total_suffix_tokens, int64_t num_requests,
                                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                          int64_t max_blocks_per_seq, int32_t block_size);

/*
 * pkv_suffix_prefill_attn_split — pkv_suffix_prefill_attn for batches with
 * few suffix rows and long prefixes: one conversation's next turn ([C] §5,
 * third limit: each turn of a multi-turn conversation carries every earlier
 * turn, whose K, V are cached; [A] §03: only the new suffix is computed),
 * which a plain launch spreads over only H_kv work-groups per 256 rows. The keys of each row tile are split:
 * parts 0 .. parts-2 take chunks of the prefix's whole 64-key stages (every
 * suffix row sees them all), the last part the remaining prefix keys and the
 * suffix (causally); each part writes an unnormalised partial (O, m, l) and a
 * second launch merges them by log-sum-exp. Same arguments, contract and
 * result as pkv_suffix_prefill_attn (the sums run in another order, so the
 * bits may differ within rounding), plus:
 *  workspace     at least pkv_suffix_prefill_workspace_bytes(...) bytes
 *                (max_blocks_per_seq = block_tables.shape[1]), 16-byte
 *                aligned, no initial contents needed; may be NULL when that
 *                size is 0, and the call is then pkv_suffix_prefill_attn.
 *                Calls sharing one workspace must be ordered on one stream.
 */
int pkv_suffix_prefill_attn_split(const pkv_tensor* q_suffix, const pkv_tensor* k_cache,
                                  const pkv_tensor* v_cache, const pkv_tensor* block_tables,
                                  const pkv_tensor* prefix_lens, const pkv_tensor* suffix_lens,
                                  float scale, float k_scale, float v_scale, void* workspace,
                                  size_t workspace_bytes, const pkv_tensor* out, void* stream);

/*
 * pkv_cascade_workspace_bytes — bytes of device workspace pkv_cascade_decode_attn
 * needs on the CURRENT device: the decode workspace (rounded up to 16 bytes)
 * plus, for the shared part, one partial result per (key chunk, sequence,
 * query head): splits * num_seqs * H_q * (head_dim + 2) floats. The shared
 * keys form one chunk (splits = 1) unless the environment variable
 * PKV_CASCADE_SPLITS (1..16) sets another count, for both calls. Returns 0
 * on invalid sizes.
 */
size_t pkv_cascade_workspace_bytes(int64_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim);

/*
 * pkv_cascade_decode_attn — one decode step for sequences that share prefix
 * blocks, reading each shared block once per group instead of once per
 * sequence.
 * [A] §03: a common prefix is stored once and reused by every request that
 * starts with it; [B] "RadixAttention": one system prompt shared by many chat
 * requests; [C] §1, §3: the decode attention equation.
 * The result is the one pkv_decode_attn computes for the same inputs:
 * out[s, h] = softmax(scale * q[s,h] K_s^T) V_s over context_lens[s] tokens.
 * It is computed in two parts merged by log-sum-exp: for each group, all
 * queries of its sequences against its shared prefix at once (matrix cores),
 * and for each sequence the tokens after the shared prefix. Both parts run in
 * one kernel launch, followed by a merge launch, on `stream`.
 *
 *  q, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale,
 *  out           as for pkv_decode_attn; q and out must be f16 or bf16.
 *  group_starts  [G + 1] int32, ascending, group_starts[0] = 0 and
 *                group_starts[G] = num_seqs: group g is sequences
 *                group_starts[g] .. group_starts[g+1] - 1.
 *  shared_lens   [num_seqs] int32: tokens of the sequence's group prefix, the
 *                same for every sequence of a group. The first
 *                shared_lens[s] / B entries of the block tables of a group
 *                must name the same blocks (a group of one with
 *                shared_lens 0 is a plain decode). Lengths are rounded down to
 *                whole blocks and cut to each sequence's context; the shared
 *                part is read through the group's first sequence's table.
 *  workspace     at least pkv_cascade_workspace_bytes(...) bytes, 16-byte
 *                aligned; no initial contents needed; calls sharing one
 *                workspace must be ordered on one stream.
 * Inputs that break the group contract give unspecified results, but every
 * access stays inside the caller's buffers.
 */
int pkv_cascade_decode_attn(const pkv_tensor* q, const pkv_tensor* k_cache, const pkv_tensor* v_cache,
                            const pkv_tensor* block_tables, const pkv_tensor* context_lens,
                            const pkv_tensor* group_starts, const pkv_tensor* shared_lens, float scale,
                            float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                            const pkv_tensor* out, void* stream);

/* Description of the last error on the calling thread ("" if none). The
 * pointer stays valid until the next pkv_* call on this thread. */
const char* pkv_last_error(void);

/* PKV_ABI_VERSION of the loaded library. */
int pkv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
