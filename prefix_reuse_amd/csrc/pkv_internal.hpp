// Internal host/device interface of libpkv: launch parameter blocks and the
// launchers each kernel file provides. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr float kLog2eHost = 1.4426950408889634f;

enum class DT : int { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3, I32 = 4, I64 = 5 };

struct AppendParams {
  const void* k; const void* v;       // [T, Hkv, D]
  int64_t k_s0, k_s1, v_s0, v_s1;     // element strides of token / head
  const void* slots; int slots_i64;   // [T]
  void* k_cache; void* v_cache;       // [NB, Hkv, B, D] / [NB, Hkv, D, B]
  int64_t num_tokens;
  int32_t hkv, num_blocks;
  float k_scale, v_scale;
};

struct DecodeParams {
  const void* q; int64_t q_s0, q_s1;  // [S, Hq, D]
  const void* k_cache; const void* v_cache;
  const int32_t* block_tables; int64_t bt_s0; int32_t max_blocks;
  const int32_t* context_lens;
  void* out; int64_t o_s0, o_s1;
  float* ws_o;                        // [waves_per_head + S, Hq, D] unnormalised partial outputs
  float* ws_ml;                       // [waves_per_head + S, Hq, 2] running max (log2 units) and sum
  int32_t* seq_info;                  // [S, 2] first wave and number of waves of each sequence
  int32_t num_seqs, hq, hkv, group, head_chunks, num_blocks;
  int32_t waves_per_head;             // waves sharing the chunks of one (KV head, head chunk)
  int32_t total_wgs;                  // one wave per work-group
  float qk_scale_log2;                // softmax scale * k_scale * log2(e)
  float v_scale;
  // cascade decode (nullptr otherwise): each sequence's shared-prefix length
  // (rounded down to whole blocks, at most its context); the decode kernel
  // covers only the tokens after it and writes every result as a partial,
  // and the combine merges in the shared partial [S, Hq, D] / [S, Hq, 2]
  const int32_t* shared_lens;
  const float* sh_o;                  // [sh_splits, S, Hq, D]: one partial per key split
  const float* sh_ml;                 // [sh_splits, S, Hq, 2]
  int32_t sh_splits;
  // decode step (nullptr otherwise): the newest token of each sequence,
  // [S, Hkv, D] in the cache dtype (in the q dtype for an fp8 cache), at
  // position context_lens[s] - 1. The wave that reads that position takes it
  // from here and writes it into the cache slot, as pkv_append would.
  const void* k_new; const void* v_new;
  int64_t kn_s0, kn_s1, vn_s0, vn_s1;
  float k_quant, v_quant;             // fp8: code = e4m3fn(x / scale)
};

// Suffix-prefill work-group: kPrefillWaves waves of 32 (token, head) rows each.
constexpr int kPrefillWaves = 8;
constexpr int kPrefillRowsPerWg = 32 * kPrefillWaves;

struct PrefillParams {
  const void* q; int64_t q_s0, q_s1;  // [total, Hq, D]
  const void* k_cache; const void* v_cache;
  const int32_t* block_tables; int64_t bt_s0; int32_t max_blocks;
  const int32_t* prefix_lens; const int32_t* suffix_lens;
  void* out; int64_t o_s0, o_s1;
  int32_t num_reqs, hq, hkv, group, num_blocks;
  int64_t total_rows;                 // sum_r S_r (host-known)
  int32_t tiles_per_head;             // grid size / hkv (upper bound on tiles)
  float qk_scale_log2;                // |softmax scale * k_scale| * log2(e), > 0
  float v_scale;
  int32_t q_mode;                     // 0: q as given; 1: q negated (negative scale); 2: q zeroed (zero scale)
  // cascade decode's shared part (group_starts == nullptr otherwise): the
  // "requests" are groups of sequences group_starts[g] .. group_starts[g+1]-1,
  // one query row per (sequence, head), attending to the group's shared
  // prefix (shared_lens of its first sequence, whole blocks, read through
  // that sequence's block table) up to each sequence's own context length;
  // unnormalised partials go to ws_o [S, Hq, D] and ws_ml [S, Hq, 2]
  const int32_t* group_starts;
  const int32_t* context_lens;
  const int32_t* shared_lens;
  float* ws_o;                        // [key_splits, S, Hq, D]
  float* ws_ml;                       // [key_splits, S, Hq, 2]
  int32_t key_splits;                 // work-groups sharing one row tile's shared keys
  // key-split suffix prefill (launch_prefill_split): key_splits parts per row
  // tile, the first key_splits - 1 on chunks of the prefix's whole stages
  // (split_prefix_keys), the last on the keys after them; partials go to
  // ws_o [key_splits, total_rows, Hq, D] and ws_ml [key_splits, total_rows, Hq, 2]
};

// Cascade decode: the shared keys of a group (L, whole blocks) are cut into
// `splits` chunks of whole 64-key stages; chunk i covers keys
// [i * chunk, min(L, (i + 1) * chunk)).
constexpr int kCascadeChunkAlign = 64;
__host__ __device__ inline int cascade_chunk(int L, int splits) {
  const int c = (L + splits - 1) / splits;
  return (c + kCascadeChunkAlign - 1) / kCascadeChunkAlign * kCascadeChunkAlign;
}

// Key-split suffix prefill: the prefix keys that the split parts take (whole
// 64-key stages; the last part takes the rest of the prefix and the suffix),
// cut into chunks as above.
__host__ __device__ inline int split_prefix_keys(int P) { return P - P % kCascadeChunkAlign; }

// Supplies a decode workspace of `need` bytes in place of the caller's (the
// entry point that allocates nothing); returns a pkv_status.
typedef int (*ScratchFn)(size_t need, void** ptr);

// Validation and launch of pkv_decode_attn (k_new = v_new = nullptr) and
// pkv_decode_step_attn; with `scratch` set, the workspace arguments are
// ignored and scratch(need, &ptr) supplies the workspace once every argument
// is valid.
int decode_call(const pkv_tensor* q, const pkv_tensor* k_new, const pkv_tensor* v_new, const pkv_tensor* k_cache,
                const pkv_tensor* v_cache, const pkv_tensor* block_tables, const pkv_tensor* context_lens,
                float scale, float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                ScratchFn scratch, const pkv_tensor* out, void* stream);

// Decode launch plan shared by the launcher and the workspace-size query.
struct DecodePlan { int32_t waves_per_head; int32_t total_waves; };
DecodePlan plan_decode(int64_t num_seqs, int32_t hkv, int32_t head_chunks, int32_t num_cus);

hipError_t launch_append(const AppendParams& p, DT row_dt, DT cache_dt, int head_dim,
                         int block_size, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, DT q_dt, DT cache_dt, int head_dim,
                         int block_size, hipStream_t stream);
// the decode's combine kernel alone (after a cascade kernel wrote the partials)
hipError_t launch_decode_combine(const DecodeParams& p, DT q_dt, DT cache_dt, int head_dim,
                                 int block_size, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, DT q_dt, DT cache_dt, int head_dim,
                          int block_size, hipStream_t stream);
// The suffix prefill with its keys split (p.key_splits >= 2 parts per row
// tile, tiles_per_head counting the parts), then the merge of the parts.
hipError_t launch_prefill_split(const PrefillParams& p, DT q_dt, DT cache_dt, int head_dim,
                                int block_size, hipStream_t stream);
// Cascade decode: the shared part (work-groups [0, shared_wgs), a multiple of
// 8 and at least sp.hkv * sp.tiles_per_head) and the private-token decode
// (dp.total_wgs waves, eight per work-group) in one launch, then the combine.
hipError_t launch_cascade(const PrefillParams& sp, const DecodeParams& dp, int shared_wgs, DT q_dt, DT cache_dt,
                          int head_dim, int block_size, hipStream_t stream);

}  // namespace pkv
