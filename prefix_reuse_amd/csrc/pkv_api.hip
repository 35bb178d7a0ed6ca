// extern "C" entry points of libpkv: host-side validation of the tensor
// descriptors, launch planning and kernel launches on the caller's stream.
// Nothing here reads device memory or synchronises.
#include "../../include/pkv.h"
#include "pkv_internal.hpp"

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <string>

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return PKV_OK;
}

size_t dtype_size(int dt) {
  switch (dt) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3FN: return 1;
    case PKV_I32: return 4;
    case PKV_I64: return 8;
    default: return 0;
  }
}

const char* dtype_name(int dt) {
  switch (dt) {
    case PKV_F32: return "f32";
    case PKV_F16: return "f16";
    case PKV_BF16: return "bf16";
    case PKV_FP8_E4M3FN: return "fp8_e4m3fn";
    case PKV_I32: return "i32";
    case PKV_I64: return "i64";
    default: return "?";
  }
}

// Basic sanity of a descriptor: non-null, known dtype, expected rank.
int check_tensor(const pkv_tensor* t, const char* name, int ndim) {
  if (!t) return fail(PKV_ERR_NULL, "%s: descriptor is NULL", name);
  if (dtype_size(t->dtype) == 0) return fail(PKV_ERR_DTYPE, "%s: unknown dtype %d", name, t->dtype);
  if (t->ndim != ndim) return fail(PKV_ERR_SHAPE, "%s: expected %d dims, got %d", name, ndim, t->ndim);
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] < 0) return fail(PKV_ERR_SHAPE, "%s: negative extent in dim %d", name, i);
  int64_t numel = 1;
  for (int i = 0; i < ndim; ++i) {
    if (t->shape[i] > 0 && numel > INT64_MAX / t->shape[i])
      return fail(PKV_ERR_SHAPE, "%s: element count overflows 64 bits", name);
    numel *= t->shape[i];
  }
  if (numel > 0 && !t->data) return fail(PKV_ERR_NULL, "%s: data pointer is NULL", name);
  return PKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Rows of a [n, heads, d] tensor: last dim contiguous, row starts 16-byte aligned.
int check_rows(const pkv_tensor* t, const char* name) {
  if (t->shape[2] > 1 && t->stride[2] != 1) return fail(PKV_ERR_LAYOUT, "%s: last dim must be contiguous", name);
  const size_t es = dtype_size(t->dtype);
  const bool s0 = t->shape[0] <= 1 || (t->stride[0] * (int64_t)es) % 16 == 0;
  const bool s1 = t->shape[1] <= 1 || (t->stride[1] * (int64_t)es) % 16 == 0;
  if (!aligned16(t->data) || !s0 || !s1)
    return fail(PKV_ERR_LAYOUT, "%s: rows must start on 16-byte boundaries", name);
  return PKV_OK;
}

struct CacheGeom {
  int64_t num_blocks;
  int32_t hkv, block, dim;
  int dtype;
};

// k_cache [NB, Hkv, B, D] and v_cache [NB, Hkv, D, B], both contiguous.
int check_caches(const pkv_tensor* kc, const pkv_tensor* vc, CacheGeom* g) {
  int rc;
  if ((rc = check_tensor(kc, "k_cache", 4))) return rc;
  if ((rc = check_tensor(vc, "v_cache", 4))) return rc;
  if (kc->dtype != vc->dtype) return fail(PKV_ERR_DTYPE, "k_cache and v_cache dtypes differ");
  if (kc->dtype == PKV_I32 || kc->dtype == PKV_I64) return fail(PKV_ERR_DTYPE, "cache dtype must be floating point");
  const int64_t nb = kc->shape[0], h = kc->shape[1], b = kc->shape[2], d = kc->shape[3];
  if (vc->shape[0] != nb || vc->shape[1] != h || vc->shape[2] != d || vc->shape[3] != b)
    return fail(PKV_ERR_SHAPE, "v_cache must be [num_blocks, H_kv, d, B] matching k_cache [num_blocks, H_kv, B, d]");
  if (!(d == 64 || d == 128)) return fail(PKV_ERR_UNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)d);
  if (!(b == 16 || b == 32)) return fail(PKV_ERR_UNSUPPORTED, "block size %lld not supported (16 or 32)", (long long)b);
  if (nb < 1 || h < 1) return fail(PKV_ERR_SHAPE, "caches must hold at least one block and one head");
  if (nb > INT32_MAX) return fail(PKV_ERR_SHAPE, "too many blocks");
  // contiguous in the stated order; the stride of a dim of extent 1 is irrelevant
  const int64_t ks[4] = {h * b * d, b * d, d, 1}, vs[4] = {h * d * b, d * b, b, 1};
  for (int i = 0; i < 4; ++i) {
    if (kc->shape[i] > 1 && kc->stride[i] != ks[i])
      return fail(PKV_ERR_LAYOUT, "k_cache must be contiguous [num_blocks, H_kv, B, d]");
    if (vc->shape[i] > 1 && vc->stride[i] != vs[i])
      return fail(PKV_ERR_LAYOUT, "v_cache must be contiguous [num_blocks, H_kv, d, B]");
  }
  if (!aligned16(kc->data) || !aligned16(vc->data)) return fail(PKV_ERR_LAYOUT, "caches must be 16-byte aligned");
  g->num_blocks = nb; g->hkv = (int32_t)h; g->block = (int32_t)b; g->dim = (int32_t)d; g->dtype = kc->dtype;
  return PKV_OK;
}

int check_int_vector(const pkv_tensor* t, const char* name, int64_t n) {
  int rc;
  if ((rc = check_tensor(t, name, 1))) return rc;
  if (t->dtype != PKV_I32) return fail(PKV_ERR_DTYPE, "%s must be int32", name);
  if (t->shape[0] != n) return fail(PKV_ERR_SHAPE, "%s: expected %lld entries, got %lld", name, (long long)n, (long long)t->shape[0]);
  if (n > 1 && t->stride[0] != 1) return fail(PKV_ERR_LAYOUT, "%s must be contiguous", name);
  return PKV_OK;
}

int check_block_tables(const pkv_tensor* t, int64_t rows) {
  int rc;
  if ((rc = check_tensor(t, "block_tables", 2))) return rc;
  if (t->dtype != PKV_I32) return fail(PKV_ERR_DTYPE, "block_tables must be int32");
  if (t->shape[0] != rows) return fail(PKV_ERR_SHAPE, "block_tables has %lld rows, expected %lld", (long long)t->shape[0], (long long)rows);
  if (t->shape[1] < 1) return fail(PKV_ERR_SHAPE, "block_tables needs at least one column");
  // max_blocks * B <= 2^29: with at most 2^30 rows, every position sum the
  // kernels form (prefix + suffix) stays inside int
  if (t->shape[1] > ((int64_t)1 << 24)) return fail(PKV_ERR_SHAPE, "block_tables too wide (at most 2^24 blocks per row)");
  if ((t->shape[1] > 1 && t->stride[1] != 1) || (rows > 1 && t->stride[0] < t->shape[1]))
    return fail(PKV_ERR_LAYOUT, "block_tables rows must be contiguous");
  return PKV_OK;
}

// The decode walks every 32-token chunk of every sequence with 32-bit chunk
// indices; with the device lengths cut to the tables' capacity, the most
// chunks a batch can hold must fit.
int check_chunk_count(int64_t num_seqs, int64_t max_blocks, int32_t block) {
  if (num_seqs * ((max_blocks * block + 31) / 32) > INT32_MAX)
    return fail(PKV_ERR_SHAPE, "num_seqs x table capacity exceeds 2^31 32-token chunks");
  return PKV_OK;
}

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

pkv::DT to_dt(int d) { return static_cast<pkv::DT>(d); }

// The score multiplier of the kernels, scale * k_scale * log2(e) (k_scale = 1
// for 16- and 32-bit caches). It must be finite.
int score_scale(float scale, bool fp8, float k_scale, float* qk) {
  if (!std::isfinite(scale)) return fail(PKV_ERR_SHAPE, "scale must be finite");
  *qk = scale * (fp8 ? k_scale : 1.0f) * pkv::kLog2eHost;
  if (!std::isfinite(*qk)) return fail(PKV_ERR_SHAPE, "scale * k_scale * log2(e) overflows float");
  return PKV_OK;
}

// The matrix-core kernels (suffix prefill, the cascade's shared part) take
// the row maximum of the raw scores and scale it afterwards, which needs a
// positive multiplier: a negative one is applied by negating q (exact), a
// zero one by zeroing q (every score 0, uniform weights), as softmax(scale *
// q K^T) asks for any finite scale.
void fold_scale(float qk, float* c2, int32_t* q_mode) {
  if (qk > 0.f) { *c2 = qk; *q_mode = 0; }
  else if (qk < 0.f) { *c2 = -qk; *q_mode = 1; }
  else { *c2 = pkv::kLog2eHost; *q_mode = 2; }
}

// Workspace: partial results [waves_per_head + S][Hq][D + 2] floats, then
// [S][2] ints of per-sequence partition info.
size_t decode_ws_bytes(int64_t num_seqs, int32_t hq, int32_t hkv, int32_t d, pkv::DecodePlan* plan_out) {
  const int32_t group = hq / hkv;
  const int32_t head_chunks = (group + 15) / 16;
  pkv::DecodePlan plan = pkv::plan_decode(num_seqs, hkv, head_chunks, device_cus());
  if (plan_out) *plan_out = plan;
  const size_t slots = (size_t)plan.waves_per_head + (size_t)num_seqs;
  return slots * hq * (size_t)(d + 2) * sizeof(float) + (size_t)num_seqs * 2 * sizeof(int32_t);
}

// Key-split suffix prefill: parts per row tile (1: no split), from what the
// host knows. A batch whose row tiles already give every CU half a
// work-group stays whole; otherwise each tile gets enough parts to fill the
// CUs (at most 17: 16 chunks of the prefix and the rest), with prefix chunks
// of at least 256 keys at the table's capacity. PKV_PREFILL_SPLITS (1..17)
// forces the count.
int prefill_parts(int64_t total, int32_t hq, int32_t hkv, int64_t max_blocks, int32_t block) {
  if (const char* env = getenv("PKV_PREFILL_SPLITS")) {
    const long forced = atol(env);
    if (forced >= 1 && forced <= 17) return (int)forced;
  }
  const int64_t W = pkv::kPrefillRowsPerWg;
  const int64_t tiles = (total * (hq / hkv) + W - 1) / W;  // row tiles of the fullest packing
  const int64_t wgs = tiles * hkv;
  const int64_t cus = device_cus();
  if (wgs == 0 || 2 * wgs > cus) return 1;
  int64_t parts = cus / wgs;
  parts = parts < 17 ? parts : 17;
  const int64_t by_keys = max_blocks * block / 256 + 1;
  parts = parts < by_keys ? parts : by_keys;
  return (int)(parts > 1 ? parts : 1);
}

// the partials of a key-split prefill: O [parts, total, H_q, d] and (m, l)
// [parts, total, H_q, 2] floats
size_t prefill_ws_bytes(int parts, int64_t total, int32_t hq, int32_t d) {
  return parts > 1 ? (size_t)parts * total * hq * (size_t)(d + 2) * sizeof(float) : 0;
}

// cascade: how many work-groups share one row tile of the shared part (each
// takes one chunk of the shared keys). The shared part runs beside the
// private-token decode in one launch, so it needs only to finish before the
// decode does, and every split adds a partial per (sequence, head) that is
// written and read back. PKV_CASCADE_SPLITS (1..16) forces the count.
int cascade_splits(int64_t num_seqs, int32_t hq, int32_t hkv) {
  if (const char* env = getenv("PKV_CASCADE_SPLITS")) {
    const long forced = atol(env);
    if (forced >= 1 && forced <= 16) return (int)forced;
  }
  (void)num_seqs, (void)hq, (void)hkv;
  return 1;
}

// cascade: the decode workspace (rounded up to 16 bytes; sized for a decode on
// every CU, the most the launch uses), then the shared partials
// O [splits, S, Hq, d] and (m, l) [splits, S, Hq, 2]
size_t cascade_ws_bytes(int64_t num_seqs, int32_t hq, int32_t hkv, int32_t d, pkv::DecodePlan* plan_out,
                        size_t* shared_offset, int* splits_out) {
  const size_t dec = (decode_ws_bytes(num_seqs, hq, hkv, d, plan_out) + 15) / 16 * 16;
  const int splits = cascade_splits(num_seqs, hq, hkv);
  if (shared_offset) *shared_offset = dec;
  if (splits_out) *splits_out = splits;
  return dec + (size_t)splits * num_seqs * hq * (size_t)(d + 2) * sizeof(float);
}

}  // namespace

namespace pkv {
// status of the calls implemented in other sources (the prefix index): the
// same thread-local message pkv_last_error() returns
int record_status(int code, const char* msg) {
  if (code == PKV_OK) g_error.clear();
  else g_error = msg ? msg : "";
  return code;
}
}  // namespace pkv

extern "C" {

int pkv_abi_version(void) { return PKV_ABI_VERSION; }


size_t pkv_cascade_workspace_bytes(int64_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim) {
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 || head_dim < 1)
    return 0;
  return cascade_ws_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, nullptr, nullptr, nullptr);
}

int pkv_cascade_decode_attn(const pkv_tensor* q, const pkv_tensor* k_cache, const pkv_tensor* v_cache,
                            const pkv_tensor* block_tables, const pkv_tensor* context_lens,
                            const pkv_tensor* group_starts, const pkv_tensor* shared_lens, float scale,
                            float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                            const pkv_tensor* out, void* stream) {
  int rc;
  CacheGeom cg;
  if ((rc = check_caches(k_cache, v_cache, &cg))) return rc;
  if ((rc = check_tensor(q, "q", 3))) return rc;
  if ((rc = check_tensor(out, "out", 3))) return rc;
  const int64_t S = q->shape[0], hq = q->shape[1];
  if (q->shape[2] != cg.dim) return fail(PKV_ERR_SHAPE, "q head_dim %lld != cache head_dim %d", (long long)q->shape[2], cg.dim);
  for (int i = 0; i < 3; ++i)
    if (out->shape[i] != q->shape[i]) return fail(PKV_ERR_SHAPE, "out shape differs from q");
  if (hq < 1 || hq % cg.hkv != 0) return fail(PKV_ERR_UNSUPPORTED, "H_q=%lld is not a multiple of H_kv=%d", (long long)hq, cg.hkv);
  if (hq > INT32_MAX || S > INT32_MAX) return fail(PKV_ERR_SHAPE, "too many sequences or heads");
  if (out->dtype != q->dtype) return fail(PKV_ERR_DTYPE, "out dtype must equal q dtype");
  if (q->dtype != PKV_F16 && q->dtype != PKV_BF16)
    return fail(PKV_ERR_DTYPE, "cascade decode needs q in f16 or bf16 (the shared part runs on matrix cores)");
  const bool fp8 = cg.dtype == PKV_FP8_E4M3FN;
  if (fp8) {
    if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
      return fail(PKV_ERR_SHAPE, "fp8 cache needs finite positive k_scale and v_scale");
  } else if (q->dtype != cg.dtype) {
    return fail(PKV_ERR_DTYPE, "q is %s but the cache is %s", dtype_name(q->dtype), dtype_name(cg.dtype));
  }
  if ((rc = check_block_tables(block_tables, S))) return rc;
  if ((rc = check_int_vector(context_lens, "context_lens", S))) return rc;
  if ((rc = check_chunk_count(S, block_tables->shape[1], cg.block))) return rc;
  if ((rc = check_int_vector(shared_lens, "shared_lens", S))) return rc;
  if ((rc = check_tensor(group_starts, "group_starts", 1))) return rc;
  const int64_t G = group_starts->shape[0] - 1;
  if (G < 0) return fail(PKV_ERR_SHAPE, "group_starts needs at least one entry");
  if ((rc = check_int_vector(group_starts, "group_starts", G + 1))) return rc;
  float qk = 0.f;
  if ((rc = score_scale(scale, fp8, k_scale, &qk))) return rc;
  if (S == 0) return ok();
  if ((rc = check_rows(q, "q"))) return rc;
  if ((rc = check_rows(out, "out"))) return rc;
  if (S * (hq / cg.hkv) > INT32_MAX / 2 || G > INT32_MAX) return fail(PKV_ERR_SHAPE, "too many rows");

  pkv::DecodePlan plan;
  size_t sh_off = 0;
  int splits = 1;
  const size_t need = cascade_ws_bytes(S, (int32_t)hq, cg.hkv, cg.dim, &plan, &sh_off, &splits);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "cascade workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(PKV_ERR_LAYOUT, "workspace must be 16-byte aligned");
  float* sh_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + sh_off);
  float* sh_ml = sh_o + (size_t)splits * S * hq * cg.dim;

  // the shared part: every group's queries over its shared prefix, once per
  // row tile (matrix cores)
  pkv::PrefillParams sp{};
  int64_t shared_wgs = 0;
  if (G > 0) {
    sp.q = q->data; sp.q_s0 = q->stride[0]; sp.q_s1 = q->stride[1];
    sp.k_cache = k_cache->data; sp.v_cache = v_cache->data;
    sp.block_tables = reinterpret_cast<const int32_t*>(block_tables->data);
    sp.bt_s0 = block_tables->stride[0]; sp.max_blocks = (int32_t)block_tables->shape[1];
    sp.num_reqs = (int32_t)G; sp.hq = (int32_t)hq; sp.hkv = cg.hkv; sp.group = (int32_t)(hq / cg.hkv);
    sp.num_blocks = (int32_t)cg.num_blocks; sp.total_rows = S;
    constexpr int64_t W = pkv::kPrefillRowsPerWg;
    // the row tiles of all groups: sum_g ceil(n_g G / W) <= floor(S G / W) + G
    // (exact for one group); work-groups past the real tiles return at once
    const int64_t rows = S * sp.group;
    const int64_t tiles = (G == 1 ? (rows + W - 1) / W : rows / W + G) * splits;
    if (tiles * cg.hkv > INT32_MAX / 2) return fail(PKV_ERR_SHAPE, "problem too large for one launch");
    sp.tiles_per_head = (int32_t)tiles;
    sp.key_splits = splits;
    fold_scale(qk, &sp.qk_scale_log2, &sp.q_mode);
    sp.v_scale = fp8 ? v_scale : 1.0f;
    sp.group_starts = reinterpret_cast<const int32_t*>(group_starts->data);
    sp.context_lens = reinterpret_cast<const int32_t*>(context_lens->data);
    sp.shared_lens = reinterpret_cast<const int32_t*>(shared_lens->data);
    sp.ws_o = sh_o;
    sp.ws_ml = sh_ml;
    shared_wgs = (tiles * cg.hkv + 7) / 8 * 8;
  }
  // the private-token decode, on the compute units the shared part leaves
  // (each shared work-group holds a whole CU), then the merge of all partials
  const int cus = device_cus();
  const int64_t busy = shared_wgs < cus / 2 ? shared_wgs : cus / 2;
  const int32_t head_chunks = (int32_t)((hq / cg.hkv + 15) / 16);
  const pkv::DecodePlan dplan = pkv::plan_decode(S, cg.hkv, head_chunks, (int32_t)(cus - busy));
  if (dplan.waves_per_head > plan.waves_per_head)
    return fail(PKV_ERR_WORKSPACE, "cascade decode plan exceeds its workspace");
  pkv::DecodeParams p{};
  p.q = q->data; p.q_s0 = q->stride[0]; p.q_s1 = q->stride[1];
  p.k_cache = k_cache->data; p.v_cache = v_cache->data;
  p.block_tables = reinterpret_cast<const int32_t*>(block_tables->data);
  p.bt_s0 = block_tables->stride[0]; p.max_blocks = (int32_t)block_tables->shape[1];
  p.context_lens = reinterpret_cast<const int32_t*>(context_lens->data);
  p.out = out->data; p.o_s0 = out->stride[0]; p.o_s1 = out->stride[1];
  p.num_seqs = (int32_t)S; p.hq = (int32_t)hq; p.hkv = cg.hkv; p.group = (int32_t)(hq / cg.hkv);
  p.head_chunks = head_chunks; p.num_blocks = (int32_t)cg.num_blocks;
  p.waves_per_head = dplan.waves_per_head;
  p.total_wgs = dplan.total_waves;
  const size_t slots = (size_t)dplan.waves_per_head + (size_t)S;
  p.ws_o = reinterpret_cast<float*>(workspace);
  p.ws_ml = p.ws_o + slots * hq * cg.dim;
  p.seq_info = reinterpret_cast<int32_t*>(p.ws_ml + slots * hq * 2);
  p.qk_scale_log2 = qk;
  p.v_scale = fp8 ? v_scale : 1.0f;
  p.shared_lens = reinterpret_cast<const int32_t*>(shared_lens->data);
  p.sh_o = sh_o;
  p.sh_ml = sh_ml;
  p.sh_splits = splits;
  if (shared_wgs + (p.total_wgs + 7) / 8 > INT32_MAX) return fail(PKV_ERR_SHAPE, "problem too large for one launch");
  hipError_t e = pkv::launch_cascade(sp, p, (int)shared_wgs, to_dt(q->dtype), to_dt(cg.dtype), cg.dim, cg.block,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "cascade decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

const char* pkv_last_error(void) { return g_error.c_str(); }

int pkv_append(const pkv_tensor* k, const pkv_tensor* v, const pkv_tensor* slot_mapping,
               const pkv_tensor* k_cache, const pkv_tensor* v_cache, float k_scale, float v_scale,
               void* stream) {
  int rc;
  CacheGeom cg;
  if ((rc = check_caches(k_cache, v_cache, &cg))) return rc;
  if ((rc = check_tensor(k, "k", 3))) return rc;
  if ((rc = check_tensor(v, "v", 3))) return rc;
  if ((rc = check_tensor(slot_mapping, "slot_mapping", 1))) return rc;
  const int64_t T = k->shape[0];
  for (int i = 0; i < 3; ++i)
    if (v->shape[i] != k->shape[i]) return fail(PKV_ERR_SHAPE, "k and v shapes differ");
  if (k->shape[1] != cg.hkv || k->shape[2] != cg.dim)
    return fail(PKV_ERR_SHAPE, "k/v rows are [%lld, %lld] but the cache holds [H_kv=%d, d=%d]",
                (long long)k->shape[1], (long long)k->shape[2], cg.hkv, cg.dim);
  if (slot_mapping->shape[0] != T) return fail(PKV_ERR_SHAPE, "slot_mapping has %lld entries for %lld tokens",
                                               (long long)slot_mapping->shape[0], (long long)T);
  if (slot_mapping->dtype != PKV_I32 && slot_mapping->dtype != PKV_I64)
    return fail(PKV_ERR_DTYPE, "slot_mapping must be int32 or int64");
  if (T > 1 && slot_mapping->stride[0] != 1) return fail(PKV_ERR_LAYOUT, "slot_mapping must be contiguous");
  if (k->dtype != v->dtype) return fail(PKV_ERR_DTYPE, "k and v dtypes differ");
  if (k->dtype != PKV_F32 && k->dtype != PKV_F16 && k->dtype != PKV_BF16)
    return fail(PKV_ERR_DTYPE, "k/v rows must be f32, f16 or bf16 (got %s)", dtype_name(k->dtype));
  if (cg.dtype == PKV_FP8_E4M3FN) {
    if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
      return fail(PKV_ERR_SHAPE, "fp8 cache needs finite positive k_scale and v_scale");
  } else if (k->dtype != cg.dtype) {
    return fail(PKV_ERR_DTYPE, "rows are %s but the cache is %s (only an fp8 cache converts)",
                dtype_name(k->dtype), dtype_name(cg.dtype));
  }
  if (T == 0) return ok();
  if ((rc = check_rows(k, "k"))) return rc;
  if ((rc = check_rows(v, "v"))) return rc;
  // two threads per (row, KV head, 8 dims), at most 2^31 - 1 work-groups of 256
  if (T > ((int64_t)1 << 37) / ((int64_t)cg.hkv * (cg.dim / 8)))
    return fail(PKV_ERR_SHAPE, "too many rows (%lld) for one append", (long long)T);

  pkv::AppendParams p{};
  p.k = k->data; p.v = v->data;
  p.k_s0 = k->stride[0]; p.k_s1 = k->stride[1]; p.v_s0 = v->stride[0]; p.v_s1 = v->stride[1];
  p.slots = slot_mapping->data; p.slots_i64 = slot_mapping->dtype == PKV_I64;
  p.k_cache = k_cache->data; p.v_cache = v_cache->data;
  p.num_tokens = T; p.hkv = cg.hkv; p.num_blocks = (int32_t)cg.num_blocks;
  p.k_scale = k_scale; p.v_scale = v_scale;
  hipError_t e = pkv::launch_append(p, to_dt(k->dtype), to_dt(cg.dtype), cg.dim, cg.block, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "append launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t pkv_decode_workspace_bytes(int64_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int64_t max_blocks_per_seq, int32_t block_size) {
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 ||
      head_dim < 1 || max_blocks_per_seq < 1 || block_size < 1)
    return 0;
  (void)max_blocks_per_seq;
  (void)block_size;
  return decode_ws_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, nullptr);
}

}  // extern "C"

namespace pkv {
// pkv_decode_attn, and with k_new / v_new (both or neither) pkv_decode_step_attn.
// With `scratch` set, the workspace arguments are ignored: once every argument
// is valid, scratch(need, &ptr) supplies a workspace of the `need` bytes the
// launch uses, or returns a status (having set the error message).
int decode_call(const pkv_tensor* q, const pkv_tensor* k_new, const pkv_tensor* v_new, const pkv_tensor* k_cache,
                const pkv_tensor* v_cache, const pkv_tensor* block_tables, const pkv_tensor* context_lens,
                float scale, float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                ScratchFn scratch, const pkv_tensor* out, void* stream) {
  int rc;
  CacheGeom cg;
  if ((rc = check_caches(k_cache, v_cache, &cg))) return rc;
  if ((rc = check_tensor(q, "q", 3))) return rc;
  if ((rc = check_tensor(out, "out", 3))) return rc;
  const int64_t S = q->shape[0], hq = q->shape[1];
  if (q->shape[2] != cg.dim) return fail(PKV_ERR_SHAPE, "q head_dim %lld != cache head_dim %d", (long long)q->shape[2], cg.dim);
  for (int i = 0; i < 3; ++i)
    if (out->shape[i] != q->shape[i]) return fail(PKV_ERR_SHAPE, "out shape differs from q");
  if (hq < 1 || hq % cg.hkv != 0) return fail(PKV_ERR_UNSUPPORTED, "H_q=%lld is not a multiple of H_kv=%d", (long long)hq, cg.hkv);
  if (hq > INT32_MAX || S > INT32_MAX) return fail(PKV_ERR_SHAPE, "too many sequences or heads");
  if (out->dtype != q->dtype) return fail(PKV_ERR_DTYPE, "out dtype must equal q dtype");
  const bool fp8 = cg.dtype == PKV_FP8_E4M3FN;
  if (fp8) {
    if (q->dtype != PKV_F16 && q->dtype != PKV_BF16) return fail(PKV_ERR_DTYPE, "an fp8 cache needs q in f16 or bf16");
    if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
      return fail(PKV_ERR_SHAPE, "fp8 cache needs finite positive k_scale and v_scale");
  } else if (q->dtype != cg.dtype) {
    return fail(PKV_ERR_DTYPE, "q is %s but the cache is %s", dtype_name(q->dtype), dtype_name(cg.dtype));
  }
  if ((rc = check_block_tables(block_tables, S))) return rc;
  if ((rc = check_int_vector(context_lens, "context_lens", S))) return rc;
  if ((rc = check_chunk_count(S, block_tables->shape[1], cg.block))) return rc;
  float qk = 0.f;
  if ((rc = score_scale(scale, fp8, k_scale, &qk))) return rc;
  const bool step = k_new != nullptr || v_new != nullptr;
  if (step) {
    if ((rc = check_tensor(k_new, "k_new", 3))) return rc;
    if ((rc = check_tensor(v_new, "v_new", 3))) return rc;
    for (int i = 0; i < 3; ++i)
      if (k_new->shape[i] != v_new->shape[i]) return fail(PKV_ERR_SHAPE, "k_new and v_new shapes differ");
    if (k_new->shape[0] != S || k_new->shape[1] != cg.hkv || k_new->shape[2] != cg.dim)
      return fail(PKV_ERR_SHAPE, "k_new/v_new must be [num_seqs=%lld, H_kv=%d, d=%d]", (long long)S, cg.hkv, cg.dim);
    const int want = fp8 ? q->dtype : cg.dtype;
    if (k_new->dtype != want || v_new->dtype != want)
      return fail(PKV_ERR_DTYPE, "k_new/v_new must be %s (%s)", dtype_name(want),
                  fp8 ? "the q dtype, quantized into the fp8 cache" : "the cache dtype, copied bit for bit");
  }
  if (S == 0) return ok();
  if ((rc = check_rows(q, "q"))) return rc;
  if ((rc = check_rows(out, "out"))) return rc;
  if (step) {
    if ((rc = check_rows(k_new, "k_new"))) return rc;
    if ((rc = check_rows(v_new, "v_new"))) return rc;
  }

  pkv::DecodePlan plan;
  const size_t need = decode_ws_bytes(S, (int32_t)hq, cg.hkv, cg.dim, &plan);
  if (scratch) {
    if ((rc = scratch(need, &workspace))) return rc;
    workspace_bytes = need;
  }
  if (workspace == nullptr || workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "decode workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(PKV_ERR_LAYOUT, "workspace must be 16-byte aligned");

  pkv::DecodeParams p{};
  p.q = q->data; p.q_s0 = q->stride[0]; p.q_s1 = q->stride[1];
  p.k_cache = k_cache->data; p.v_cache = v_cache->data;
  p.block_tables = reinterpret_cast<const int32_t*>(block_tables->data);
  p.bt_s0 = block_tables->stride[0]; p.max_blocks = (int32_t)block_tables->shape[1];
  p.context_lens = reinterpret_cast<const int32_t*>(context_lens->data);
  p.out = out->data; p.o_s0 = out->stride[0]; p.o_s1 = out->stride[1];
  p.num_seqs = (int32_t)S; p.hq = (int32_t)hq; p.hkv = cg.hkv; p.group = (int32_t)(hq / cg.hkv);
  p.head_chunks = (p.group + 15) / 16; p.num_blocks = (int32_t)cg.num_blocks;
  p.waves_per_head = plan.waves_per_head;
  p.total_wgs = plan.total_waves;
  const size_t slots = (size_t)plan.waves_per_head + (size_t)S;
  p.ws_o = reinterpret_cast<float*>(workspace);
  p.ws_ml = p.ws_o + slots * hq * cg.dim;
  p.seq_info = reinterpret_cast<int32_t*>(p.ws_ml + slots * hq * 2);
  p.qk_scale_log2 = qk;  // the decode scales before its maximum: any sign works
  p.v_scale = fp8 ? v_scale : 1.0f;
  if (step) {
    p.k_new = k_new->data; p.kn_s0 = k_new->stride[0]; p.kn_s1 = k_new->stride[1];
    p.v_new = v_new->data; p.vn_s0 = v_new->stride[0]; p.vn_s1 = v_new->stride[1];
    p.k_quant = k_scale;
    p.v_quant = v_scale;
  }
  hipError_t e = pkv::launch_decode(p, to_dt(q->dtype), to_dt(cg.dtype), cg.dim, cg.block, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}
}  // namespace pkv

namespace {
// pkv_suffix_prefill_attn, and with `split` pkv_suffix_prefill_attn_split
// (which falls back to the plain launch when the shape calls for no split).
int prefill_call(const pkv_tensor* q, const pkv_tensor* k_cache, const pkv_tensor* v_cache,
                 const pkv_tensor* block_tables, const pkv_tensor* prefix_lens, const pkv_tensor* suffix_lens,
                 float scale, float k_scale, float v_scale, void* workspace, size_t workspace_bytes, bool split,
                 const pkv_tensor* out, void* stream) {
  int rc;
  CacheGeom cg;
  if ((rc = check_caches(k_cache, v_cache, &cg))) return rc;
  if ((rc = check_tensor(q, "q_suffix", 3))) return rc;
  if ((rc = check_tensor(out, "out", 3))) return rc;
  const int64_t total = q->shape[0], hq = q->shape[1];
  if (q->shape[2] != cg.dim) return fail(PKV_ERR_SHAPE, "q_suffix head_dim %lld != cache head_dim %d", (long long)q->shape[2], cg.dim);
  for (int i = 0; i < 3; ++i)
    if (out->shape[i] != q->shape[i]) return fail(PKV_ERR_SHAPE, "out shape differs from q_suffix");
  if (hq < 1 || hq % cg.hkv != 0) return fail(PKV_ERR_UNSUPPORTED, "H_q=%lld is not a multiple of H_kv=%d", (long long)hq, cg.hkv);
  if (out->dtype != q->dtype) return fail(PKV_ERR_DTYPE, "out dtype must equal q_suffix dtype");
  if (q->dtype != PKV_F16 && q->dtype != PKV_BF16) return fail(PKV_ERR_DTYPE, "q_suffix must be f16 or bf16 (matrix cores)");
  const bool fp8 = cg.dtype == PKV_FP8_E4M3FN;
  if (fp8) {
    if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
      return fail(PKV_ERR_SHAPE, "fp8 cache needs finite positive k_scale and v_scale");
  } else if (q->dtype != cg.dtype) {
    return fail(PKV_ERR_DTYPE, "q_suffix is %s but the cache is %s", dtype_name(q->dtype), dtype_name(cg.dtype));
  }
  if ((rc = check_tensor(prefix_lens, "prefix_lens", 1))) return rc;
  const int64_t R = prefix_lens->shape[0];
  if ((rc = check_int_vector(prefix_lens, "prefix_lens", R))) return rc;
  if ((rc = check_int_vector(suffix_lens, "suffix_lens", R))) return rc;
  if ((rc = check_block_tables(block_tables, R))) return rc;
  float qk = 0.f;
  if ((rc = score_scale(scale, fp8, k_scale, &qk))) return rc;
  if (total == 0 || R == 0) return ok();
  if ((rc = check_rows(q, "q_suffix"))) return rc;
  if ((rc = check_rows(out, "out"))) return rc;
  if (total * (hq / cg.hkv) > INT32_MAX / 2 || R > INT32_MAX) return fail(PKV_ERR_SHAPE, "too many rows");

  pkv::PrefillParams p{};
  p.q = q->data; p.q_s0 = q->stride[0]; p.q_s1 = q->stride[1];
  p.k_cache = k_cache->data; p.v_cache = v_cache->data;
  p.block_tables = reinterpret_cast<const int32_t*>(block_tables->data);
  p.bt_s0 = block_tables->stride[0]; p.max_blocks = (int32_t)block_tables->shape[1];
  p.prefix_lens = reinterpret_cast<const int32_t*>(prefix_lens->data);
  p.suffix_lens = reinterpret_cast<const int32_t*>(suffix_lens->data);
  p.out = out->data; p.o_s0 = out->stride[0]; p.o_s1 = out->stride[1];
  p.num_reqs = (int32_t)R; p.hq = (int32_t)hq; p.hkv = cg.hkv; p.group = (int32_t)(hq / cg.hkv);
  p.num_blocks = (int32_t)cg.num_blocks; p.total_rows = total;
  // upper bound on row tiles per KV head: sum_r ceil(S_r * G / W) <= ceil(total * G / W) + R
  constexpr int64_t W = pkv::kPrefillRowsPerWg;
  const int64_t tiles = (total * p.group + W - 1) / W + R;
  if (tiles * cg.hkv > INT32_MAX) return fail(PKV_ERR_SHAPE, "problem too large for one launch");
  p.tiles_per_head = (int32_t)tiles;
  fold_scale(qk, &p.qk_scale_log2, &p.q_mode);
  p.v_scale = fp8 ? v_scale : 1.0f;
  const int parts = split ? prefill_parts(total, (int32_t)hq, cg.hkv, p.max_blocks, cg.block) : 1;
  if (parts > 1) {
    const size_t need = prefill_ws_bytes(parts, total, (int32_t)hq, cg.dim);
    if (workspace == nullptr || workspace_bytes < need)
      return fail(PKV_ERR_WORKSPACE, "suffix prefill workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if (!aligned16(workspace)) return fail(PKV_ERR_LAYOUT, "workspace must be 16-byte aligned");
    if (tiles * parts * cg.hkv > INT32_MAX || total * ((hq + 7) / 8) > INT32_MAX)
      return fail(PKV_ERR_SHAPE, "problem too large for one launch");
    p.key_splits = parts;
    p.tiles_per_head = (int32_t)(tiles * parts);
    p.ws_o = reinterpret_cast<float*>(workspace);
    p.ws_ml = p.ws_o + (size_t)parts * total * hq * cg.dim;
    hipError_t e = pkv::launch_prefill_split(p, to_dt(q->dtype), to_dt(cg.dtype), cg.dim, cg.block,
                                             (hipStream_t)stream);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
    return ok();
  }
  hipError_t e = pkv::launch_prefill(p, to_dt(q->dtype), to_dt(cg.dtype), cg.dim, cg.block, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int pkv_decode_attn(const pkv_tensor* q, const pkv_tensor* k_cache, const pkv_tensor* v_cache,
                    const pkv_tensor* block_tables, const pkv_tensor* context_lens, float scale,
                    float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                    const pkv_tensor* out, void* stream) {
  return pkv::decode_call(q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
                          v_scale, workspace, workspace_bytes, nullptr, out, stream);
}

int pkv_decode_step_attn(const pkv_tensor* q, const pkv_tensor* k_new, const pkv_tensor* v_new,
                         const pkv_tensor* k_cache, const pkv_tensor* v_cache, const pkv_tensor* block_tables,
                         const pkv_tensor* context_lens, float scale, float k_scale, float v_scale, void* workspace,
                         size_t workspace_bytes, const pkv_tensor* out, void* stream) {
  if (!k_new) return fail(PKV_ERR_NULL, "k_new: descriptor is NULL");
  if (!v_new) return fail(PKV_ERR_NULL, "v_new: descriptor is NULL");
  return pkv::decode_call(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale,
                          workspace, workspace_bytes, nullptr, out, stream);
}

int pkv_suffix_prefill_attn(const pkv_tensor* q, const pkv_tensor* k_cache, const pkv_tensor* v_cache,
                            const pkv_tensor* block_tables, const pkv_tensor* prefix_lens,
                            const pkv_tensor* suffix_lens, float scale, float k_scale, float v_scale,
                            const pkv_tensor* out, void* stream) {
  return prefill_call(q, k_cache, v_cache, block_tables, prefix_lens, suffix_lens, scale, k_scale, v_scale, nullptr,
                      0, false, out, stream);
}

size_t pkv_suffix_prefill_workspace_bytes(int64_t total_suffix_tokens, int64_t num_requests, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim, int64_t max_blocks_per_seq,
                                          int32_t block_size) {
  if (total_suffix_tokens < 0 || num_requests < 0 || num_q_heads < 1 || num_kv_heads < 1 ||
      num_q_heads % num_kv_heads != 0 || head_dim < 1 || max_blocks_per_seq < 1 || block_size < 1)
    return 0;
  const int parts = prefill_parts(total_suffix_tokens, num_q_heads, num_kv_heads, max_blocks_per_seq, block_size);
  return prefill_ws_bytes(parts, total_suffix_tokens, num_q_heads, head_dim);
}

int pkv_suffix_prefill_attn_split(const pkv_tensor* q, const pkv_tensor* k_cache, const pkv_tensor* v_cache,
                                  const pkv_tensor* block_tables, const pkv_tensor* prefix_lens,
                                  const pkv_tensor* suffix_lens, float scale, float k_scale, float v_scale,
                                  void* workspace, size_t workspace_bytes, const pkv_tensor* out, void* stream) {
  return prefill_call(q, k_cache, v_cache, block_tables, prefix_lens, suffix_lens, scale, k_scale, v_scale,
                      workspace, workspace_bytes, true, out, stream);
}

}  // extern "C"
