/*
 * A consumer of libpkv written in plain C99 against include/pkv.h and
 * include/pkv_prefix.h, with the HIP runtime's C API for device memory: the
 * boundary needs neither C++ nor Python. Test infrastructure, built by
 * prefix_reuse_amd/build.py and run by tests/test_c_abi_host.py (host mode)
 * and tests/test_c_abi_gpu.py (decode mode).
 *
 *   c_abi_consumer host        status codes, errors, the prefix cache and the
 *                              radix tree (no GPU call)
 *   c_abi_consumer decode DIR  reads a decode batch that the test wrote into
 *                              DIR, appends each sequence's newest token
 *                              (pkv_append), runs pkv_decode_attn and writes
 *                              the output to DIR/out.bin
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "pkv.h"
#include "pkv_prefix.h"

#define CHECK(c)                                                             \
  do {                                                                       \
    if (!(c)) {                                                              \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      return 1;                                                              \
    }                                                                        \
  } while (0)

static int host_checks(void) {
  CHECK(pkv_abi_version() == PKV_ABI_VERSION);
  CHECK(pkv_decode_workspace_bytes(0, 4, 3, 64, 4, 16) == 0); /* 4 % 3 != 0 */
  CHECK(pkv_decode_workspace_bytes(3, 8, 2, 64, 4, 16) > 0);

  /* missing tensors are refused before anything is launched */
  CHECK(pkv_append(NULL, NULL, NULL, NULL, NULL, 1.f, 1.f, NULL) == PKV_ERR_NULL);
  CHECK(strlen(pkv_last_error()) > 0);

  /* chain-hash prefix cache: 8 blocks of 4 tokens */
  pkv_prefix_cache* pc = NULL;
  CHECK(pkv_pc_create(8, 4, &pc) == PKV_OK);
  const int32_t tokens[10] = {5, 6, 7, 8, 9, 10, 11, 12, 13, 14};
  int32_t bt1[3], bt2[3], bt3[3];
  int64_t slots1[10], slots2[10], slots3[10];
  int64_t plen = -1, req1 = -1, req2 = -1, req3 = -1, published = -1;
  CHECK(pkv_pc_admit(pc, tokens, 10, 0, 0, bt1, 3, slots1, &plen, &req1) == PKV_OK);
  CHECK(plen == 0);
  for (int i = 0; i < 10; ++i) CHECK(slots1[i] == (int64_t)bt1[i / 4] * 4 + i % 4);
  CHECK(pkv_pc_commit(pc, req1, &published) == PKV_OK);
  CHECK(published == 2); /* the two full blocks */
  /* the same tokens again: both full blocks are reused, the tail is new */
  CHECK(pkv_pc_admit(pc, tokens, 10, 0, 0, bt2, 3, slots2, &plen, &req2) == PKV_OK);
  CHECK(plen == 8);
  CHECK(bt2[0] == bt1[0] && bt2[1] == bt1[1] && bt2[2] != bt1[2]);
  CHECK(slots2[0] == (int64_t)bt2[2] * 4 && slots2[1] == (int64_t)bt2[2] * 4 + 1);
  /* another tenant's salt shares nothing */
  CHECK(pkv_pc_admit(pc, tokens, 10, 7, 0, bt3, 3, slots3, &plen, &req3) == PKV_OK);
  CHECK(plen == 0);
  for (int i = 0; i < 3; ++i) CHECK(bt3[i] != bt1[0] && bt3[i] != bt1[1]);
  int64_t free_blocks = -1, evictable = -1, cached = -1;
  CHECK(pkv_pc_stats(pc, &free_blocks, &evictable, &cached) == PKV_OK);
  CHECK(free_blocks == 8 - 3 - 1 - 3 && evictable == 0 && cached == 2);
  CHECK(pkv_pc_release(pc, req1) == PKV_OK);
  CHECK(pkv_pc_release(pc, req2) == PKV_OK);
  CHECK(pkv_pc_release(pc, req3) == PKV_OK);
  CHECK(pkv_pc_stats(pc, &free_blocks, &evictable, &cached) == PKV_OK);
  CHECK(free_blocks == 6 && evictable == 2 && cached == 2);
  CHECK(pkv_pc_release(pc, req1) == PKV_ERR_NOT_FOUND);
  pkv_pc_destroy(pc);

  /* radix tree at token level */
  pkv_radix* rt = NULL;
  CHECK(pkv_radix_create(1, &rt) == PKV_OK);
  const int32_t a[4] = {1, 2, 3, 4}, b[4] = {1, 2, 3, 9};
  const int64_t va[4] = {10, 11, 12, 13}, vb[4] = {20, 21, 22, 23};
  int64_t got[4], existing = -1, matched = -1, total = -1, evicted = -1;
  CHECK(pkv_radix_insert(rt, a, 4, va, &existing) == PKV_OK && existing == 0);
  CHECK(pkv_radix_match(rt, b, 4, got, &matched) == PKV_OK);
  CHECK(matched == 3 && got[0] == 10 && got[1] == 11 && got[2] == 12);
  CHECK(pkv_radix_insert(rt, b, 4, vb, &existing) == PKV_OK && existing == 3); /* splits the edge */
  CHECK(pkv_radix_total_tokens(rt, &total) == PKV_OK && total == 5);
  /* the least recently used leaf goes first: token 4 (value 13) */
  CHECK(pkv_radix_evict(rt, 1, got, 4, &evicted) == PKV_OK);
  CHECK(evicted == 1 && got[0] == 13);
  CHECK(pkv_radix_total_tokens(rt, &total) == PKV_OK && total == 4);
  pkv_radix_destroy(rt);
  printf("host ok\n");
  return 0;
}

/* ---- decode mode ---- */

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* buf = malloc(bytes ? bytes : 1);
  const size_t n = buf ? fread(buf, 1, bytes, f) : 0;
  fclose(f);
  if (n != bytes) {
    free(buf);
    return NULL;
  }
  return buf;
}

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes ? bytes : 1) != hipSuccess) return NULL;
  if (bytes && hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

static pkv_tensor tensor(void* data, int dtype, int ndim, const int64_t* shape) {
  pkv_tensor t;
  memset(&t, 0, sizeof t);
  t.data = data;
  t.dtype = dtype;
  t.ndim = ndim;
  int64_t stride = 1;
  for (int i = ndim - 1; i >= 0; --i) {
    t.shape[i] = shape[i];
    t.stride[i] = stride;
    stride *= shape[i];
  }
  return t;
}

static int decode(const char* dir) {
  char path[4096];
  snprintf(path, sizeof path, "%s/meta.txt", dir);
  FILE* f = fopen(path, "r");
  CHECK(f != NULL);
  long long S, hq, hkv, d, B, nb, maxb;
  float scale;
  const int got = fscanf(f, "%lld %lld %lld %lld %lld %lld %lld %f", &S, &hq, &hkv, &d, &B, &nb, &maxb, &scale);
  fclose(f);
  CHECK(got == 8);

  const size_t q_bytes = (size_t)(S * hq * d) * 2, cache_bytes = (size_t)(nb * hkv * B * d) * 2;
  const size_t new_bytes = (size_t)(S * hkv * d) * 2;
  void* q = read_file(dir, "q.bin", q_bytes);
  void* kc = read_file(dir, "k_cache.bin", cache_bytes);
  void* vc = read_file(dir, "v_cache.bin", cache_bytes);
  void* kn = read_file(dir, "k_new.bin", new_bytes);
  void* vn = read_file(dir, "v_new.bin", new_bytes);
  void* bt = read_file(dir, "block_tables.bin", (size_t)(S * maxb) * 4);
  void* cl = read_file(dir, "context_lens.bin", (size_t)S * 4);
  void* sm = read_file(dir, "slot_mapping.bin", (size_t)S * 8);
  CHECK(q && kc && vc && kn && vn && bt && cl && sm);

  void* dq = to_device(q, q_bytes);
  void* dkc = to_device(kc, cache_bytes);
  void* dvc = to_device(vc, cache_bytes);
  void* dkn = to_device(kn, new_bytes);
  void* dvn = to_device(vn, new_bytes);
  void* dbt = to_device(bt, (size_t)(S * maxb) * 4);
  void* dcl = to_device(cl, (size_t)S * 4);
  void* dsm = to_device(sm, (size_t)S * 8);
  void* dout = NULL;
  CHECK(dq && dkc && dvc && dkn && dvn && dbt && dcl && dsm);
  CHECK(hipMalloc(&dout, q_bytes) == hipSuccess);

  const int64_t q_shape[3] = {S, hq, d}, new_shape[3] = {S, hkv, d};
  const int64_t k_shape[4] = {nb, hkv, B, d}, v_shape[4] = {nb, hkv, d, B};
  const int64_t bt_shape[2] = {S, maxb}, s_shape[1] = {S};
  const pkv_tensor tq = tensor(dq, PKV_F16, 3, q_shape), tout = tensor(dout, PKV_F16, 3, q_shape);
  const pkv_tensor tkn = tensor(dkn, PKV_F16, 3, new_shape), tvn = tensor(dvn, PKV_F16, 3, new_shape);
  const pkv_tensor tkc = tensor(dkc, PKV_F16, 4, k_shape), tvc = tensor(dvc, PKV_F16, 4, v_shape);
  const pkv_tensor tbt = tensor(dbt, PKV_I32, 2, bt_shape), tcl = tensor(dcl, PKV_I32, 1, s_shape);
  const pkv_tensor tsm = tensor(dsm, PKV_I64, 1, s_shape);

  int rc = pkv_append(&tkn, &tvn, &tsm, &tkc, &tvc, 1.f, 1.f, NULL);
  if (rc != PKV_OK) fprintf(stderr, "pkv_append: %d %s\n", rc, pkv_last_error());
  CHECK(rc == PKV_OK);
  const size_t ws_bytes = pkv_decode_workspace_bytes(S, (int32_t)hq, (int32_t)hkv, (int32_t)d, maxb, (int32_t)B);
  void* ws = NULL;
  CHECK(ws_bytes > 0 && hipMalloc(&ws, ws_bytes) == hipSuccess);
  rc = pkv_decode_attn(&tq, &tkc, &tvc, &tbt, &tcl, scale, 1.f, 1.f, ws, ws_bytes, &tout, NULL);
  if (rc != PKV_OK) fprintf(stderr, "pkv_decode_attn: %d %s\n", rc, pkv_last_error());
  CHECK(rc == PKV_OK);
  CHECK(hipDeviceSynchronize() == hipSuccess);

  void* out = malloc(q_bytes);
  CHECK(out != NULL);
  CHECK(hipMemcpy(out, dout, q_bytes, hipMemcpyDeviceToHost) == hipSuccess);
  snprintf(path, sizeof path, "%s/out.bin", dir);
  f = fopen(path, "wb");
  CHECK(f != NULL);
  CHECK(fwrite(out, 1, q_bytes, f) == q_bytes);
  fclose(f);

  void* dev[] = {dq, dkc, dvc, dkn, dvn, dbt, dcl, dsm, dout, ws};
  for (size_t i = 0; i < sizeof dev / sizeof dev[0]; ++i) CHECK(hipFree(dev[i]) == hipSuccess);
  void* host[] = {q, kc, vc, kn, vn, bt, cl, sm, out};
  for (size_t i = 0; i < sizeof host / sizeof host[0]; ++i) free(host[i]);
  printf("decode ok\n");
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 2 && strcmp(argv[1], "host") == 0) return host_checks();
  if (argc == 3 && strcmp(argv[1], "decode") == 0) return decode(argv[2]);
  fprintf(stderr, "usage: %s host | decode DIR\n", argv[0]);
  return 2;
}
