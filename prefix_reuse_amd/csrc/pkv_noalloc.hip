// pkv_decode_attn_noalloc: the paged decode of pkv_decode_attn for callers
// that cannot allocate device memory (code under HIP graph capture, serving
// loops without an allocator, harnesses that forbid it). The partial results
// that pkv_decode_attn keeps in the caller's workspace live here in a
// device-resident array of fixed size, one copy per GPU, held until the
// process ends. No call in this file allocates or frees memory.
#include "pkv_internal.hpp"
#include "pkv_status.hpp"

#include <atomic>
#include <cstdio>
#include <mutex>

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per GPU

// Each GPU the library runs on holds its own copy. In host code `scratch` is
// a stand-in for the symbol, not a device address: kernels get the address
// that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The scratch array's address on the current device, looked up once per
// device (with that device current) on its first call.
int device_scratch(size_t need, void** ptr) {
  char msg[256];
  if (need > kScratchBytes) {
    snprintf(msg, sizeof(msg),
             "pkv_decode_attn_noalloc: this batch needs %zu bytes of scratch but the device-resident scratch "
             "holds %zu; use pkv_decode_attn with a workspace",
             need, kScratchBytes);
    return pkv::record_status(PKV_ERR_WORKSPACE, msg);
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    snprintf(msg, sizeof(msg), "pkv_decode_attn_noalloc: no usable current device (%s)", hipGetErrorString(e));
    return pkv::record_status(PKV_ERR_HIP, msg);
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) {
        snprintf(msg, sizeof(msg), "pkv_decode_attn_noalloc: scratch address lookup failed (%s)",
                 hipGetErrorString(e));
        return pkv::record_status(PKV_ERR_HIP, msg);
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return PKV_OK;
}

}  // namespace

extern "C" int pkv_decode_attn_noalloc(const pkv_tensor* q, const pkv_tensor* k_cache, const pkv_tensor* v_cache,
                                       const pkv_tensor* block_tables, const pkv_tensor* context_lens, float scale,
                                       float k_scale, float v_scale, const pkv_tensor* out, void* stream) {
  return pkv::decode_call(q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
                          v_scale, nullptr, 0, device_scratch, out, stream);
}
