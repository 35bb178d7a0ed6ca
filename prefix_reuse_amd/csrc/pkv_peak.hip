// Measured ceilings of the chip, for reporting the kernels' fractions against
// what this device actually reaches as well as against its published peaks.
// Built into libpkv_peak.so (not part of libpkv's ABI); bench.py times each
// launch with HIP events on the launch stream.
//
//  pkv_peak_stream_read  every byte of a large buffer read once with 16-byte
//                        loads (the best case for an HBM-bound kernel)
//  pkv_peak_tile_gather  whole 4 KiB tiles read in random order, one wave per
//                        tile, eight waves per compute unit: the access
//                        pattern of the paged decode (one (block, KV head) tile
//                        of K or V per load group)
//  pkv_peak_mfma_bf16    back-to-back v_mfma_f32_32x32x16_bf16 on every SIMD,
//                        four independent accumulators per wave; the first
//                        wave also reads the shader clock counter and the
//                        100 MHz constant counter around its loop, which
//                        gives the shader clock under full matrix load
//
// Each kernel folds what it reads or computes into a value it stores only
// under a condition the inputs never meet, so nothing is optimised away and
// nothing is written in practice. All buffers are the caller's; sizes are
// checked on the host before launch.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                               uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  // four loads in flight per thread
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    const u32x4 x = a ^ b ^ c ^ d;
    acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// One wave per tile at a time; wave w of the grid takes tiles w, w + waves, ...
// of the list. A 4 KiB tile is four 1 KiB wave-wide loads.
__global__ __launch_bounds__(64) void tile_gather_kernel(const char* __restrict__ buf, const int32_t* __restrict__ ids,
                                                         int32_t n_ids, int64_t num_tiles, uint32_t* sink) {
  const int lane = threadIdx.x;
  uint32_t acc = 0;
  for (int32_t t = blockIdx.x; t < n_ids; t += gridDim.x) {
    int64_t id = ids[t];
    id = id < 0 ? 0 : (id >= num_tiles ? num_tiles - 1 : id);
    const u32x4* tile = reinterpret_cast<const u32x4*>(buf + id * 4096);
    const u32x4 a = tile[lane], b = tile[64 + lane], c = tile[128 + lane], d = tile[192 + lane];
    const u32x4 x = a ^ b ^ c ^ d;
    acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

__global__ __launch_bounds__(kThreads) void mfma_bf16_kernel(int32_t iters, uint32_t* sink, uint64_t* clock) {
  const bool stamp = clock != nullptr && blockIdx.x == 0 && threadIdx.x < 64;
  uint64_t t0 = 0, r0 = 0;
  if (stamp) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  const uint32_t seed = threadIdx.x * 2654435761u + blockIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((seed >> i) & 7) * (__bf16)0.125f;
    b[i] = (__bf16)(float)((seed >> (i + 3)) & 7) * (__bf16)0.125f;
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int32_t it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  const f32x16 s = c0 + c1 + c2 + c3;
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) t += s[i];
  if (t == -1.0f) sink[0] = __float_as_uint(t);  // sums of non-negative products: never -1
  if (stamp) {  // the loop's results are summed above, so the stamps follow every product
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
      clock[0] = t1 - t0;  // shader clock cycles
      clock[1] = r1 - r0;  // ticks of the 100 MHz counter
    }
  }
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, buffer 16-byte aligned) once. Returns a
// hipError_t value (0 on success).
int pkv_peak_stream_read(const void* buf, int64_t bytes, void* sink, int32_t blocks, void* stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 != 0 || blocks < 1 || ((uintptr_t)buf & 15u) != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(buf), bytes / 16, static_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}

// Reads the 4 KiB tiles ids[0 .. n_ids) of a buffer of num_tiles tiles (ids
// are clamped into range) with `waves` one-wave work-groups.
int pkv_peak_tile_gather(const void* buf, int64_t num_tiles, const int32_t* ids, int32_t n_ids, void* sink,
                         int32_t waves, void* stream) {
  if (!buf || !ids || !sink || num_tiles < 1 || n_ids < 0 || waves < 1 || ((uintptr_t)buf & 15u) != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(tile_gather_kernel, dim3(waves), dim3(64), 0, (hipStream_t)stream,
                     static_cast<const char*>(buf), ids, n_ids, num_tiles, static_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}

// `blocks` work-groups of 4 waves, each wave issuing 4 * iters matrix
// products of 32x32x16 (32,768 FLOP each). clock (nullable, two uint64):
// the first wave's shader clock cycles and 100 MHz ticks over its loop.
int pkv_peak_mfma_bf16(int32_t blocks, int32_t iters, void* sink, void* clock, void* stream) {
  if (!sink || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, iters,
                     static_cast<uint32_t*>(sink), static_cast<uint64_t*>(clock));
  return (int)hipGetLastError();
}

}  // extern "C"
