// Append new tokens' K and V rows to their cache slots (page "KV Cache에 대해
// 알아보자 (Feat. Attention)" §3: the new token's K, V are added to the cache;
// page "PagedAttention과 RadixAttention으로 LLM KV 캐시 최적화" §02: the slot
// is physical block * B + offset, chosen by the block table).
//
// The grid has two parts. In the first, one thread moves 8 consecutive dims
// of one (token, KV head) row of K: a 16-byte (16-bit rows) or 32-byte (f32)
// read and one contiguous store into its [B][d] tile, so a wave writes whole
// rows. In the second, one thread moves 8 dims of one token's V row into its
// [d][B] tile: 8 stores one token-column apart. There the token index varies
// fastest across the lanes, so when consecutive rows go to consecutive slots
// (a suffix being appended) the lanes' stores to one V^T row are adjacent and
// the wave writes runs of a row instead of isolated elements. For an fp8
// cache each value is divided by the scale in float32 and rounded to e4m3fn
// (nearest, ties to even, saturating).
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

#include <type_traits>

namespace pkv {
namespace {

constexpr int kThreads = 256;

template <typename TR, typename TC, int D, int BLK>
__device__ __forceinline__ int64_t slot_of(const AppendParams& p, int64_t tok) {
  const int64_t slot = p.slots_i64 ? reinterpret_cast<const int64_t*>(p.slots)[tok]
                                   : (int64_t)reinterpret_cast<const int32_t*>(p.slots)[tok];
  return (slot < 0 || slot >= (int64_t)p.num_blocks * BLK) ? -1 : slot;
}

template <typename TR, typename TC, int D, int BLK>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendParams p, int64_t k_threads) {
  constexpr int kPieces = D / 8;
  int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool v_part = gid >= k_threads;  // uniform per work-group: k_threads is a multiple of kThreads
  int64_t tok;
  int h, d0;
  if (!v_part) {  // [token][head][piece]: a wave covers whole K rows
    const int64_t per_token = (int64_t)p.hkv * kPieces;
    tok = gid / per_token;
    const int rem = (int)(gid % per_token);
    h = rem / kPieces;
    d0 = (rem % kPieces) * 8;
  } else {  // [head][piece][token]: a wave covers consecutive tokens
    gid -= k_threads;
    tok = gid % p.num_tokens;
    const int64_t rem = gid / p.num_tokens;
    h = (int)(rem / kPieces);
    d0 = (int)(rem % kPieces) * 8;
    if (h >= p.hkv) return;
  }
  if (tok >= p.num_tokens) return;
  const int64_t slot = slot_of<TR, TC, D, BLK>(p, tok);
  if (slot < 0) return;
  const int64_t blk = slot / BLK;
  const int off = (int)(slot % BLK);
  const int64_t tile = (blk * p.hkv + h) * (int64_t)(BLK * D);

  if (!v_part) {
    const TR* ksrc = reinterpret_cast<const TR*>(p.k) + tok * p.k_s0 + h * p.k_s1 + d0;
    TC* kdst = reinterpret_cast<TC*>(p.k_cache) + tile + (int64_t)off * D + d0;
    if constexpr (std::is_same<TC, uint8_t>::value) {
      // quantize: code = e4m3fn(x / scale), float32 IEEE division
      float kx[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) kx[j] = to_f32(ksrc[j]);
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lo |= f32_to_e4m3fn(kx[j] / p.k_scale) << (8 * j);
        hi |= f32_to_e4m3fn(kx[j + 4] / p.k_scale) << (8 * j);
      }
      *reinterpret_cast<u32x2*>(kdst) = u32x2{lo, hi};
    } else {
      static_assert(std::is_same<TR, TC>::value, "non-fp8 caches copy rows bit for bit");
      *reinterpret_cast<u32x4*>(kdst) = *reinterpret_cast<const u32x4*>(ksrc);
      if constexpr (sizeof(TC) == 4)  // f32 rows: 32 bytes
        *reinterpret_cast<u32x4*>(kdst + 4) = *reinterpret_cast<const u32x4*>(ksrc + 4);
    }
    return;
  }
  const TR* vsrc = reinterpret_cast<const TR*>(p.v) + tok * p.v_s0 + h * p.v_s1 + d0;
  TC* vdst = reinterpret_cast<TC*>(p.v_cache) + tile + (int64_t)d0 * BLK + off;
  if constexpr (std::is_same<TC, uint8_t>::value) {
    float vx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) vx[j] = to_f32(vsrc[j]);
#pragma unroll
    for (int j = 0; j < 8; ++j) vdst[(int64_t)j * BLK] = (uint8_t)f32_to_e4m3fn(vx[j] / p.v_scale);
  } else {
    TC vv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) vv[j] = vsrc[j];
#pragma unroll
    for (int j = 0; j < 8; ++j) vdst[(int64_t)j * BLK] = vv[j];
  }
}

template <typename TR, typename TC, int D, int BLK>
hipError_t launch_typed(const AppendParams& p, hipStream_t stream) {
  const int64_t threads = p.num_tokens * p.hkv * (D / 8);  // per part
  if (threads == 0) return hipSuccess;
  const int64_t part_blocks = (threads + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((append_kernel<TR, TC, D, BLK>), dim3((unsigned)(2 * part_blocks)), dim3(kThreads), 0, stream, p,
                     part_blocks * kThreads);
  return hipGetLastError();
}

template <typename TR, typename TC>
hipError_t launch_shape(const AppendParams& p, int d, int b, hipStream_t s) {
  if (d == 128 && b == 16) return launch_typed<TR, TC, 128, 16>(p, s);
  if (d == 128 && b == 32) return launch_typed<TR, TC, 128, 32>(p, s);
  if (d == 64 && b == 16) return launch_typed<TR, TC, 64, 16>(p, s);
  if (d == 64 && b == 32) return launch_typed<TR, TC, 64, 32>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_append(const AppendParams& p, DT row_dt, DT cache_dt, int d, int b, hipStream_t s) {
  if (cache_dt == DT::FP8) {
    if (row_dt == DT::F32) return launch_shape<float, uint8_t>(p, d, b, s);
    if (row_dt == DT::F16) return launch_shape<f16_t, uint8_t>(p, d, b, s);
    if (row_dt == DT::BF16) return launch_shape<bf16_t, uint8_t>(p, d, b, s);
    return hipErrorInvalidValue;
  }
  if (row_dt != cache_dt) return hipErrorInvalidValue;
  if (row_dt == DT::F32) return launch_shape<float, float>(p, d, b, s);
  if (row_dt == DT::F16) return launch_shape<f16_t, f16_t>(p, d, b, s);
  if (row_dt == DT::BF16) return launch_shape<bf16_t, bf16_t>(p, d, b, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv
