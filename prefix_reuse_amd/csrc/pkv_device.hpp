// Device-side helpers shared by the libpkv kernels (gfx950 / CDNA4 only).
//
// Matrix-core conventions used throughout (wave64):
//  * v_mfma_f32_16x16x32_{bf16,f16}: lane l holds A[l%16][8*(l/16) .. +8],
//    B[8*(l/16) .. +8][l%16]; the 16x16 fp32 result D[4*(l/16)+i][l%16] sits
//    in element i of the lane's 4-vector.
//  * v_mfma_f32_16x16x4_f32: lane l holds A[l%16][l/16], B[l/16][l%16]; same
//    result layout.
//  * v_mfma_f32_32x32x16_{bf16,f16}: lane l holds A[l%32][8*(l/32) .. +8],
//    B[8*(l/32) .. +8][l%32]; result D[8*(i/4) + 4*(l/32) + i%4][l%32] in
//    element i of the lane's 16-vector.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16_t;
typedef _Float16 f16_t;

typedef __attribute__((__vector_size__(8 * sizeof(bf16_t)))) bf16_t bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(f16_t)))) f16_t f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(bf16_t)))) bf16_t bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(f16_t)))) f16_t f16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// 8-element fragments of a 16-bit matrix-core operand
// ---------------------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<bf16_t> { typedef bf16x8 type; };
template <> struct Frag<f16_t> { typedef f16x8 type; };
template <> struct Frag<float> { typedef float type; };  // f32 operands are scalars

template <typename T>
__device__ __forceinline__ typename Frag<T>::type load_frag8(const T* p) {
  u32x4 raw = *reinterpret_cast<const u32x4*>(p);
  return __builtin_bit_cast(typename Frag<T>::type, raw);
}

__device__ __forceinline__ u32x4 load_u32x4(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 load_u32x2(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

// ---------------------------------------------------------------------------
// fp8 e4m3fn (OCP) -> 16-bit, exact: every e4m3fn value is representable in
// bf16 and in f16. The gfx950 scaled-convert instructions with scale 1.0 do it
// two bytes at a time (bytes 0-1 with hi=false, bytes 2-3 with hi=true).
// ---------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ typename Frag<T>::type fp8x8_to(u32x2 w);

template <>
__device__ __forceinline__ bf16x8 fp8x8_to<bf16_t>(u32x2 w) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

template <>
__device__ __forceinline__ f16x8 fp8x8_to<f16_t>(u32x2 w) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, false);
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, true);
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, false);
  f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, true);
  f16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// ---------------------------------------------------------------------------
// fp32 -> fp8 e4m3fn with round-to-nearest-even and saturation to +-448.
// Bit manipulation on the IEEE float32 input, no hardware convert (so the
// rounding and clamping rules are exactly the ones written here).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t sign = (u >> 24) & 0x80u;
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fu;  // NaN
  float a = __uint_as_float(u & 0x7fffffffu);
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0.015625f) {  // below 2^-6: subnormal grid, step 2^-9
    // a * 512 is exact; rint rounds half to even; 8 means 2^-6, code 0x08.
    uint32_t m = (uint32_t)__builtin_rintf(a * 512.0f);
    return sign | m;
  }
  int32_t e = (int32_t)((u >> 23) & 0xffu) - 127;  // -6 .. 8
  uint32_t mant = u & 0x7fffffu;
  uint32_t r = mant >> 20;
  uint32_t rem = mant & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
  if (r == 8u) { r = 0u; ++e; }
  uint32_t code = ((uint32_t)(e + 7) << 3) | r;
  if (code > 0x7eu) code = 0x7eu;
  return sign | code;
}

// ---------------------------------------------------------------------------
// Matrix-core wrappers
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Conversions of fp32 results to the storage types
// ---------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float x) { return (f16_t)x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }

template <typename T>
__device__ __forceinline__ typename Frag<T>::type pack8(const float* p) {
  typename Frag<T>::type r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (T)p[j];
  return r;
}

// Work-group index remap so that consecutive logical indices run on the same
// XCD (MI355X has 8 XCDs with private L2s; hardware hands work-groups to XCDs
// round-robin). Logical ranges [k*N/8, (k+1)*N/8) land on XCD k.
__device__ __forceinline__ int xcd_remap(int linear, int total) {
  constexpr int kXcd = 8;
  int xcd = linear % kXcd;
  int idx = linear / kXcd;
  int q = total / kXcd, r = total % kXcd;
  return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

}  // namespace pkv
