// Device code of the suffix-prefill attention (one work-group of 8 waves per
// row tile), shared by the prefill kernel and the cascade kernel.
#pragma once
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

#include <math.h>
#include <type_traits>

namespace pkv {
namespace {

constexpr int kWaves = kPrefillWaves;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsWave = 32;
constexpr int kRowsWg = kRowsWave * kWaves;
constexpr int kStage = 64;     // keys per LDS stage = two 32-key sub-tiles
constexpr int kRing = 4;       // LDS buffers per operand (stage s lives in buffer s % kRing)
constexpr float kLazy = 8.0f;  // log2 headroom before the running max moves
// bf16 cache, fast pass: the full steps take no row maximum. A row's max moves
// only once one of its P values passes kPCap, seen as a lane's 16 P values
// summing past 16 kPCap (each P then stays far inside f16 range).
constexpr float kPCap = 64.0f;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(4))) const int32_t sconst_i32;  // read with scalar loads

// ---- LDS tile layouts (element offsets), XOR swizzles of 16-byte pieces ----
// K: [kStage keys][D] in the Q type; piece = 8 dims.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  if constexpr (D == 128) return (row & 7) | (((row >> 4) & 1) << 3);
  else return ((row >> 1) & 3) | (((row >> 4) & 1) << 2);
}
template <int D>
__device__ __forceinline__ int k_off(int row, int piece) {  // piece in [0, D/8)
  return row * D + ((piece ^ k_swz<D>(row)) << 3);
}
// V^T: one [D][BLK] tile per cache block of the stage, block-major, exactly as
// the cache stores it; piece = 8 keys, swizzled within the tile's rows.
template <int D, int BLK>
__device__ __forceinline__ int v_off(int blk, int d, int piece) {  // piece in [0, BLK/8)
  constexpr int kPpr = BLK / 8;
  constexpr int kSh = kPpr == 2 ? 3 : 2;
  return (blk * D + d) * BLK + ((piece ^ ((d >> kSh) & (kPpr - 1))) << 3);
}

__device__ __forceinline__ int sel4(int b0, int b1, int b2, int b3, int i) {  // i uniform
  return i < 2 ? (i == 0 ? b0 : b1) : (i == 2 ? b2 : b3);
}

// A wave-uniform address kept in scalar registers, so that a load can add a
// 32-bit per-lane offset to it without vector 64-bit arithmetic.
__device__ __forceinline__ const char* uniform_ptr(const void* base, int64_t off) {
  const uint64_t b = (uint64_t)base + (uint64_t)off;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}

// One wave-wide direct-to-LDS load of 16 bytes per lane: lane l reads
// base + voff and writes LDS bytes lds + 16l .. +15 (base and lds uniform).
// Issued as inline assembly so that the compiler does not see it: its own
// wait insertion would otherwise drain every direct load in flight before each
// LDS read, because it cannot tell which buffer a load writes. The kernel
// orders these loads itself with explicit waits before its barriers.
// The LDS destination travels in m0, a register the compiler reserves: the
// block saves m0 and restores it after the load has been issued (the load
// reads m0 at issue), so whatever the compiler keeps there survives. On the
// GFX9 family a load that takes its LDS address from m0 must not directly
// follow the scalar write of m0: one wait state (s_nop 0) separates them.
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(base)
      : "memory");
}
// Work-group barrier that is also a compiler memory barrier: no LDS (or
// other memory) access is moved across it, in either direction. Its wait is
// the caller's explicit s_waitcnt, which the compiler's own wait insertion
// sees and accounts for.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ uint32_t lds_address(const char* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p);
}

// kFast: a bf16 cache's values are converted to f16 in LDS (exact for
// 2^-17 <= |v| < 65520; smaller values land in f16's subnormal range, within
// 2^-25 absolute; f16 P carries 11 bits, as with an f16 cache); a work-group
// that meets a larger or non-finite value redoes its rows without it.
template <typename TQ, typename TC, bool kFast>
struct Types {
  static constexpr bool kFp8 = std::is_same<TC, uint8_t>::value;
  static constexpr bool kConvV = kFast && std::is_same<TC, bf16_t>::value;
  // PV operand type: the cache's own 16-bit type, f16 for an fp8 cache or a
  // converted bf16 one
  typedef typename std::conditional<kFp8 || kConvV, f16_t, TC>::type VOp;
  static constexpr bool kSplitP = std::is_same<VOp, bf16_t>::value;
};

// Physical block ids of the kStage/BLK blocks of one stage (plain ints:
// arrays here end up in scratch). Scalar loads; entries past the last live
// block repeat it. load_ids_raw only issues the loads, so that their latency
// can pass under a barrier's wait; clamp_ids then bounds the ids to the pool.
struct Ids {
  int b0, b1, b2, b3;
};
template <int BLK>
__device__ __forceinline__ Ids load_ids_raw(const int32_t* bt, int st, int last) {
  constexpr int kB = kStage / BLK;
  const sconst_i32* t = (const sconst_i32*)bt;
  int v[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < kB; ++i) v[i] = t[min(st * kB + i, last)];
  return Ids{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ Ids clamp_ids(Ids r, int num_blocks) {
  auto c = [&](int v) { return min(max(v, 0), num_blocks - 1); };
  return Ids{c(r.b0), c(r.b1), c(r.b2), c(r.b3)};
}
template <int BLK>
__device__ __forceinline__ Ids load_ids(const int32_t* bt, int st, int last, int num_blocks) {
  return clamp_ids(load_ids_raw<BLK>(bt, st, last), num_blocks);
}

// 16-bit caches: every load is one wave-wide global_load_lds of 1 KB that
// lies inside a single cache block, so its address is a scalar block base
// plus a per-lane offset fixed for the whole kernel, and its LDS destination
// is a contiguous 1 KB (lane l writes bytes 16l .. 16l+15).
template <int D, int BLK>
struct Dma {
  static constexpr int kKeysPerInst = 1024 / (D * 2);            // K rows per load
  static constexpr int kKInst = kStage / kKeysPerInst / kWaves;    // K loads per wave per stage
  static constexpr int kChunks = D * BLK * 2 / 1024;             // 1 KB pieces of a V tile
  static constexpr int kVInst = D * kStage * 2 / 1024 / kWaves;    // V loads per wave per stage
  static constexpr int kPpr = BLK / 8;
  static constexpr int kSh = kPpr == 2 ? 3 : 2;
  static constexpr int kRowsPerChunk = 1024 / (BLK * 2);
  uint32_t koff[kKInst], voff[kVInst];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kKInst; ++i) {
      const int r = (i * kWaves + wave) * kKeysPerInst + lane / (D / 8);
      const int piece = (lane % (D / 8)) ^ k_swz<D>(r);
      koff[i] = (uint32_t)(((r % BLK) * D + piece * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < kVInst; ++i) {
      const int c = i * kWaves + wave;
      const int d = (c % kChunks) * kRowsPerChunk + lane / kPpr;
      const int piece = (lane % kPpr) ^ ((d >> kSh) & (kPpr - 1));
      voff[i] = (uint32_t)((d * BLK + piece * 8) * 2);
    }
  }
  __device__ __forceinline__ void issue_k(const void* cache, int64_t bstride, int64_t hoff, Ids ids, char* dst,
                                          int wave) const {
#pragma unroll
    for (int i = 0; i < kKInst; ++i) {
      const int r0 = (i * kWaves + wave) * kKeysPerInst;
      const int bid = sel4(ids.b0, ids.b1, ids.b2, ids.b3, r0 / BLK);
      const char* base = uniform_ptr(cache, (int64_t)bid * bstride + hoff);
      dma16(base, koff[i], lds_address(dst + r0 * D * 2));
    }
  }
  __device__ __forceinline__ void issue_v(const void* cache, int64_t bstride, int64_t hoff, Ids ids, char* dst,
                                          int wave) const {
#pragma unroll
    for (int i = 0; i < kVInst; ++i) {
      const int c = i * kWaves + wave;
      const int bid = sel4(ids.b0, ids.b1, ids.b2, ids.b3, c / kChunks);
      const char* base = uniform_ptr(cache, (int64_t)bid * bstride + hoff);
      dma16(base, voff[i], lds_address(dst + c * 1024));
    }
  }
};

// fp8 caches: 16-code pieces staged through registers and converted exactly
// (K to the Q type, V to f16) when written to LDS.
template <typename TQ, int D, int BLK>
struct Fp8Stage {
  static constexpr int kPieces = kStage * D / 16;               // per stage, K and V alike
  static constexpr int kP = (kPieces + kThreads - 1) / kThreads;  // pieces per thread
  static constexpr int kPiecesPerTile = D * BLK / 16;
  u32x4 kr[kP], vr[kP];

  __device__ __forceinline__ void issue_k(const uint8_t* cache, int64_t bstride, int64_t hoff, Ids ids,
                                          int tid) {
#pragma unroll
    for (int i = 0; i < kP; ++i) {
      const int pi = tid + kThreads * i;
      if (kPieces % kThreads != 0 && pi >= kPieces) break;
      const int row = pi / (D / 16), q = pi % (D / 16);
      const int bid = sel4(ids.b0, ids.b1, ids.b2, ids.b3, __builtin_amdgcn_readfirstlane(row / BLK));
      kr[i] = load_u32x4(cache + (int64_t)bid * bstride + hoff + (row % BLK) * D + q * 16);
    }
  }
  __device__ __forceinline__ void issue_v(const uint8_t* cache, int64_t bstride, int64_t hoff, Ids ids,
                                          int tid) {
#pragma unroll
    for (int i = 0; i < kP; ++i) {
      const int pi = tid + kThreads * i;
      if (kPieces % kThreads != 0 && pi >= kPieces) break;
      const int tile = pi / kPiecesPerTile, rem = pi % kPiecesPerTile;
      const int d = rem / (BLK / 16), h = rem % (BLK / 16);
      const int bid = sel4(ids.b0, ids.b1, ids.b2, ids.b3, __builtin_amdgcn_readfirstlane(tile));
      vr[i] = load_u32x4(cache + (int64_t)bid * bstride + hoff + d * BLK + h * 16);
    }
  }
  __device__ __forceinline__ void commit_k(TQ* k_lds, int tid) const {
    typedef typename Frag<TQ>::type F;
#pragma unroll
    for (int i = 0; i < kP; ++i) {
      const int pi = tid + kThreads * i;
      if (kPieces % kThreads != 0 && pi >= kPieces) break;
      const int row = pi / (D / 16), q = pi % (D / 16);
      const u32x2 lo = {kr[i][0], kr[i][1]}, hi = {kr[i][2], kr[i][3]};
      *reinterpret_cast<F*>(k_lds + k_off<D>(row, 2 * q)) = fp8x8_to<TQ>(lo);
      *reinterpret_cast<F*>(k_lds + k_off<D>(row, 2 * q + 1)) = fp8x8_to<TQ>(hi);
    }
  }
  __device__ __forceinline__ void commit_v(f16_t* v_lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kP; ++i) {
      const int pi = tid + kThreads * i;
      if (kPieces % kThreads != 0 && pi >= kPieces) break;
      const int tile = pi / kPiecesPerTile, rem = pi % kPiecesPerTile;
      const int d = rem / (BLK / 16), h = rem % (BLK / 16);
      const u32x2 lo = {vr[i][0], vr[i][1]}, hi = {vr[i][2], vr[i][3]};
      // exact: every e4m3fn value is an f16 value
      *reinterpret_cast<f16x8*>(v_lds + v_off<D, BLK>(tile, d, 2 * h)) = fp8x8_to<f16_t>(lo);
      *reinterpret_cast<f16x8*>(v_lds + v_off<D, BLK>(tile, d, 2 * h + 1)) = fp8x8_to<f16_t>(hi);
    }
  }
};

// P^T fragments of one 32-key sub-tile: the B operands of the two PV steps,
// as rounded values and (bf16 only) the rounding remainders.
template <typename FV>
struct PFrag {
  FV hi[2], lo[2];
};

// LDS of a work-group: kRing K stages and kRing V stages, 16-bit elements
template <int D>
constexpr int kLdsBytes = kRing * 2 * kStage * D * 2;

// The rows of one work-group. Returns false (having written nothing) when a
// kFast pass met a value it cannot convert; the caller then runs the exact pass.
// kSplit: the suffix prefill with its keys split over several work-groups per
// row tile (see below); each writes an unnormalised partial for the merge.
template <typename TQ, typename TC, int D, int BLK, bool kFast, bool kCasc, bool kSplit>
__device__ __forceinline__ bool attend(const PrefillParams& p, char* lds, int wg) {
  typedef Types<TQ, TC, kFast> T;
  typedef typename T::VOp VOp;
  typedef typename Frag<TQ>::type F;
  typedef typename Frag<VOp>::type FV;
  constexpr int QS = D / 16;  // k-steps of the score product
  constexpr int NT = D / 32;  // dim tiles of the output
  constexpr int kKBytes = kStage * D * (int)sizeof(TQ);
  constexpr int kVBytes = kStage * D * (int)sizeof(VOp);
  static_assert(kRing * (kKBytes + kVBytes) == kLdsBytes<D>, "LDS budget");
  char* const k_lds0 = lds;                    // K stages: buffers 0 .. kRing-1
  char* const v_lds0 = lds + kRing * kKBytes;  // V stages: buffers 0 .. kRing-1

  // ---- which (KV head, request, row tile) ----
  const int logical = xcd_remap(wg, p.hkv * p.tiles_per_head);
  const int hk = logical / p.tiles_per_head;
  int tile = logical % p.tiles_per_head;
  // cascade decode's shared part (the requests are groups of sequences) and
  // the key-split prefill: key_splits work-groups share a row tile, each on
  // one part of the keys
  constexpr bool casc = kCasc;  // a kernel of its own: the suffix prefill carries none of it
  int split = 0;
  if (casc || kSplit) {
    split = tile % p.key_splits;
    tile /= p.key_splits;
  }
  int r = p.num_reqs, row_base = 0, rows_r = 0;
  if constexpr (kCasc) {
    // the cascade's groups, one after the other (the fused kernel also holds
    // the decode waves, and the search below costs it registers)
    r = 0;
    for (; r < p.num_reqs; ++r) {
      int s = p.group_starts[r + 1] - p.group_starts[r];
      s = s < 0 ? 0 : s;
      if (row_base + s > p.total_rows) s = (int)(p.total_rows - row_base);
      rows_r = s * p.group;
      const int nt = (rows_r + kRowsWg - 1) / kRowsWg;
      if (tile < nt) break;
      tile -= nt;
      row_base += s;
    }
  } else {
    // which request this tile belongs to: 64 requests at a time, one per
    // lane, with prefix sums of their (clamped) row counts and tile counts
    // across the wave; the first request whose tile range holds `tile` wins.
    // One round trip instead of one dependent load per earlier request.
    const int ln = (int)(threadIdx.x % 64);
    int64_t rows_before = 0;  // rows of the requests before this batch (at most total_rows)
    int tiles_before = 0;
    for (int r0 = 0; r0 < p.num_reqs; r0 += 64) {
      const int rr = r0 + ln;
      // device lengths are not trusted: each is cut to [0, total_rows] and
      // summed in 64 bits, so no sum can wrap
      int64_t s = 0;
      if (rr < p.num_reqs) s = p.suffix_lens[rr];
      s = s < 0 ? 0 : (s > p.total_rows ? p.total_rows : s);
      int64_t incl = s;  // inclusive prefix sum of s over the lanes
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int64_t t = __shfl_up(incl, off);
        if (ln >= off) incl += t;
      }
      // the running row count is cut at total_rows, so each request keeps
      // what is left of it
      const int64_t rb = min(rows_before + (incl - s), p.total_rows);
      const int64_t re = min(rows_before + incl, p.total_rows);
      const int rows = (int)(re - rb) * p.group;
      const int nt = (rows + kRowsWg - 1) / kRowsWg;
      int tincl = nt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(tincl, off);
        if (ln >= off) tincl += t;
      }
      const int t0 = tiles_before + tincl - nt;
      const uint64_t hit = __ballot(rr < p.num_reqs && tile >= t0 && tile < t0 + nt);
      if (hit) {
        const int L = __builtin_ctzll(hit);
        r = r0 + L;
        row_base = (int)__builtin_amdgcn_readlane((int)rb, L);
        rows_r = __builtin_amdgcn_readlane(rows, L);
        tile -= __builtin_amdgcn_readlane(t0, L);
        break;
      }
      rows_before = min(rows_before + __shfl(incl, 63), p.total_rows);
      tiles_before += __builtin_amdgcn_readlane(tincl, 63);
    }
  }
  if (r >= p.num_reqs) return true;
  const int S = rows_r / p.group;
  const int cap = p.max_blocks * BLK;
  int P, kv_len, k0 = 0;
  bool prefix_part = false;  // kSplit: a chunk of the prefix, no mask
  const int32_t* bt;
  if (casc) {  // the group's shared prefix, whole blocks, through its first sequence's table
    P = p.shared_lens[row_base];
    P = P < 0 ? 0 : (P > cap ? cap : P);
    P -= P % BLK;
    const int chunk = cascade_chunk(P, p.key_splits);
    k0 = split * chunk;  // this work-group's keys: k0 .. k0 + kv_len - 1
    kv_len = max(min(P - k0, chunk), 0);
    bt = p.block_tables + (int64_t)row_base * p.bt_s0 + (kv_len > 0 ? k0 / BLK : 0);
  } else {
    // the prefix is cut to the table's capacity before the suffix is added:
    // cap <= 2^29 and S <= 2^30 (both checked on the host), so P + S and
    // every P + i below stay inside int
    P = p.prefix_lens[r];
    P = P < 0 ? 0 : (P > cap ? cap : P);
    kv_len = P + S;
    if (kv_len > cap) kv_len = cap;
    bt = p.block_tables + (int64_t)r * p.bt_s0;
    if constexpr (kSplit) {
      // parts 0 .. key_splits-2 take chunks of the prefix's whole stages,
      // which every suffix row sees in full (no mask); the last part takes
      // the keys after them, causally, as the unsplit kernel would, with the
      // table and the prefix length shifted past the chunks
      const int nsplit = p.key_splits - 1;
      const int Ps = split_prefix_keys(P);
      if (split < nsplit) {
        const int chunk = cascade_chunk(Ps, nsplit);
        k0 = split * chunk;  // this work-group's keys: k0 .. k0 + kv_len - 1
        kv_len = max(min(Ps - k0, chunk), 0);
        if (kv_len > 0) bt += k0 / BLK;
        prefix_part = true;
      } else {
        P -= Ps;
        kv_len -= Ps;
        bt += Ps / BLK;
      }
    }
  }

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int h0 = lane / 32, c32 = lane % 32;

  const int q0 = tile * kRowsWg;  // first row of the work-group
  const int tok_last_wg = min(S - 1, (q0 + kRowsWg - 1) / p.group);
  const int wq0 = q0 + wave * kRowsWave;  // first row of this wave
  const int tok_first_w = wq0 / p.group;
  const int tok_last_w = min(S - 1, (wq0 + kRowsWave - 1) / p.group);
  const bool wave_active = wq0 < rows_r;
  // cascade: a sequence shorter than the shared prefix sees only its own
  // tokens of it; ctx_row is the lane row's key count
  int ctx_row = kv_len;
  if (casc && wq0 + (int)(threadIdx.x % 32) < rows_r) {
    int c = p.context_lens[row_base + (wq0 + (int)(threadIdx.x % 32)) / p.group] - k0;
    ctx_row = c < 0 ? 0 : (c < kv_len ? c : kv_len);
  }
  const bool nc = casc || prefix_part;  // every row sees all of this work-group's keys (up to ctx_row)
  int ctx_min_w = ctx_row;
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) ctx_min_w = min(ctx_min_w, __shfl_xor(ctx_min_w, off));
  const int keys_wg = nc ? kv_len : min(kv_len, P + tok_last_wg + 1);
  const int nst = (keys_wg + kStage - 1) / kStage;
  const int keys_w = wave_active ? (nc ? kv_len : min(kv_len, P + tok_last_w + 1)) : 0;
  const int nsub = (keys_w + 31) / 32;  // 32-key sub-tiles of this wave
  // keys below need no mask in this wave
  const int full_keys_w = nc ? __builtin_amdgcn_readfirstlane(ctx_min_w) : min(P + tok_first_w + 1, kv_len);
  if (nst == 0) return true;  // uniform over the work-group

  // ---- Q^T fragments for this lane's row ----
  const int row = wq0 + c32;
  const bool rvalid = row < rows_r;
  const int tok = rvalid ? row / p.group : 0;
  const int qh = hk * p.group + (rvalid ? row % p.group : 0);
  const TQ* qrow = reinterpret_cast<const TQ*>(p.q) + (int64_t)(row_base + tok) * p.q_s0 + (int64_t)qh * p.q_s1;
  // the kernel's score scale c2 is positive: a negative softmax scale is
  // applied by negating q (exact), a zero one by zeroing it (every score 0)
  auto qfrag = [&](int c) -> F {
    F v = {};
    if (rvalid) v = load_frag8(qrow + 16 * c + 8 * h0);
    if (p.q_mode != 0) {
      const uint32_t keep = p.q_mode == 1 ? ~0u : 0u;
      u32x4 w = __builtin_bit_cast(u32x4, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (w[e] & keep) ^ (keep & 0x80008000u);
      v = __builtin_bit_cast(F, w);
    }
    return v;
  };
  // The fragments stay in registers, except in the exact pass of a bf16
  // cache, which reads them again for each score product (and, in its steps,
  // reads the K operands only after the value products): that pass runs only
  // for a work-group that met a V value beyond f16 range, and with these
  // registers freed both passes fit in one kernel with no scratch.
  F qf[QS];
  if constexpr (!T::kSplitP) {
#pragma unroll
    for (int c = 0; c < QS; ++c) qf[c] = qfrag(c);
  }
  const int lim = nc ? ctx_row - 1 : P + tok;  // last key position this row may see
  const float c2 = p.qk_scale_log2;

  // LDS byte addresses of this lane's operands (buffer 0, sub-tile 0)
  // score A operand: permuted key row so that each lane ends up with 16
  // consecutive keys of one row - the B operand of the PV product
  const int krow = 16 * ((c32 % 8) / 4) + 4 * (c32 / 8) + (c32 % 4);
  // k-step c reads piece (2c + h0) ^ swz of row krow, i.e. byte address
  // kx ^ 32c: the swizzle's upper bits permute whole 32-byte piece pairs
  const int kx = k_off<D>(krow, h0) * (int)sizeof(TQ);
  static_assert(sizeof(TQ) == 2, "16-bit score operands");
  // PV A operand, step u of a sub-tile: dim 32n + c32, keys 16*h0 + 8u .. +8
  int vaddr[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if constexpr (BLK == 16) vaddr[u] = v_off<D, BLK>(h0, c32, u) * (int)sizeof(VOp);  // block 2t + h0
    else vaddr[u] = v_off<D, BLK>(0, c32, 2 * h0 + u) * (int)sizeof(VOp);               // block t
  }
  // byte distance between sub-tiles t = 0 and 1 of a stage, and between dim tiles
  constexpr int kKSub = 32 * D * (int)sizeof(TQ);
  constexpr int kVSub = (BLK == 16 ? 2 : 1) * D * BLK * (int)sizeof(VOp);
  constexpr int kVDim = 32 * BLK * (int)sizeof(VOp);

  // ---- loaders ----
  const int64_t tile_bytes = (int64_t)BLK * D * (int64_t)sizeof(TC);
  const int64_t bstride = (int64_t)p.hkv * tile_bytes;
  const int64_t hoff = (int64_t)hk * tile_bytes;
  const int last_blk = min((kv_len - 1) / BLK, p.max_blocks - 1);
  typedef typename std::conditional<T::kFp8, Fp8Stage<TQ, D, BLK>, Dma<D, BLK>>::type Loader;
  Loader ld;
  if constexpr (!T::kFp8) ld.init(wave, lane);
  auto issue_k = [&](int st, Ids ids) {
    char* dst = k_lds0 + (st % kRing) * kKBytes;
    if constexpr (T::kFp8) {
      ld.issue_k(reinterpret_cast<const uint8_t*>(p.k_cache), bstride, hoff, ids, tid);
      (void)dst;
    } else {
      ld.issue_k(p.k_cache, bstride, hoff, ids, dst, wave);
    }
  };
  auto issue_v = [&](int st, Ids ids) {
    char* dst = v_lds0 + (st % kRing) * kVBytes;
    if constexpr (T::kFp8) {
      ld.issue_v(reinterpret_cast<const uint8_t*>(p.v_cache), bstride, hoff, ids, tid);
      (void)dst;
    } else {
      ld.issue_v(p.v_cache, bstride, hoff, ids, dst, wave);
    }
  };
  // fp8: write the staged pieces of K stage `sk` and V stage `sv` (-1: none)
  auto commit = [&](int sk, int sv) {
    if constexpr (T::kFp8) {
      if (sk >= 0) ld.commit_k(reinterpret_cast<TQ*>(k_lds0 + (sk % kRing) * kKBytes), tid);
      if (sv >= 0) ld.commit_v(reinterpret_cast<f16_t*>(v_lds0 + (sv % kRing) * kVBytes), tid);
    }
  };

  // ---- per-row softmax state and accumulators ----
  f32x16 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;  // finite start: -inf - (-inf) would be NaN

  // ---- per-step pieces ----
  // operands of one step, read from LDS before the softmax so that their
  // latency is hidden behind it
  struct VOps {
    FV v[2][NT];
  };
  struct KOps {
    F k[QS];
  };
  // K^T operands of sub-tile t of the stage in K buffer `buf`; k-step c reads
  // piece (2c + h0) ^ swz of the lane's key row, i.e. byte address kx ^ 32c
  auto load_k = [&](int buf, int t, KOps& ko) {
    const char* kl = k_lds0 + buf * kKBytes + t * kKSub;
#pragma unroll
    for (int c = 0; c < QS; ++c) ko.k[c] = *reinterpret_cast<const F*>(kl + (kx ^ (c << 5)));
  };
  // V^T operands of sub-tile t of the stage in V buffer `buf`
  auto load_v = [&](int buf, int t, VOps& vo) {
    const char* vl = v_lds0 + buf * kVBytes + t * kVSub;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int n = 0; n < NT; ++n) vo.v[u][n] = *reinterpret_cast<const FV*>(vl + vaddr[u] + n * kVDim);
  };
  // values of keys >= kv_len are zeroed: the loads brought whatever those
  // cache slots hold, and 0 * NaN would be NaN
  auto zero_tail = [&](VOps& vo, int key0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kb = key0 + 16 * h0 + 8 * u;
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int e = 0; e < 8; ++e) vo.v[u][n][e] = kb + e < kv_len ? vo.v[u][n][e] : (VOp)0.f;
    }
  };
  auto qk = [&](const KOps& ko) -> f32x16 {  // S^T[key][row], unscaled
    f32x16 sc = {};
#pragma unroll
    for (int c = 0; c < QS; ++c) {
      if constexpr (!T::kSplitP) sc = mfma32x32x16(ko.k[c], qf[c], sc);
      else sc = mfma32x32x16(ko.k[c], qfrag(c), sc);
    }
    return sc;
  };
  auto pv = [&](const VOps& vo, const PFrag<FV>& pf) {  // O^T += V^T P^T
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] = mfma32x32x16(vo.v[u][n], pf.hi[u], acc[n]);
      if constexpr (T::kSplitP) {
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[n] = mfma32x32x16(vo.v[u][n], pf.lo[u], acc[n]);
      }
    }
  };
  // scores of a sub-tile (in place) -> P fragments. The running max moves
  // only when some row's max grows by more than 2^kLazy (rare); the factor
  // the accumulators then need is returned in `alpha` and applied by the
  // caller once the products of the previous sub-tile have been added.
  auto sm_max = [&](f32x16& sc, int key0, bool mask, float& alpha) -> bool {
    if (mask) {
      const int kb = key0 + 16 * h0;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = (kb + i <= lim && kb + i < kv_len) ? sc[i] : -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
    {  // the other 16 keys of this row sit in lane l ^ 32
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c2;  // c2 > 0: max commutes
    }
    const bool grow = mx > m_run + kLazy;
    const bool any = __any(grow);
    alpha = 1.f;
    if (any) {
      const float m_new = grow ? mx : m_run;
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 1 for rows that keep their max
      m_run = m_new;
      l_run *= alpha;
    }
    return any;
  };
  auto sm_exp = [&](f32x16& sc, PFrag<FV>& out) {
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sc[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], c2, -m_run));
      sum += sc[i];
    }
    l_run += sum;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float a = sc[8 * h + e], b = sc[8 * h + e + 1];
        const VOp ha = (VOp)a, hb = (VOp)b;
        out.hi[h][e] = ha;
        out.hi[h][e + 1] = hb;
        if constexpr (T::kSplitP) {
          // the rounded pair as floats: bf16 bits are the top half of fp32
          typedef __attribute__((__vector_size__(2 * sizeof(VOp)))) VOp VOpx2;
          const VOpx2 hp = {ha, hb};
          const uint32_t bits = __builtin_bit_cast(uint32_t, hp);
          const float fa = __uint_as_float(bits << 16), fb = __uint_as_float(bits & 0xffff0000u);
          out.lo[h][e] = (VOp)(a - fa);
          out.lo[h][e + 1] = (VOp)(b - fb);
        }
      }
    }
  };
  auto softmax = [&](f32x16& sc, int key0, bool mask, PFrag<FV>& out, float& alpha) -> bool {
    const bool any = sm_max(sc, key0, mask, alpha);
    sm_exp(sc, out);
    return any;
  };

  // ---- pipeline ----
  // Sub-tile j (keys 32j .. 32j+31) belongs to stage j/2. Step j first reads
  // from LDS the V operands of sub-tile j and the K operands of sub-tile j+2,
  // then turns S(j+1) into P(j+1) on the vector units while those reads are in
  // flight, and only then issues the 24 matrix products PV(j) and
  // S(j+2) = QK(j+2) back to back. The score product thus runs two sub-tiles
  // ahead of the value product, and the two waves of a SIMD can overlap one's
  // softmax with the other's products.
  // K stage s and V stage s live in buffers s % kRing. During stage X the
  // waves read K stage X+1 and V stage X; at its end (barrier B_X) K stage
  // X+2 and V stage X+1 must have landed, and the freed buffers receive K
  // stage X+kKAhead and V stage X+kVAhead (issued in that order: V, then K).
  // Direct-to-LDS loads keep three stages in flight; fp8 stages wait in
  // registers, so they run one stage ahead. A converted bf16 V stage must
  // land one stage earlier: stage X converts V stage X+1 in place, and B_X
  // publishes the result.
  constexpr int kKAhead = T::kFp8 ? 3 : kRing + 1;
  constexpr int kVAhead = kKAhead - 1;
  // vector-memory instructions a stage issues per wave (direct loads) and
  // the number of them allowed to stay in flight at B_X
  constexpr int kKI = T::kFp8 ? 0 : Dma<D, BLK>::kKInst;
  constexpr int kVI = T::kFp8 ? 0 : Dma<D, BLK>::kVInst;
  constexpr int kInFlight = T::kConvV ? 2 * kKI + kVI : 2 * kKI + 2 * kVI;
  static_assert(kInFlight < 16, "vmcnt field");
  PFrag<FV> pa, pb;  // P of sub-tiles 2X (pa) and 2X+1 (pb)
  f32x16 sc;         // S of the next sub-tile to turn into P

  auto lgkm_barrier = [&]() {  // LDS reads of this wave done, then meet the others
    __builtin_amdgcn_s_waitcnt((0xF) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    block_barrier();
  };
  // B_X: this wave's loads of the stages needed next have landed (all but
  // those of the last issue points, when they were all made) and its LDS
  // accesses are done; then meet the other waves
  auto ring_barrier = [&](bool keep) {
    if constexpr (!T::kFp8) {
      if (keep) __builtin_amdgcn_s_waitcnt(kInFlight | (7 << 4));  // vmcnt(kInFlight) lgkmcnt(0)
      else __builtin_amdgcn_s_waitcnt(7 << 4);                     // vmcnt(0) lgkmcnt(0)
    } else {
      __builtin_amdgcn_s_waitcnt(7 << 4);
    }
    block_barrier();
  };

  // bf16 -> f16 in place for this thread's share of V stage `st` (keys >=
  // kv_len hold whatever the cache slots hold and are zeroed before use). A
  // value beyond f16 range becomes inf here; the check after the last stage
  // finds it in the accumulators.
  // two bf16 values (one word) -> two f16 values
  auto conv_word = [&](uint32_t x) -> uint32_t {
    const f16x2 h = {(f16_t)__uint_as_float(x << 16), (f16_t)__uint_as_float(x & 0xffff0000u)};
    return __builtin_bit_cast(uint32_t, h);
  };
  auto convert_v = [&](int st) {
    if constexpr (T::kConvV) {
      constexpr int kPieces = kStage * D / 8;  // 16-byte pieces of a V stage
      char* vl = v_lds0 + (st % kRing) * kVBytes;
#pragma unroll
      for (int i0 = 0; i0 < kPieces; i0 += kThreads) {
        const int i = i0 + tid;
        if (kPieces % kThreads != 0 && i >= kPieces) break;
        const u32x4 w = *reinterpret_cast<const u32x4*>(vl + i * 16);
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = conv_word(w[e]);
        *reinterpret_cast<u32x4*>(vl + i * 16) = o;
      }
    }
  };

  // prologue: K stages 0, 1 and V stage 0 loaded and awaited together with
  // the Q fragments (one full wait, so that no load of the Q registers is left
  // outstanding inside the loop) and V stage 0 converted; then V stages
  // 1 .. kVAhead-2 and K stages 2 .. kKAhead-2 issued, P(0) and S(1)
  // computed, and V stage kVAhead-1 and K stage kKAhead-1 issued once every
  // wave has read K stage 0.
  Ids ids0 = load_ids_raw<BLK>(bt, 0, last_blk);
  Ids ids1 = load_ids_raw<BLK>(bt, 1, last_blk);
  Ids ids2 = load_ids_raw<BLK>(bt, 2, last_blk);
  Ids ids3 = load_ids_raw<BLK>(bt, 3, last_blk);
  ids0 = clamp_ids(ids0, p.num_blocks);
  ids1 = clamp_ids(ids1, p.num_blocks);
  issue_k(0, ids0);
  issue_v(0, ids0);
  commit(0, 0);
  if (nst > 1) {
    issue_k(1, ids1);
    commit(1, -1);
  }
  __builtin_amdgcn_s_waitcnt(7 << 4);  // vmcnt(0) lgkmcnt(0)
  asm volatile("" ::: "memory");       // the stage's own loads have landed: no LDS access moves above
  convert_v(0);
  Ids idsv = ids1;  // V stage s-1 goes with K stage s
#pragma unroll
  for (int s2 = 2; s2 < kKAhead - 1; ++s2) {  // direct loads only (fp8: kKAhead - 1 == 2)
    const Ids idsk = clamp_ids(s2 == 2 ? ids2 : ids3, p.num_blocks);
    if (s2 - 1 < nst) issue_v(s2 - 1, idsv);
    if (s2 < nst) issue_k(s2, idsk);
    idsv = idsk;
  }
  const Ids ids4raw = load_ids_raw<BLK>(bt, kKAhead - 1, last_blk);
  const Ids ids5raw = load_ids_raw<BLK>(bt, kKAhead, last_blk);
  lgkm_barrier();
  if (nsub > 0) {
    KOps k0;
    load_k(0, 0, k0);
    sc = qk(k0);
    float alpha;
    softmax(sc, 0, 32 > full_keys_w, pa, alpha);  // the accumulators are still zero
  }
  if (nsub > 1) {
    KOps k1;
    load_k(0, 1, k1);
    sc = qk(k1);
  }
  // B_{-1}: K stage 0 has been read (its buffer takes K stage kKAhead-1);
  // a converted V stage 1 must have landed
  ring_barrier(kKAhead - 2 < nst);
  Ids idsk = clamp_ids(ids4raw, p.num_blocks);
  int pend_k = -1, pend_v = -1;  // fp8 stages waiting in registers
  if (kVAhead - 1 < nst) {
    issue_v(kVAhead - 1, idsv);
    pend_v = kVAhead - 1;
  }
  if (kKAhead - 1 < nst) {
    issue_k(kKAhead - 1, idsk);
    pend_k = kKAhead - 1;
  }
  idsv = idsk;                                                 // V stage X+kVAhead at B_X
  idsk = clamp_ids(ids5raw, p.num_blocks);  // K stage X+kKAhead at B_X

  // step j (every branch is uniform over the wave): PV(j) with pcur,
  // P(j+1) = softmax(S(j+1)) into pnext, S(j+2) = QK(j+2)
  auto step = [&](int j, int bk, int bv, int t, const PFrag<FV>& pcur, PFrag<FV>& pnext) {
    const bool do_pv = j < nsub, do_sm = j + 1 < nsub, do_qk = j + 2 < nsub;
    VOps vo;
    KOps ko;
    if (do_pv) load_v(bv, t, vo);
    if constexpr (!T::kSplitP) {
      if (do_qk) load_k(bk, t, ko);
    }
    float alpha = 1.f;
    bool rescale = false;
    if (do_sm) rescale = softmax(sc, 32 * (j + 1), 32 * (j + 2) > full_keys_w, pnext, alpha);
    if (do_pv) {
      if (32 * (j + 1) > kv_len) zero_tail(vo, 32 * j);
      pv(vo, pcur);
    }
    if (rescale) {
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] *= alpha;
    }
    if constexpr (T::kSplitP) {  // the exact pass: V operands dead before the K ones are read
      if (do_qk) load_k(bk, t, ko);
    }
    if (do_qk) sc = qk(ko);
  };
  // A step away from the edges (no mask, no tail, every product present).
  // Nothing of P(j+1) feeds PV(j) or S(j+2) = QK(j+2), so the row max of
  // S(j+1) is taken between the value products and its exponentials between
  // the score products, on the vector units while the matrix core works.
  // vo, ko hold this step's operands; with `next`, the operands of sub-tile
  // t+1 of the same stage are read into them once their products are issued.
  // The order is fixed chunk by chunk: no instruction crosses a
  // sched_barrier, and the empty asm statements keep each value computed in
  // its chunk rather than next to its use.
  // A converted bf16 cache's V stage `cst` (the next one, no tail) is
  // converted here too: the thread's piece t is read first, converted a word
  // at a time between the score products and written back at the end.
  // A thread converts the same pieces (t * kThreads + tid) here as in
  // convert_v: waves of one work-group can run different loops during the
  // same stage (their full-step counts differ), and every piece must be
  // converted exactly once. Those pieces lie in the 1 KB chunks that the
  // thread's own wave loads, which lets the prologue convert V stage 0 after
  // its own loads' wait, with no barrier.
  auto step_full = [&](int bk, int bv, int t, const PFrag<FV>& pcur, PFrag<FV>& pnext, VOps& vo, KOps& ko,
                       bool next, int cst) {
    if constexpr (!T::kSplitP) {  // one value product per operand
      constexpr int kCP = kStage * D / 8 / kThreads;  // 16-byte pieces per thread and V stage
      static_assert(kCP * kThreads * 8 == kStage * D, "whole pieces");
      const bool conv = T::kConvV && t < kCP;
      char* const cp = v_lds0 + (cst % kRing) * kVBytes + (t * kThreads + tid) * 16;
      u32x4 cw = {};
      if (conv) cw = *reinterpret_cast<const u32x4*>(cp);
      constexpr int kE = 16 / (2 * NT);  // elements handled per value product
      // kConvV: no row maximum here; the exponentials below use the running
      // max as it stands and P(j+1) is checked after them (below). A score
      // that outgrew the max by more than 2^128 makes P infinite; the
      // accumulators then end non-finite and the exact pass redoes the rows.
      constexpr bool kNoMax = T::kConvV;
      float mx = sc[0];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          acc[n] = mfma32x32x16(vo.v[u][n], pcur.hi[u], acc[n]);
          if constexpr (!kNoMax) {
            const int i0 = (u * NT + n) * kE;
#pragma unroll
            for (int e = 0; e < kE; ++e) mx = fmaxf(mx, sc[i0 + e]);
            asm volatile("" : "+v"(mx));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (next) load_v(bv, t + 1, vo);
      __builtin_amdgcn_sched_barrier(0);
      bool rescale = false;
      float alpha = 1.f;
      if constexpr (!kNoMax) {
        {  // the other 16 keys of this row sit in lane l ^ 32
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c2;  // c2 > 0: max commutes
        }
        const bool grow = mx > m_run + kLazy;
        rescale = __any(grow);
        if (rescale) {
          const float m_new = grow ? mx : m_run;
          alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 1 for rows that keep their max
          m_run = m_new;
          l_run *= alpha;
        }
      }
      // score products, each followed by 16/QS exponentials of P(j+1) and,
      // with `next`, the read of the K operand it has just consumed
      constexpr int kX = 16 / QS;
      const char* kl_next = k_lds0 + bk * kKBytes + (t + 1) * kKSub;
      f32x16 s2 = {};
      float x[16];
#pragma unroll
      for (int c = 0; c < QS; ++c) {
        s2 = mfma32x32x16(ko.k[c], qf[c], s2);
#pragma unroll
        for (int e = 0; e < kX; ++e) {
          const int i = c * kX + e;
          x[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], c2, -m_run));
          asm volatile("" : "+v"(x[i]));
        }
        if (next) ko.k[c] = *reinterpret_cast<const F*>(kl_next + (kx ^ (c << 5)));
        if (conv && c % (QS / 4) == QS / 4 - 1) cw[c / (QS / 4)] = conv_word(cw[c / (QS / 4)]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (conv) *reinterpret_cast<u32x4*>(cp) = cw;
      if constexpr (kNoMax) {
        // row sum of P(j+1); when a lane's sum passes 16 kPCap, the rows whose
        // largest P passed kPCap move their max by that P's binary exponent,
        // so that P, l and (at the end of the step) the accumulators scale by
        // an exact power of two, whatever the size of the jump (the kernel
        // keeps fp32 denormals, so 2^-128 is exact; a factor computed with
        // v_exp_f32 would flush to 0 below 2^-126 and take the row's new
        // largest P with it). An infinite P (a jump past 2^128) is left as it
        // is: the accumulators then end non-finite and the exact pass redoes
        // the work-group.
        auto psum = [&]() {
          float part[8];
#pragma unroll
          for (int pr = 0; pr < 8; ++pr) part[pr] = x[2 * pr] + x[2 * pr + 1];
          return ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
        };
        float lsum = psum();
        rescale = __any(!(lsum <= 16.f * kPCap));
        if (rescale) {
          float px = x[0];
#pragma unroll
          for (int i = 1; i < 16; ++i) px = fmaxf(px, x[i]);
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(px), __float_as_uint(px), false, false);
          px = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
          // px = f 2^e with f in [0.5, 1); e = 0 for rows that keep their max
          const int e = px > kPCap && px <= 3.4028235e38f ? __builtin_amdgcn_frexp_expf(px) : 0;
          m_run += (float)e;
          alpha = __builtin_ldexpf(1.f, -e);  // 2^-e, exact (a denormal past 2^-126)
          l_run *= alpha;
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] *= alpha;
          lsum = psum();
        }
        l_run += lsum;
#pragma unroll
        for (int pr = 0; pr < 8; ++pr) {  // packing of P(j+1): elements 2pr, 2pr+1
          const int h = pr / 4, e = 2 * (pr % 4);
          pnext.hi[h][e] = (VOp)x[2 * pr];
          pnext.hi[h][e + 1] = (VOp)x[2 * pr + 1];
        }
      } else {
        // row sum and packing of P(j+1)
        float part[8];
#pragma unroll
        for (int pr = 0; pr < 8; ++pr) {  // elements 2pr, 2pr+1
          const int h = pr / 4, e = 2 * (pr % 4);
          pnext.hi[h][e] = (VOp)x[2 * pr];
          pnext.hi[h][e + 1] = (VOp)x[2 * pr + 1];
          part[pr] = x[2 * pr] + x[2 * pr + 1];
        }
        l_run += ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
      }
      sc = s2;
      if (rescale) {
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[n] *= alpha;
      }
    }
  };
  // B_X and the loads it frees buffers for (the ids of K stage X+kKAhead+1
  // are fetched before the barrier's wait, which covers their latency)
  auto stage_end = [&](int X) {
    commit(pend_k, pend_v);
    const Ids raw = load_ids_raw<BLK>(bt, X + kKAhead + 1, last_blk);
    ring_barrier(X + kKAhead - 1 < nst);
    pend_k = X + kKAhead < nst ? X + kKAhead : -1;
    pend_v = X + kVAhead < nst ? X + kVAhead : -1;
    if (X + kVAhead < nst) issue_v(X + kVAhead, idsv);
    if (X + kKAhead < nst) issue_k(X + kKAhead, idsk);
    idsv = idsk;
    idsk = clamp_ids(raw, p.num_blocks);
  };
  // Stages X < x_full have only full steps: sub-tiles up to 2X+3 exist in
  // this wave and need no mask (then X + 1 < nst, since nsub <= 2 nst), and
  // stage X+1 has no key at or beyond kv_len, so its conversion needs no mask
  // either. They run in a loop of their own, so that neither loop carries the
  // other's register needs.
  const int a_full = min(nsub - 1, full_keys_w / 32);
  const int x_full = T::kSplitP ? 0
                                : __builtin_amdgcn_readfirstlane(
                                      min(a_full >= 3 ? (a_full - 3) / 2 + 1 : 0, max(kv_len / kStage - 1, 0)));
  int X = 0;
  for (; X < x_full; ++X) {
    const int bv = X % kRing, bk = (X + 1) % kRing;
    VOps vo;
    KOps ko;
    load_v(bv, 0, vo);
    load_k(bk, 0, ko);
    // fp8: the registers hold the staged loads, so sub-tile 1's operands are
    // read only once sub-tile 0's products are done
    constexpr bool kAhead = !T::kFp8;
    step_full(bk, bv, 0, pa, pb, vo, ko, kAhead, X + 1);
    if (!kAhead) {
      load_v(bv, 1, vo);
      load_k(bk, 1, ko);
    }
    step_full(bk, bv, 1, pb, pa, vo, ko, false, X + 1);
    stage_end(X);
  }
  for (; X < nst; ++X) {
    const int bv = X % kRing, bk = (X + 1) % kRing;
    if (X + 1 < nst) convert_v(X + 1);
    step(2 * X, bk, bv, 0, pa, pb);
    step(2 * X + 1, bk, bv, 1, pb, pa);
    stage_end(X);
  }
  if constexpr (T::kConvV) {
    // a V value beyond f16 range became inf in the conversion and made some
    // accumulator non-finite (inf, or NaN where its weight was 0): redo
    // these rows exactly
    float fs = 0.f;
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) fs += acc[n][i];
    const int big = !__builtin_isfinite(fs);
    if (__syncthreads_or(big)) return false;
  }

  // ---- epilogue: O = O^T / l; element i of acc[n] is dim 32n + 8(i/4) + 4h0 + i%4 ----
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (casc || kSplit) {  // unnormalised partial (O, m, l) of each (row, head) for the merge
    if (rvalid) {
      const int64_t srow = ((int64_t)split * p.total_rows + row_base + tok) * p.hq + qh;
      float* orow = p.ws_o + srow * D;
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          *reinterpret_cast<f32x4*>(orow + 32 * n + 8 * k + 4 * h0) =
              f32x4{acc[n][4 * k], acc[n][4 * k + 1], acc[n][4 * k + 2], acc[n][4 * k + 3]};
      if (h0 == 0) *reinterpret_cast<f32x2*>(p.ws_ml + srow * 2) = f32x2{m_run, l_run};
    }
    return true;
  }
  if (rvalid) {
    const float inv = p.v_scale / l_run;
    TQ* orow = reinterpret_cast<TQ*>(p.out) + (int64_t)(row_base + tok) * p.o_s0 + (int64_t)qh * p.o_s1;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {  // 4 consecutive dims per store
        typedef __attribute__((__vector_size__(4 * sizeof(TQ)))) TQ TQx4;
        TQx4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = from_f32<TQ>(acc[n][4 * k + e] * inv);
        *reinterpret_cast<TQx4*>(orow + 32 * n + 8 * k + 4 * h0) = o;
      }
    }
  }
  return true;
}

// One row tile. For a bf16 cache the fast pass (V converted to f16 in LDS)
// reports whether every V value fitted; if one did not, the tile is redone
// with the exact bf16 hi/lo products.
template <typename TQ, typename TC, int D, int BLK, bool kCasc, bool kSplit = false>
__device__ __forceinline__ void attend_tile(const PrefillParams& p, char* lds, int wg) {
  if constexpr (std::is_same<TC, bf16_t>::value) {
    if (!attend<TQ, TC, D, BLK, true, kCasc, kSplit>(p, lds, wg)) {
      // rare: redo exactly. The empty asm hides that this pass works on the
      // same work-group, so nothing computed for the fast pass is kept alive
      // for it.
      asm volatile("" : "+s"(wg));
      attend<TQ, TC, D, BLK, false, kCasc, kSplit>(p, lds, wg);
    }
  } else {
    attend<TQ, TC, D, BLK, false, kCasc, kSplit>(p, lds, wg);
  }
}

}  // namespace
}  // namespace pkv
