// Suffix-only prefill attention over a cached prefix, for gfx950.
//
// What it computes (page "PagedAttention과 RadixAttention으로 LLM KV 캐시
// 최적화" §03: reuse the longest cached prefix and compute only the suffix;
// page "KV Cache에 대해 알아보자 (Feat. Attention)" §1 equation and §3: prefill
// handles the new tokens at once): suffix row i of request r attends to key
// positions 0 .. P_r + i of that request (the cached prefix in full, the suffix
// causally), keys and values read through the block table.
//
// Design (a dense contraction, so it runs on the matrix cores):
//  * Rows of the problem are (suffix token, query head of the GQA group)
//    pairs, token-major, so one K/V read serves all G heads of a KV head and a
//    tile's causal diagonal spans few tokens. A work-group of 4 waves owns 128
//    rows of one (request, KV head); each wave owns 32 rows, whose Q^T stays in
//    registers.
//  * Keys are consumed 64 per stage, double buffered in LDS (the next stage's
//    loads are in flight while this one is computed; one barrier per stage).
//    16-bit K and V go from global memory straight to LDS (global_load_lds);
//    fp8 tiles are staged through registers and converted. Values of keys past
//    the end are zeroed in LDS (they meet P = 0, and 0 * NaN would be NaN).
//    Both LDS tiles are XOR-swizzled so that the matrix-core operand reads are
//    free of bank conflicts. Block ids come from scalar loads two stages ahead.
//  * Per wave and 32-key sub-tile, on v_mfma_f32_32x32x16:
//      S^T[key][row] = K[key][:] . Q[row][:]
//      O^T[dim][row] += V^T[dim][keys] . P^T[keys][row]
//    K rows are read in a permuted order so that each lane ends up holding 16
//    consecutive keys of one row: the B operand of the PV product.
//  * Precision of P in the PV product: with f16 operands P is rounded to f16
//    (11 bits, P is in [0, 2^8] thanks to the lazy rescale below). With bf16
//    operands P would carry only 8 bits - too few for 2e-3 on short contexts -
//    so P goes in as bf16(P) + bf16(P - bf16(P)): two products on the matrix
//    cores, which have room to spare, instead of converting V on the vector
//    units, which do not. fp8 V is converted exactly to f16 while staging.
//  * Online softmax in base 2 with the scale folded into one FMA per score and
//    the raw v_exp_f32 (results below 2^-126 flush to 0); the running max moves
//    only when a row's max grows by more than 2^8 (lazy rescale), so the
//    output accumulators are rarely rescaled. The causal mask is applied only
//    on key tiles that reach past the wave's first token.
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

#include <math.h>
#include <type_traits>

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsWave = 32;
constexpr int kRowsWg = kRowsWave * kWaves;
constexpr int kStage = 64;     // keys per LDS stage
constexpr float kLazy = 8.0f;  // log2 headroom before the running max moves

typedef __attribute__((address_space(3))) void lds_void;

// ---- LDS tile layouts (element offsets), with XOR swizzles of 16-byte pieces ----
// K: [kStage keys][D] in the operand type; piece = 8 dims.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  if constexpr (D == 128) return (row & 7) | (((row >> 4) & 1) << 3);
  else return ((row >> 1) & 3) | (((row >> 4) & 1) << 2);
}
template <int D>
__device__ __forceinline__ int k_off(int row, int piece) {  // piece in [0, D/8)
  return row * D + ((piece ^ k_swz<D>(row)) << 3);
}
// V^T: [D][kStage keys] in f16; piece = 8 keys.
__device__ __forceinline__ int v_off(int d, int piece) {  // piece in [0, 8)
  return d * kStage + ((piece ^ ((d >> 1) & 7)) << 3);
}

template <typename TQ, typename TC>
struct Types {
  static constexpr bool kFp8 = std::is_same<TC, uint8_t>::value;
  static constexpr bool kDirect = !kFp8;  // 16-bit tiles land in LDS as stored
  // PV operand type: the cache's own 16-bit type, f16 for an fp8 cache
  typedef typename std::conditional<kFp8, f16_t, TC>::type VOp;
  static constexpr bool kSplitP = std::is_same<VOp, bf16_t>::value;
};

template <typename TQ, typename TC, int D, int BLK>
struct Stage {
  typedef Types<TQ, TC> T;
  typedef typename T::VOp VOp;
  static constexpr int kBlocks = kStage / BLK;  // blocks per stage
  // fp8 register staging: K pieces of 16 dims (16 codes), V pieces of 8 keys
  // (8 codes); an empty struct for 16-bit tiles, which go straight to LDS
  static constexpr int kKPieces = kStage * (D / 16) / kThreads;
  static constexpr int kVPieces = D * (kStage / 8) / kThreads;
  struct Fp8Regs {
    u32x4 kr[kKPieces];
    u32x2 vr[kVPieces];
  };
  struct NoRegs {};
  typedef typename std::conditional<T::kDirect, NoRegs, Fp8Regs>::type Regs;

  // Block ids of one stage, kept in four plain ints (arrays or structs here
  // end up in LDS or scratch). Loaded with scalar loads: pointer and index
  // are uniform; entries past the end repeat the last block with a live key.
  __device__ __forceinline__ static void load_ids(int& b0, int& b1, int& b2, int& b3, const int32_t* bt, int st,
                                                  int kv_len, int max_blocks, int num_blocks) {
    static_assert(kBlocks == 2 || kBlocks == 4, "16- or 32-token blocks");
    const int last = min((kv_len - 1) / BLK, max_blocks - 1);
    auto id = [&](int i) {
      const int jb = min(st * kBlocks + i, last);
      return min(max(bt[jb], 0), num_blocks - 1);
    };
    b0 = id(0);
    b1 = id(1);
    b2 = kBlocks == 4 ? id(2) : 0;
    b3 = kBlocks == 4 ? id(3) : 0;
  }
  __device__ __forceinline__ static int pick(int b0, int b1, int b2, int b3, int i) {  // i in [0, kBlocks)
    if constexpr (kBlocks == 2) return i == 0 ? b0 : b1;
    else return i < 2 ? (i == 0 ? b0 : b1) : (i == 2 ? b2 : b3);
  }

  // Issue this thread's loads of stage `st` (keys st*kStage ..) with the
  // stage's block ids: direct-to-LDS for 16-bit tiles, registers for fp8.
  __device__ __forceinline__ static void issue(Regs& rg, const TC* kbase, const TC* vbase, int b0, int b1, int b2,
                                               int b3, int hk, int hkv, int st, int kv_len, TQ* k_lds, VOp* v_lds,
                                               int wave, int lane) {
    const int key0 = st * kStage;
    const int64_t tile = (int64_t)BLK * D;
    if constexpr (T::kDirect) {
      // K: 1 KB per instruction, lane-linear, rows of D*2 bytes
      constexpr int kInst = kStage * D * 2 / 1024;
      constexpr int kRowsPerInst = 1024 / (D * 2);
      constexpr int kLanesPerRow = 64 / kRowsPerInst;
#pragma unroll
      for (int i = 0; i < kInst / kWaves; ++i) {
        const int j = wave * (kInst / kWaves) + i;
        int row = j * kRowsPerInst + lane / kLanesPerRow;
        const int piece = (lane % kLanesPerRow) ^ k_swz<D>(row);
        if (key0 + row >= kv_len) row = kv_len - 1 - key0 >= 0 ? kv_len - 1 - key0 : 0;  // any live row
        const TC* src = kbase + ((int64_t)pick(b0, b1, b2, b3, row / BLK) * hkv + hk) * tile + (int64_t)(row % BLK) * D + piece * 8;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), (lds_void*)(k_lds + j * 512), 16, 0, 0);
      }
      // V^T: 1 KB per instruction = 8 rows of 64 keys
      constexpr int kVInst = D * kStage * 2 / 1024;
#pragma unroll
      for (int i = 0; i < kVInst / kWaves; ++i) {
        const int j = wave * (kVInst / kWaves) + i;
        const int d = j * 8 + lane / 8;
        const int piece = (lane % 8) ^ ((d >> 1) & 7);
        const int k8 = piece * 8;  // first key of the piece within the stage
        const TC* src = vbase + ((int64_t)pick(b0, b1, b2, b3, k8 / BLK) * hkv + hk) * tile + (int64_t)d * BLK + (k8 % BLK);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), (lds_void*)(v_lds + j * 512), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kKPieces; ++i) {  // 16 codes = dims 16q .. 16q+15 of one key
        const int pi = lane + 64 * (wave + kWaves * i);
        const int row = pi / (D / 16), q = pi % (D / 16);
        u32x4 w = {0u, 0u, 0u, 0u};
        if (key0 + row < kv_len)
          w = load_u32x4(kbase + ((int64_t)pick(b0, b1, b2, b3, row / BLK) * hkv + hk) * tile + (int64_t)(row % BLK) * D + q * 16);
        rg.kr[i] = w;
      }
#pragma unroll
      for (int i = 0; i < kVPieces; ++i) {  // 8 codes = keys 8p .. 8p+7 of one dim
        const int pi = lane + 64 * (wave + kWaves * i);
        const int d = pi / (kStage / 8), piece = pi % (kStage / 8);
        u32x2 w = {0u, 0u};
        if (key0 + piece * 8 < kv_len)
          w = load_u32x2(vbase + ((int64_t)pick(b0, b1, b2, b3, piece * 8 / BLK) * hkv + hk) * tile + (int64_t)d * BLK + (piece * 8) % BLK);
        rg.vr[i] = w;
      }
    }
  }

  // fp8: convert the register-staged pieces of stage `st` and write them to LDS.
  __device__ __forceinline__ static void commit(Regs& rg, int st, int kv_len, TQ* k_lds, VOp* v_lds, int wave,
                                                int lane) {
    if constexpr (!T::kDirect) {
      typedef typename Frag<TQ>::type F;
#pragma unroll
      for (int i = 0; i < kKPieces; ++i) {
        const int pi = lane + 64 * (wave + kWaves * i);
        const int row = pi / (D / 16), q = pi % (D / 16);
        u32x2 lo = {rg.kr[i][0], rg.kr[i][1]}, hi = {rg.kr[i][2], rg.kr[i][3]};
        *reinterpret_cast<F*>(k_lds + k_off<D>(row, 2 * q)) = fp8x8_to<TQ>(lo);
        *reinterpret_cast<F*>(k_lds + k_off<D>(row, 2 * q + 1)) = fp8x8_to<TQ>(hi);
      }
      const int key0 = st * kStage;
#pragma unroll
      for (int i = 0; i < kVPieces; ++i) {
        const int pi = lane + 64 * (wave + kWaves * i);
        const int d = pi / (kStage / 8), piece = pi % (kStage / 8);
        f16x8 f = fp8x8_to<f16_t>(rg.vr[i]);  // exact: every e4m3fn value is an f16 value
        const int pos = key0 + piece * 8;
        if (pos + 8 > kv_len) {
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = pos + e < kv_len ? f[e] : (f16_t)0.f;
        }
        *reinterpret_cast<f16x8*>(v_lds + v_off(d, piece)) = f;
      }
    }
  }

  // 16-bit tiles: after the stage has landed, zero V of keys >= kv_len (the
  // direct loads brought whatever those cache slots hold). Call with all
  // threads of the work-group; only the stage holding kv_len has such keys.
  __device__ __forceinline__ static void zero_tail(int st, int kv_len, VOp* v_lds, int tid) {
    const int key0 = st * kStage;
    const int first = kv_len - key0;  // first dead key within the stage
    const int dead = kStage - first;
    for (int idx = tid; idx < D * dead; idx += kThreads) {
      const int d = idx / dead, k = first + idx % dead;
      v_lds[v_off(d, k / 8) + (k % 8)] = (VOp)0.f;
    }
  }
};

template <typename TQ, typename TC, int D, int BLK>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillParams p) {
  typedef Types<TQ, TC> T;
  typedef typename T::VOp VOp;
  typedef typename Frag<TQ>::type F;
  typedef typename Frag<VOp>::type FV;
  typedef Stage<TQ, TC, D, BLK> STG;
  constexpr int QS = D / 16;  // k-steps of the score product
  constexpr int NT = D / 32;  // dim tiles of the output
  constexpr int kKElems = kStage * D, kVElems = D * kStage;
  __shared__ __attribute__((aligned(16))) TQ k_lds_all[2 * kKElems];
  __shared__ __attribute__((aligned(16))) VOp v_lds_all[2 * kVElems];

  // ---- which (KV head, request, row tile) ----
  const int logical = xcd_remap(blockIdx.x, p.hkv * p.tiles_per_head);
  const int hk = logical / p.tiles_per_head;
  int tile = logical % p.tiles_per_head;
  int r = 0, row_base = 0, rows_r = 0;
  for (; r < p.num_reqs; ++r) {
    int s = p.suffix_lens[r];
    s = s < 0 ? 0 : s;
    if (row_base + s > p.total_rows) s = (int)(p.total_rows - row_base);
    rows_r = s * p.group;
    const int nt = (rows_r + kRowsWg - 1) / kRowsWg;
    if (tile < nt) break;
    tile -= nt;
    row_base += s;
  }
  if (r >= p.num_reqs) return;
  const int S = rows_r / p.group;
  int P = p.prefix_lens[r];
  P = P < 0 ? 0 : P;
  const int cap = p.max_blocks * BLK;
  int kv_len = P + S;
  if (kv_len > cap) kv_len = cap;
  const int32_t* bt = p.block_tables + (int64_t)r * p.bt_s0;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int h0 = lane / 32, c32 = lane % 32;

  const int q0 = tile * kRowsWg;                  // first row of the work-group
  const int tok_last_wg = min(S - 1, (q0 + kRowsWg - 1) / p.group);
  const int wq0 = q0 + wave * kRowsWave;          // first row of this wave
  const int tok_first_w = wq0 / p.group;
  const int tok_last_w = min(S - 1, (wq0 + kRowsWave - 1) / p.group);
  const bool wave_active = wq0 < rows_r;
  const int keys_wg = min(kv_len, P + tok_last_wg + 1);
  const int nst = (keys_wg + kStage - 1) / kStage;
  const int keys_w = wave_active ? min(kv_len, P + tok_last_w + 1) : 0;
  const int full_keys_w = min(P + tok_first_w + 1, kv_len);  // keys below need no mask in this wave

  // ---- Q^T fragments for this lane's row ----
  const int row = wq0 + c32;
  const bool rvalid = row < rows_r;
  const int tok = rvalid ? row / p.group : 0;
  const int qh = hk * p.group + (rvalid ? row % p.group : 0);
  const TQ* qrow = reinterpret_cast<const TQ*>(p.q) + (int64_t)(row_base + tok) * p.q_s0 + (int64_t)qh * p.q_s1;
  F qf[QS];
#pragma unroll
  for (int c = 0; c < QS; ++c) {
    F v = {};
    if (rvalid) v = load_frag8(qrow + 16 * c + 8 * h0);
    qf[c] = v;
  }
  const int lim = P + tok;  // last key position this row may see
  // permuted key row (within a 32-key sub-tile) read by this lane for the score A operand
  const int krow_perm = 16 * ((c32 % 8) / 4) + 4 * (c32 / 8) + (c32 % 4);

  f32x16 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const TC* kbase = reinterpret_cast<const TC*>(p.k_cache);
  const TC* vbase = reinterpret_cast<const TC*>(p.v_cache);
  typename STG::Regs regs;
  const bool tail_stage_exists = nst > 0 && kv_len < nst * kStage;

  int a0 = 0, a1 = 0, a2 = 0, a3 = 0;  // block ids of stage st+1
  int n0 = 0, n1 = 0, n2 = 0, n3 = 0;  // block ids of stage st+2
  if (nst > 0) {
    int z0, z1, z2, z3;
    STG::load_ids(z0, z1, z2, z3, bt, 0, kv_len, p.max_blocks, p.num_blocks);
    STG::issue(regs, kbase, vbase, z0, z1, z2, z3, hk, p.hkv, 0, kv_len, k_lds_all, v_lds_all, wave, lane);
    STG::commit(regs, 0, kv_len, k_lds_all, v_lds_all, wave, lane);
    STG::load_ids(a0, a1, a2, a3, bt, 1, kv_len, p.max_blocks, p.num_blocks);
  }
  __builtin_amdgcn_s_waitcnt(0);  // direct-to-LDS loads of stage 0 have landed
  __syncthreads();
  if constexpr (T::kDirect) {
    if (tail_stage_exists && nst == 1) {
      STG::zero_tail(0, kv_len, v_lds_all, tid);
      __syncthreads();
    }
  }

  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    TQ* k_lds = k_lds_all + buf * kKElems;
    VOp* v_lds = v_lds_all + buf * kVElems;
    TQ* k_nxt = k_lds_all + (buf ^ 1) * kKElems;
    VOp* v_nxt = v_lds_all + (buf ^ 1) * kVElems;
    if (st + 1 < nst) {
      STG::issue(regs, kbase, vbase, a0, a1, a2, a3, hk, p.hkv, st + 1, kv_len, k_nxt, v_nxt, wave, lane);
      STG::load_ids(n0, n1, n2, n3, bt, st + 2, kv_len, p.max_blocks, p.num_blocks);
    }

#pragma unroll
    for (int t = 0; t < kStage / 32; ++t) {
      const int key0 = st * kStage + 32 * t;  // first key of the sub-tile
      if (key0 < keys_w) {                    // uniform per wave
        // scores: element i = key key0 + 16*h0 + i, row c32 (unscaled)
        f32x16 s = {};
        const int krow = 32 * t + krow_perm;
#pragma unroll
        for (int c = 0; c < QS; ++c) {
          const F kf = *reinterpret_cast<const F*>(k_lds + k_off<D>(krow, 2 * c + h0));
          s = mfma32x32x16(kf, qf[c], s);
        }
        if (key0 + 32 > full_keys_w) {
          const int kb = key0 + 16 * h0;
#pragma unroll
          for (int i = 0; i < 16; ++i) s[i] = (kb + i <= lim && kb + i < kv_len) ? s[i] : -INFINITY;
        }
        float cmax = s[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) cmax = fmaxf(cmax, s[i]);
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32)) * p.qk_scale_log2;  // scale > 0: max commutes
        // lazy rescale: move the running max only when it grows by more than 2^kLazy
        const bool grow = cmax > m_run + kLazy;
        if (__any(grow)) {
          const float m_new = grow ? cmax : m_run;
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 1 for rows that keep their max
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[n] *= alpha;
        }
        float pr[16];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          pr[i] = __builtin_amdgcn_exp2f(fmaf(s[i], p.qk_scale_log2, -m_run));
          psum += pr[i];
        }
        l_run += psum;
        const FV p0 = pack8<VOp>(pr), p1 = pack8<VOp>(pr + 8);
        FV p0lo, p1lo;
        if constexpr (T::kSplitP) {
          float lo[16];
#pragma unroll
          for (int i = 0; i < 8; ++i) { lo[i] = pr[i] - (float)p0[i]; lo[8 + i] = pr[8 + i] - (float)p1[i]; }
          p0lo = pack8<VOp>(lo);
          p1lo = pack8<VOp>(lo + 8);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const int d = 32 * n + c32;
          const FV v0 = *reinterpret_cast<const FV*>(v_lds + v_off(d, 4 * t + 2 * h0));
          const FV v1 = *reinterpret_cast<const FV*>(v_lds + v_off(d, 4 * t + 2 * h0 + 1));
          acc[n] = mfma32x32x16(v0, p0, acc[n]);
          acc[n] = mfma32x32x16(v1, p1, acc[n]);
          if constexpr (T::kSplitP) {
            acc[n] = mfma32x32x16(v0, p0lo, acc[n]);
            acc[n] = mfma32x32x16(v1, p1lo, acc[n]);
          }
        }
      }
    }

    if (st + 1 < nst) {
      STG::commit(regs, st + 1, kv_len, k_nxt, v_nxt, wave, lane);
      a0 = n0; a1 = n1; a2 = n2; a3 = n3;
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct-to-LDS loads of the next stage have landed
    __syncthreads();
    if constexpr (T::kDirect) {
      if (tail_stage_exists && st + 2 == nst) {  // the next stage holds kv_len: clear dead values
        STG::zero_tail(st + 1, kv_len, v_nxt, tid);
        __syncthreads();
      }
    }
  }

  // ---- epilogue: O = O^T / l; element i of acc[n] is dim 32n + 8(i/4) + 4h0 + i%4 ----
  l_run += __shfl_xor(l_run, 32);
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
}

template <typename TQ, typename TC, int D, int BLK>
hipError_t launch_typed(const PrefillParams& p, hipStream_t stream) {
  const int64_t wgs = (int64_t)p.hkv * p.tiles_per_head;
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_kernel<TQ, TC, D, BLK>), dim3((unsigned)wgs), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <typename TQ, typename TC>
hipError_t launch_shape(const PrefillParams& p, int d, int b, hipStream_t s) {
  if (d == 128 && b == 16) return launch_typed<TQ, TC, 128, 16>(p, s);
  if (d == 128 && b == 32) return launch_typed<TQ, TC, 128, 32>(p, s);
  if (d == 64 && b == 16) return launch_typed<TQ, TC, 64, 16>(p, s);
  if (d == 64 && b == 32) return launch_typed<TQ, TC, 64, 32>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, DT q_dt, DT cache_dt, int d, int b, hipStream_t s) {
  if (q_dt == DT::F16 && cache_dt == DT::F16) return launch_shape<f16_t, f16_t>(p, d, b, s);
  if (q_dt == DT::BF16 && cache_dt == DT::BF16) return launch_shape<bf16_t, bf16_t>(p, d, b, s);
  if (q_dt == DT::F16 && cache_dt == DT::FP8) return launch_shape<f16_t, uint8_t>(p, d, b, s);
  if (q_dt == DT::BF16 && cache_dt == DT::FP8) return launch_shape<bf16_t, uint8_t>(p, d, b, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv
