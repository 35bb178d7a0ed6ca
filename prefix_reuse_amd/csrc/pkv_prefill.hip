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
//    16-bit K goes from global memory straight to LDS (global_load_lds); V is
//    staged through registers, converted to f16 and zeroed past the end. Both
//    LDS tiles are XOR-swizzled so that the matrix-core operand reads are free
//    of bank conflicts.
//  * Per wave and 32-key sub-tile, on v_mfma_f32_32x32x16:
//      S^T[key][row] = K[key][:] . Q[row][:]           (bf16 or f16)
//      O^T[dim][row] += V^T[dim][keys] . P^T[keys][row]  (f16)
//    K rows are read in a permuted order so that each lane ends up holding 16
//    consecutive keys of one row: the B operand of the PV product.
//  * P and V enter the PV product as f16 (11-bit mantissa): P is in [0, 2^8]
//    (lazy rescaling below), and a bf16 V is scaled by 2^-8 on the way in
//    (exact for |v| in [2^-6, 65504 * 2^8]; below that the absolute error is
//    at most 2^-17; beyond it the value saturates), the 2^8 is put back at the
//    end. bf16 P would carry only 8 bits, too few for 2e-3 on short contexts.
//  * Online softmax in base 2 with the scale folded in; the running max moves
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
  static constexpr bool kKDirect = !kFp8;                           // K lands in LDS as stored
  // V always goes through registers: keys past the end must become 0 (they
  // meet P = 0, and 0 * NaN would be NaN), which a direct-to-LDS load cannot do.
  static constexpr bool kVDirect = false;
  static constexpr bool kVScaled = std::is_same<TC, bf16_t>::value;
};

template <typename TQ, typename TC, int D, int BLK>
struct Stage {
  typedef Types<TQ, TC> T;
  // register staging: V pieces of 8 keys (16-bit: 16 B, fp8: 8 B); fp8 K pieces of 16 dims
  static constexpr int kVPieces = T::kVDirect ? 0 : D * (kStage / 8) / kThreads;
  static constexpr int kKPieces = T::kKDirect ? 0 : kStage * (D / 16) / kThreads;
  typedef typename std::conditional<T::kFp8, u32x2, u32x4>::type VPiece;
  VPiece vr[kVPieces > 0 ? kVPieces : 1];
  u32x4 kr[kKPieces > 0 ? kKPieces : 1];

  __device__ __forceinline__ static int block_of(const int32_t* bt, int pos, int max_blocks, int num_blocks) {
    int jb = pos / BLK;
    jb = jb < max_blocks ? jb : max_blocks - 1;
    const int b = bt[jb];
    return min(max(b, 0), num_blocks - 1);
  }

  // Issue this thread's loads of stage `st` (keys st*kStage ..): direct-to-LDS
  // pieces go to (k_lds, v_lds); register pieces to kr / vr.
  __device__ __forceinline__ void issue(const TC* kbase, const TC* vbase, const int32_t* bt, int hk, int hkv,
                                        int num_blocks, int max_blocks, int st, int kv_len, TQ* k_lds,
                                        f16_t* v_lds, int wave, int lane) {
    const int key0 = st * kStage;
    const int64_t tile = (int64_t)BLK * D;
    if constexpr (T::kKDirect) {
      // 1 KB per instruction, lane-linear: rows of D*2 bytes
      constexpr int kInst = kStage * D * 2 / 1024;
      constexpr int kRowsPerInst = 1024 / (D * 2);
      constexpr int kLanesPerRow = 64 / kRowsPerInst;
#pragma unroll
      for (int i = 0; i < kInst / kWaves; ++i) {
        const int j = wave * (kInst / kWaves) + i;
        const int row = j * kRowsPerInst + lane / kLanesPerRow;
        const int piece = (lane % kLanesPerRow) ^ k_swz<D>(row);
        int pos = key0 + row;
        pos = pos < kv_len ? pos : kv_len - 1;  // past the end: any valid row (masked later)
        const int blk = block_of(bt, pos, max_blocks, num_blocks);
        const TC* src = kbase + ((int64_t)blk * hkv + hk) * tile + (int64_t)(pos % BLK) * D + piece * 8;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                         (lds_void*)(k_lds + j * 512), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kKPieces; ++i) {  // fp8: 16 codes = dims 16q .. 16q+15 of one key
        const int pi = lane + 64 * (wave + kWaves * i);
        const int row = pi / (D / 16), q = pi % (D / 16);
        const int pos = key0 + row;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (pos < kv_len) {
          const int blk = block_of(bt, pos, max_blocks, num_blocks);
          w = load_u32x4(kbase + ((int64_t)blk * hkv + hk) * tile + (int64_t)(pos % BLK) * D + q * 16);
        }
        kr[i] = w;
      }
    }
    if constexpr (T::kVDirect) {
      // 1 KB per instruction = 8 V^T rows of 64 keys (f16)
      constexpr int kInst = D * kStage * 2 / 1024;
#pragma unroll
      for (int i = 0; i < kInst / kWaves; ++i) {
        const int j = wave * (kInst / kWaves) + i;
        const int d = j * 8 + lane / 8;
        const int piece = (lane % 8) ^ ((d >> 1) & 7);
        int pos = key0 + piece * 8;
        pos = pos < kv_len ? pos : ((kv_len - 1) / 8) * 8;  // past the end: any valid piece
        const int blk = block_of(bt, pos, max_blocks, num_blocks);
        const TC* src = vbase + ((int64_t)blk * hkv + hk) * tile + (int64_t)d * BLK + (pos % BLK);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                         (lds_void*)(v_lds + j * 512), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kVPieces; ++i) {
        const int pi = lane + 64 * (wave + kWaves * i);
        const int d = pi / (kStage / 8), piece = pi % (kStage / 8);
        const int pos = key0 + piece * 8;
        VPiece w = {};
        if (pos < kv_len) {
          const int blk = block_of(bt, pos, max_blocks, num_blocks);
          w = *reinterpret_cast<const VPiece*>(vbase + ((int64_t)blk * hkv + hk) * tile + (int64_t)d * BLK + (pos % BLK));
        }
        vr[i] = w;
      }
    }
  }

  // Convert and write the register-staged pieces of stage `st` into LDS.
  __device__ __forceinline__ void commit(int st, int kv_len, TQ* k_lds, f16_t* v_lds, int wave, int lane) {
    const int key0 = st * kStage;
    if constexpr (!T::kKDirect) {
      typedef typename Frag<TQ>::type F;
#pragma unroll
      for (int i = 0; i < kKPieces; ++i) {
        const int pi = lane + 64 * (wave + kWaves * i);
        const int row = pi / (D / 16), q = pi % (D / 16);
        u32x2 lo = {kr[i][0], kr[i][1]}, hi = {kr[i][2], kr[i][3]};
        *reinterpret_cast<F*>(k_lds + k_off<D>(row, 2 * q)) = fp8x8_to<TQ>(lo);
        *reinterpret_cast<F*>(k_lds + k_off<D>(row, 2 * q + 1)) = fp8x8_to<TQ>(hi);
      }
    }
    if constexpr (!T::kVDirect) {
#pragma unroll
      for (int i = 0; i < kVPieces; ++i) {
        const int pi = lane + 64 * (wave + kWaves * i);
        const int d = pi / (kStage / 8), piece = pi % (kStage / 8);
        const int pos = key0 + piece * 8;
        f16x8 f;
        if constexpr (T::kFp8) {
          f = fp8x8_to<f16_t>(vr[i]);  // exact: every e4m3fn value is an f16 value
        } else if constexpr (!T::kVScaled) {
          f = __builtin_bit_cast(f16x8, vr[i]);  // f16 cache: as stored
        } else {                       // bf16 -> f16 with the 2^-8 range scaling, saturating
          const bf16x8 b = __builtin_bit_cast(bf16x8, vr[i]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float x = (float)b[e] * 0.00390625f;
            x = fminf(fmaxf(x, -65504.f), 65504.f);
            f[e] = (f16_t)x;
          }
        }
        if (pos + 8 > kv_len) {  // keys past the end meet P = 0; 0 * NaN would be NaN
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = pos + e < kv_len ? f[e] : (f16_t)0.f;
        }
        *reinterpret_cast<f16x8*>(v_lds + v_off(d, piece)) = f;
      }
    }
  }
};

template <typename TQ, typename TC, int D, int BLK>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillParams p) {
  typedef Types<TQ, TC> T;
  typedef typename Frag<TQ>::type F;
  constexpr int QS = D / 16;  // k-steps of the score product
  constexpr int NT = D / 32;  // dim tiles of the output
  constexpr int kKElems = kStage * D, kVElems = D * kStage;
  __shared__ __attribute__((aligned(16))) TQ k_lds_all[2 * kKElems];
  __shared__ __attribute__((aligned(16))) f16_t v_lds_all[2 * kVElems];

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
  Stage<TQ, TC, D, BLK> stg;

  if (nst > 0) {
    stg.issue(kbase, vbase, bt, hk, p.hkv, p.num_blocks, p.max_blocks, 0, kv_len, k_lds_all, v_lds_all, wave, lane);
    stg.commit(0, kv_len, k_lds_all, v_lds_all, wave, lane);
  }
  __builtin_amdgcn_s_waitcnt(0);  // direct-to-LDS loads of stage 0 have landed
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    TQ* k_lds = k_lds_all + buf * kKElems;
    f16_t* v_lds = v_lds_all + buf * kVElems;
    TQ* k_nxt = k_lds_all + (buf ^ 1) * kKElems;
    f16_t* v_nxt = v_lds_all + (buf ^ 1) * kVElems;
    if (st + 1 < nst)
      stg.issue(kbase, vbase, bt, hk, p.hkv, p.num_blocks, p.max_blocks, st + 1, kv_len, k_nxt, v_nxt, wave, lane);

#pragma unroll
    for (int t = 0; t < kStage / 32; ++t) {
      const int key0 = st * kStage + 32 * t;  // first key of the sub-tile
      if (key0 < keys_w) {                    // uniform per wave
        // scores: element i = key key0 + 16*h0 + i, row c32
        f32x16 s = {};
        const int krow = 32 * t + krow_perm;
#pragma unroll
        for (int c = 0; c < QS; ++c) {
          const F kf = *reinterpret_cast<const F*>(k_lds + k_off<D>(krow, 2 * c + h0));
          s = mfma32x32x16(kf, qf[c], s);
        }
        float sc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] = s[i] * p.qk_scale_log2;
        if (key0 + 32 > full_keys_w) {
          const int kb = key0 + 16 * h0;
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[i] = (kb + i <= lim && kb + i < kv_len) ? sc[i] : -INFINITY;
        }
        float cmax = sc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) cmax = fmaxf(cmax, sc[i]);
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
        // lazy rescale: move the running max only when it grows by more than 2^kLazy
        const bool grow = cmax > m_run + kLazy;
        if (__any(grow)) {
          const float m_new = grow ? cmax : m_run;
          const float alpha = exp2f(m_run - m_new);  // 1 for rows that keep their max
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[n] *= alpha;
        }
        float pr[16];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) { pr[i] = exp2f(sc[i] - m_run); psum += pr[i]; }
        l_run += psum;
        const f16x8 p0 = pack8<f16_t>(pr), p1 = pack8<f16_t>(pr + 8);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const int d = 32 * n + c32;
          const f16x8 v0 = *reinterpret_cast<const f16x8*>(v_lds + v_off(d, 4 * t + 2 * h0));
          const f16x8 v1 = *reinterpret_cast<const f16x8*>(v_lds + v_off(d, 4 * t + 2 * h0 + 1));
          acc[n] = mfma32x32x16(v0, p0, acc[n]);
          acc[n] = mfma32x32x16(v1, p1, acc[n]);
        }
      }
    }

    if (st + 1 < nst) stg.commit(st + 1, kv_len, k_nxt, v_nxt, wave, lane);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct-to-LDS loads of the next stage have landed
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l; element i of acc[n] is dim 32n + 8(i/4) + 4h0 + i%4 ----
  l_run += __shfl_xor(l_run, 32);
  if (rvalid) {
    const float vback = T::kVScaled ? 256.f : 1.f;
    const float inv = p.v_scale * vback / l_run;
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
