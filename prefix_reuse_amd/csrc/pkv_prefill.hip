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
//    rows of one (request, KV head); each wave owns 32 rows.
//  * Keys are consumed 32 at a time. The work-group stages the K tile
//    [32 keys][d] and the V^T tile [d][32 keys] in LDS (double buffered: the
//    global loads for tile j+1 are in flight while tile j is computed). fp8
//    caches are converted to 16-bit while staging.
//  * Per wave and key tile, on v_mfma_f32_32x32x16:
//      S^T[key][row] = K[key][:] . Q[row][:]        (Q^T held in registers)
//      O^T[dim][row] += V^T[dim][keys] . P^T[keys][row]
//    K rows are read from LDS in a permuted order so that each lane ends up
//    holding 16 consecutive keys of one row: the B operand of the PV product
//    and 16-byte contiguous reads of the V^T tile.
//  * Online softmax in base 2 per row; the causal mask is applied only on key
//    tiles that reach past the wave's first token.
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
constexpr int kKeys = 32;

template <typename TQ, int D>
struct Smem {
  static constexpr int KROW = D + 8;      // padded K row (elements)
  static constexpr int VROW = kKeys + 8;  // padded V^T row (elements)
  TQ k[2][kKeys][KROW];
  TQ v[2][D][VROW];
};

// Global -> register staging of one key tile, then register -> LDS.
template <typename TQ, typename TC, int D, int BLK>
struct Stager {
  static constexpr bool kFp8 = std::is_same<TC, uint8_t>::value;
  // K: pieces of 8 consecutive dims of a cache row; V: pieces of 8 consecutive
  // tokens of a V^T row. 16-bit pieces are 16 bytes, fp8 pieces 8 bytes.
  static constexpr int kKPieces = kKeys * D / 8 / kThreads;  // per thread
  static constexpr int kVPieces = D * kKeys / 8 / kThreads;
  typedef typename std::conditional<kFp8, u32x2, u32x4>::type Piece;
  Piece kr[kKPieces];
  Piece vr[kVPieces];

  __device__ __forceinline__ void load(const TC* kbase, const TC* vbase, const int32_t* bt,
                                       int hk, int hkv, int num_blocks, int max_blocks, int kt,
                                       int kv_len, int tid) {
    const int key0 = kt * kKeys;
#pragma unroll
    for (int i = 0; i < kKPieces; ++i) {
      const int pi = tid + i * kThreads;
      const int key = pi / (D / 8);
      const int d0 = (pi % (D / 8)) * 8;
      const int pos = key0 + key;
      Piece z = {};
      if (pos < kv_len) {
        int jb = pos / BLK;
        jb = jb < max_blocks ? jb : max_blocks - 1;
        int blk = bt[jb];
        blk = min(max(blk, 0), num_blocks - 1);
        const TC* src = kbase + ((int64_t)blk * hkv + hk) * (BLK * D) + (int64_t)(pos % BLK) * D + d0;
        z = *reinterpret_cast<const Piece*>(src);
      }
      kr[i] = z;
    }
#pragma unroll
    for (int i = 0; i < kVPieces; ++i) {
      const int pi = tid + i * kThreads;
      const int d = pi / (kKeys / 8);
      const int kq = (pi % (kKeys / 8)) * 8;
      const int pos = key0 + kq;  // 8 consecutive keys, all in one block
      Piece w = {};
      if (pos < kv_len) {
        int jb = pos / BLK;
        jb = jb < max_blocks ? jb : max_blocks - 1;
        int blk = bt[jb];
        blk = min(max(blk, 0), num_blocks - 1);
        const TC* src = vbase + ((int64_t)blk * hkv + hk) * (BLK * D) + (int64_t)d * BLK + (pos % BLK);
        w = *reinterpret_cast<const Piece*>(src);
      }
      vr[i] = w;
    }
  }

  __device__ __forceinline__ void store(Smem<TQ, D>& sm, int buf, int kt, int kv_len, int tid) {
    typedef typename Frag<TQ>::type F;
    const int key0 = kt * kKeys;
#pragma unroll
    for (int i = 0; i < kKPieces; ++i) {
      const int pi = tid + i * kThreads;
      const int key = pi / (D / 8);
      const int d0 = (pi % (D / 8)) * 8;
      F f;
      if constexpr (kFp8) f = fp8x8_to<TQ>(kr[i]);
      else f = __builtin_bit_cast(F, kr[i]);
      *reinterpret_cast<F*>(&sm.k[buf][key][d0]) = f;
    }
#pragma unroll
    for (int i = 0; i < kVPieces; ++i) {
      const int pi = tid + i * kThreads;
      const int d = pi / (kKeys / 8);
      const int kq = (pi % (kKeys / 8)) * 8;
      const int pos = key0 + kq;
      F f;
      if constexpr (kFp8) f = fp8x8_to<TQ>(vr[i]);
      else f = __builtin_bit_cast(F, vr[i]);
      if (pos + 8 > kv_len) {  // zero values past the end: they meet P = 0, and 0 * NaN is NaN
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = pos + j < kv_len ? f[j] : (TQ)0.f;
      }
      *reinterpret_cast<F*>(&sm.v[buf][d][kq]) = f;
    }
  }
};

template <typename TQ, typename TC, int D, int BLK>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
  typedef typename Frag<TQ>::type F;
  constexpr int QS = D / 16;  // k-steps of the score product
  constexpr int NT = D / 32;  // dim tiles of the output
  constexpr bool kSplitP = std::is_same<TQ, bf16_t>::value;
  __shared__ Smem<TQ, D> sm;

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
  if (kv_len > cap) { kv_len = cap; }
  const int32_t* bt = p.block_tables + (int64_t)r * p.bt_s0;

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int h0 = lane / 32, c32 = lane % 32;

  const int q0 = tile * kRowsWg;                  // first row of the work-group
  const int tok_last_wg = min(S - 1, (q0 + kRowsWg - 1) / p.group);
  const int wq0 = q0 + wave * kRowsWave;          // first row of this wave
  const int tok_first_w = wq0 / p.group;
  const int tok_last_w = min(S - 1, (wq0 + kRowsWave - 1) / p.group);
  const bool wave_active = wq0 < rows_r;
  const int nkt = (min(kv_len, P + tok_last_wg + 1) + kKeys - 1) / kKeys;
  const int nkt_w = wave_active ? (min(kv_len, P + tok_last_w + 1) + kKeys - 1) / kKeys : 0;
  const int full_w = (P + tok_first_w + 1) / kKeys;  // tiles needing no causal mask

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

  // permuted key row read by this lane for the A operand of the score product
  const int krow_perm = 16 * ((c32 % 8) / 4) + 4 * (c32 / 8) + (c32 % 4);

  f32x16 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const TC* kbase = reinterpret_cast<const TC*>(p.k_cache);
  const TC* vbase = reinterpret_cast<const TC*>(p.v_cache);
  Stager<TQ, TC, D, BLK> st;
  if (nkt > 0) {
    st.load(kbase, vbase, bt, hk, p.hkv, p.num_blocks, p.max_blocks, 0, kv_len, tid);
    st.store(sm, 0, 0, kv_len, tid);
  }
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) st.load(kbase, vbase, bt, hk, p.hkv, p.num_blocks, p.max_blocks, kt + 1, kv_len, tid);

    if (kt < nkt_w) {
      // scores: S^T tile, element i = key kt*32 + 16*h0 + i, row c32
      f32x16 s = {};
#pragma unroll
      for (int c = 0; c < QS; ++c) {
        F kf = *reinterpret_cast<const F*>(&sm.k[buf][krow_perm][16 * c + 8 * h0]);
        s = mfma32x32x16(kf, qf[c], s);
      }
      float sc[16];
      const int key0 = kt * kKeys + 16 * h0;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = s[i] * p.qk_scale_log2;
      if (kt >= full_w) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] = (key0 + i <= lim) ? sc[i] : -INFINITY;
      }
      float cmax = sc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) cmax = fmaxf(cmax, sc[i]);
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = exp2f(m_run - m_new);
      float pr[16];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) { pr[i] = exp2f(sc[i] - m_new); psum += pr[i]; }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] *= alpha;
      const F p0 = pack8<TQ>(pr), p1 = pack8<TQ>(pr + 8);
      F p0lo, p1lo;
      if constexpr (kSplitP) {  // bf16 P carries 8 bits: add the rounding remainder as a second term
        float lo[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) { lo[i] = pr[i] - (float)p0[i]; lo[8 + i] = pr[8 + i] - (float)p1[i]; }
        p0lo = pack8<TQ>(lo);
        p1lo = pack8<TQ>(lo + 8);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const F v0 = *reinterpret_cast<const F*>(&sm.v[buf][32 * n + c32][16 * h0]);
        const F v1 = *reinterpret_cast<const F*>(&sm.v[buf][32 * n + c32][16 * h0 + 8]);
        acc[n] = mfma32x32x16(v0, p0, acc[n]);
        acc[n] = mfma32x32x16(v1, p1, acc[n]);
        if constexpr (kSplitP) {
          acc[n] = mfma32x32x16(v0, p0lo, acc[n]);
          acc[n] = mfma32x32x16(v1, p1lo, acc[n]);
        }
      }
    }

    if (kt + 1 < nkt) st.store(sm, buf ^ 1, kt + 1, kv_len, tid);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, element i of acc[n] is dim 32n + 8(i/4) + 4h0 + i%4 ----
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
