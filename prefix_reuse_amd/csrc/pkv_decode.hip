// Paged decode attention for gfx950.
//
// What it computes (page "KV Cache에 대해 알아보자 (Feat. Attention)" §1 and
// §3; page "PagedAttention과 RadixAttention으로 LLM KV 캐시 최적화" §02): for
// each sequence s and query head h, out[s,h] = softmax(scale * q[s,h] K^T) V
// over the context_lens[s] cached tokens, whose rows are found through the
// block table, with query head h reading KV head h / G.
//
// Design (decode is bound by reading the KV cache from HBM):
//  * One work-group of 4 waves per (KV head, sequence, context split). The
//    whole GQA group (up to 16 query heads) is served from one read of K and V.
//  * Each wave walks 32-token chunks of its split (chunk k goes to wave k % 4).
//    Both products run on the matrix cores with operands loaded straight from
//    global memory in 16-byte pieces:
//      S^T[token][head] = K[token][:] . Q[head][:]     (A = K rows, B = Q^T)
//      O^T[dim][head]  += V^T[dim][token] . P^T[token][head]
//    The second product needs V with tokens contiguous, which is why the V
//    cache stores each (block, head) tile as [d][B]. K rows are loaded in a
//    permuted order so that the score tile leaves each lane holding 8
//    consecutive tokens of one head: exactly the B operand of the PV product,
//    and exactly 8 contiguous tokens of a V^T row.
//  * Online softmax in base 2 with the scale folded into one multiplier; the
//    running max is made uniform across the wave with two lane exchanges.
//  * The 4 waves merge through LDS in a fixed order. With one split the result
//    is written directly; otherwise an unnormalised partial (O, m, l) goes to
//    the workspace and a combine kernel merges splits in a fixed order, so the
//    result is bitwise deterministic and depends only on logical positions.
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

#include <math.h>
#include <stdlib.h>
#include <type_traits>

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 32;

template <typename TQ, typename TC, int D>
struct QFrag {
  static constexpr bool kF32 = std::is_same<TC, float>::value;
  static constexpr int kSteps = kF32 ? D / 4 : D / 32;
  typedef typename std::conditional<kF32, float, typename Frag<TQ>::type>::type T;
};

// Load the B operand of the score product: Q^T for the lane's head.
// 16-bit cache: step c covers dims 32c + 8g .. +8.
// fp8 cache:    step c = 2u + h covers dims 64u + 16g + 8h .. +8 (matches the
//               16-byte K loads, which carry 16 fp8 codes = two steps).
// f32 cache:    step c = 4u + e covers dim 16u + 4g + e.
template <typename TQ, typename TC, int D, typename QT>
__device__ __forceinline__ void load_q(QT* qf, const TQ* qrow, bool valid, int g) {
  constexpr int S = QFrag<TQ, TC, D>::kSteps;
  if constexpr (std::is_same<TC, float>::value) {
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (valid) v = *reinterpret_cast<const f32x4*>(qrow + 16 * u + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * u + e] = v[e];
    }
  } else {
#pragma unroll
    for (int c = 0; c < S; ++c) {
      int d0 = std::is_same<TC, uint8_t>::value ? 64 * (c / 2) + 16 * g + 8 * (c % 2) : 32 * c + 8 * g;
      typename Frag<TQ>::type v = {};
      if (valid) v = load_frag8(qrow + d0);
      qf[c] = v;
    }
  }
}

// Registers holding one 32-token chunk of K and V for one lane, as loaded.
// K: the lane's A-operand rows of the two 16-token score tiles; piece c of a
//    row covers dims c*4E + g*E .. +E, E = 16 / sizeof(TC) (16 bytes).
// V: for each 16-dim output tile n, 8 consecutive tokens of V^T row 16n + c16.
template <typename TC, int D>
struct ChunkRegs {
  static constexpr int E = 16 / sizeof(TC);
  static constexpr int KN = D / (4 * E);
  static constexpr int NT = D / 16;
  static constexpr int VW = 8 * sizeof(TC) / 4;  // 32-bit words per V piece
  u32x4 k[2][KN];
  uint32_t v[NT][VW];
};

template <typename TC, int D, int BLK>
__device__ __forceinline__ void load_chunk(ChunkRegs<TC, D>& r, const TC* kbase, const TC* vbase,
                                           int blk0, int blk1, int hk, int hkv, int c16, int g) {
  typedef ChunkRegs<TC, D> R;
  const int64_t tile = (int64_t)BLK * D;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int tok = 8 * (c16 / 4) + 4 * a + (c16 % 4);  // chunk-relative token of this A row
    const int blk = (BLK == 32 || tok < 16) ? blk0 : blk1;
    const TC* krow = kbase + ((int64_t)blk * hkv + hk) * tile + (int64_t)(tok % BLK) * D + g * R::E;
#pragma unroll
    for (int c = 0; c < R::KN; ++c) r.k[a][c] = load_u32x4(krow + c * 4 * R::E);
  }
  const int tokv = 8 * g;
  const int blkv = (BLK == 32 || tokv < 16) ? blk0 : blk1;
  const TC* vt = vbase + ((int64_t)blkv * hkv + hk) * tile + (tokv % BLK) + (int64_t)c16 * BLK;
#pragma unroll
  for (int n = 0; n < R::NT; ++n) {
    const TC* vr = vt + (int64_t)16 * n * BLK;
    if constexpr (R::VW == 2) {
      u32x2 w = load_u32x2(vr);
      r.v[n][0] = w[0]; r.v[n][1] = w[1];
    } else {
#pragma unroll
      for (int h = 0; h < R::VW / 4; ++h) {
        u32x4 w = load_u32x4(vr + h * (16 / sizeof(TC)));
#pragma unroll
        for (int e = 0; e < 4; ++e) r.v[n][4 * h + e] = w[e];
      }
    }
  }
}

// Scores of the 16-token tile a from loaded K rows: result element i is the
// score of chunk token 8g + 4a + i for head c16.
template <typename TQ, typename TC, int D, typename QT>
__device__ __forceinline__ f32x4 score_tile(const ChunkRegs<TC, D>& r, int a, const QT* qf) {
  typedef ChunkRegs<TC, D> R;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < R::KN; ++c) {
    if constexpr (std::is_same<TC, float>::value) {
      f32x4 kv = __builtin_bit_cast(f32x4, r.k[a][c]);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = mfma16x16x4(kv[e], qf[4 * c + e], s);
    } else if constexpr (std::is_same<TC, uint8_t>::value) {
      u32x2 lo = {r.k[a][c][0], r.k[a][c][1]}, hi = {r.k[a][c][2], r.k[a][c][3]};
      s = mfma16x16x32(fp8x8_to<TQ>(lo), qf[2 * c], s);
      s = mfma16x16x32(fp8x8_to<TQ>(hi), qf[2 * c + 1], s);
    } else {
      s = mfma16x16x32(__builtin_bit_cast(typename Frag<TQ>::type, r.k[a][c]), qf[c], s);
    }
  }
  return s;
}

template <typename TQ, typename TC, int D, int BLK>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams p) {
  typedef typename QFrag<TQ, TC, D>::T QT;
  typedef ChunkRegs<TC, D> R;
  constexpr int QS = QFrag<TQ, TC, D>::kSteps;
  constexpr int NT = D / 16;  // output dim tiles
  constexpr int LDS_ROW = D + 4;
  constexpr bool kSplitP = std::is_same<TQ, bf16_t>::value;  // bf16 P as hi + lo

  extern __shared__ float smem[];
  const int nh_max = min(16, p.group);
  float* s_acc = smem;                                  // [kWaves][nh_max][LDS_ROW]
  float* s_m = smem + kWaves * nh_max * LDS_ROW;        // [kWaves][nh_max]
  float* s_l = s_m + kWaves * nh_max;                   // [kWaves][nh_max]

  const int logical = xcd_remap(blockIdx.x, p.total_wgs);
  const int split = logical % p.num_splits;
  const int rest = logical / p.num_splits;
  const int seq = rest % p.num_seqs;
  const int hkc = rest / p.num_seqs;  // kv head * head_chunks + chunk
  const int hk = hkc / p.head_chunks;
  const int hchunk = hkc % p.head_chunks;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // uniform: scalar table reads
  const int lane = tid % 64;
  const int g = lane / 16, c16 = lane % 16;

  const int cap = p.max_blocks * BLK;
  int ctx = p.context_lens[seq];
  ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
  const int t0 = split * p.split_len;
  const int nh = min(16, p.group - hchunk * 16);  // valid query heads in this work-group

  if (t0 >= ctx) {
    if (p.num_splits == 1) {  // empty context: zero output rows
      for (int idx = tid; idx < nh * D; idx += kThreads) {
        int h = idx / D, d = idx % D;
        int qh = hk * p.group + hchunk * 16 + h;
        reinterpret_cast<TQ*>(p.out)[seq * p.o_s0 + qh * p.o_s1 + d] = from_f32<TQ>(0.f);
      }
    }
    return;
  }
  const int t1 = min(t0 + p.split_len, ctx);

  // ---- Q fragments (zero for padding heads) ----
  const bool hvalid = c16 < nh;
  const int qh_lane = hk * p.group + hchunk * 16 + (hvalid ? c16 : 0);
  const TQ* qrow = reinterpret_cast<const TQ*>(p.q) + seq * p.q_s0 + qh_lane * p.q_s1;
  QT qf[QS];
  load_q<TQ, TC, D>(qf, qrow, hvalid, g);

  const int32_t* bt = p.block_tables + seq * p.bt_s0;
  const TC* kbase = reinterpret_cast<const TC*>(p.k_cache);
  const TC* vbase = reinterpret_cast<const TC*>(p.v_cache);

  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  auto blocks_of = [&](int tb, int& b0, int& b1) {
    const int jb = tb / BLK;
    b0 = bt[jb];
    b1 = b0;
    if constexpr (BLK == 16) {
      if ((jb + 1) * BLK < t1) b1 = bt[jb + 1];  // only entries that hold live tokens
    }
    b0 = min(max(b0, 0), p.num_blocks - 1);
    b1 = min(max(b1, 0), p.num_blocks - 1);
  };

  auto compute = [&](const R& r, int tb) {
    float sc[8];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      f32x4 s = score_tile<TQ, TC, D>(r, a, qf);
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * a + i] = s[i] * p.qk_scale_log2;
    }
    // lane (g, c16) holds chunk tokens tb + 8g + j, j = 0..7, of head c16
    const int nvalid = min(max(t1 - (tb + 8 * g), 0), 8);
    const bool tail = tb + kChunk > t1;
    if (tail) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sc[j] = j < nvalid ? sc[j] : -INFINITY;
    }
    float cmax = sc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) cmax = fmaxf(cmax, sc[j]);
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = exp2f(m_run - m_new);
    float pj[8];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) { pj[j] = exp2f(sc[j] - m_new); psum += pj[j]; }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] *= alpha;

    // ---- PV: O^T[d][head] += V^T[d][8 tokens] . P^T[8 tokens][head] ----
    if constexpr (std::is_same<TC, float>::value) {
#pragma unroll
      for (int n = 0; n < NT; ++n) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float x = __builtin_bit_cast(float, r.v[n][j]);
          x = (tail && j >= nvalid) ? 0.f : x;
          acc[n] = mfma16x16x4(x, pj[j], acc[n]);
        }
      }
    } else {
      typedef typename Frag<TQ>::type F;
      const F phi = pack8<TQ>(pj);
      F plo;
      if constexpr (kSplitP) {
        float lo[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) lo[j] = pj[j] - (float)phi[j];  // exact in fp32
        plo = pack8<TQ>(lo);
      }
      F vf[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if constexpr (std::is_same<TC, uint8_t>::value) vf[n] = fp8x8_to<TQ>(u32x2{r.v[n][0], r.v[n][1]});
        else vf[n] = __builtin_bit_cast(F, u32x4{r.v[n][0], r.v[n][1], r.v[n][2], r.v[n][3]});
      }
      if (tail) {  // tokens past the end may hold anything (NaN): 0 * NaN is NaN
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int j = 0; j < 8; ++j) vf[n][j] = j < nvalid ? vf[n][j] : (TQ)0.f;
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        acc[n] = mfma16x16x32(vf[n], phi, acc[n]);
        if constexpr (kSplitP) acc[n] = mfma16x16x32(vf[n], plo, acc[n]);
      }
    }
  };

  // ---- two-stage register pipeline over this wave's chunks ----
  // The next chunk's loads are always issued (past the end they re-read the
  // current chunk's addresses), so every iteration has the same number of
  // loads in flight and the waits before each product cover only its own data.
  R bufA, bufB;
  int tb = t0 + wave * kChunk;
  constexpr int kStride = kWaves * kChunk;
  if (tb < t1) {
    int b0, b1;
    blocks_of(tb, b0, b1);
    load_chunk<TC, D, BLK>(bufA, kbase, vbase, b0, b1, hk, p.hkv, c16, g);
    for (;;) {
      int tn = tb + kStride;
      bool more = tn < t1;
      int n0 = b0, n1 = b1;
      if (more) blocks_of(tn, n0, n1);
      load_chunk<TC, D, BLK>(bufB, kbase, vbase, n0, n1, hk, p.hkv, c16, g);
      compute(bufA, tb);
      if (!more) break;
      tb = tn;
      b0 = n0; b1 = n1;
      tn = tb + kStride;
      more = tn < t1;
      if (more) blocks_of(tn, n0, n1);
      load_chunk<TC, D, BLK>(bufA, kbase, vbase, n0, n1, hk, p.hkv, c16, g);
      compute(bufB, tb);
      if (!more) break;
      tb = tn;
      b0 = n0; b1 = n1;
    }
  }

  // ---- merge the lane groups' partial sums, then the 4 waves through LDS ----
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (c16 < nh) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
      *reinterpret_cast<f32x4*>(&s_acc[(wave * nh_max + c16) * LDS_ROW + 16 * n + 4 * g]) = acc[n];
    if (g == 0) { s_m[wave * nh_max + c16] = m_run; s_l[wave * nh_max + c16] = l_run; }
  }
  __syncthreads();

  for (int idx = tid; idx < nh * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float M = s_m[h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w * nh_max + h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = exp2f(s_m[w * nh_max + h] - M);  // 0 for a wave that saw no token
      L += s_l[w * nh_max + h] * f;
      O += s_acc[(w * nh_max + h) * LDS_ROW + d] * f;
    }
    const int qh = hk * p.group + hchunk * 16 + h;
    if (p.num_splits == 1) {
      reinterpret_cast<TQ*>(p.out)[seq * p.o_s0 + qh * p.o_s1 + d] = from_f32<TQ>(O / L * p.v_scale);
    } else {
      const int64_t row = ((int64_t)seq * p.hq + qh) * p.num_splits + split;
      p.ws_o[row * D + d] = O;
      if (d == 0) { p.ws_ml[row * 2] = M; p.ws_ml[row * 2 + 1] = L; }
    }
  }
}

// Merge the splits of one (sequence, query head) in split order.
template <typename TQ, int D, int BLK>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeParams p) {
  const int seq = blockIdx.x / p.hq, qh = blockIdx.x % p.hq;
  const int d = threadIdx.x;
  const int cap = p.max_blocks * BLK;
  int ctx = p.context_lens[seq];
  ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
  const int n = (ctx + p.split_len - 1) / p.split_len;
  TQ* out = reinterpret_cast<TQ*>(p.out) + seq * p.o_s0 + qh * p.o_s1;
  if (n == 0) { out[d] = from_f32<TQ>(0.f); return; }
  const int64_t row0 = ((int64_t)seq * p.hq + qh) * p.num_splits;
  float M = -INFINITY;
  for (int i = 0; i < n; ++i) M = fmaxf(M, p.ws_ml[(row0 + i) * 2]);
  float L = 0.f, O = 0.f;
  for (int i = 0; i < n; ++i) {
    const float f = exp2f(p.ws_ml[(row0 + i) * 2] - M);
    L += p.ws_ml[(row0 + i) * 2 + 1] * f;
    O += p.ws_o[(row0 + i) * D + d] * f;
  }
  out[d] = from_f32<TQ>(O / L * p.v_scale);
}

template <typename TQ, typename TC, int D, int BLK>
hipError_t launch_typed(const DecodeParams& p, hipStream_t stream) {
  const int nh_max = p.group < 16 ? p.group : 16;
  const size_t lds = (size_t)kWaves * nh_max * ((D + 4) + 2) * sizeof(float);
  hipLaunchKernelGGL((decode_kernel<TQ, TC, D, BLK>), dim3(p.total_wgs), dim3(kThreads), lds, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_splits == 1) return e;
  hipLaunchKernelGGL((decode_combine_kernel<TQ, D, BLK>), dim3(p.num_seqs * p.hq), dim3(D), 0, stream, p);
  return hipGetLastError();
}

template <typename TQ, typename TC>
hipError_t launch_shape(const DecodeParams& p, int d, int b, hipStream_t s) {
  if (d == 128 && b == 16) return launch_typed<TQ, TC, 128, 16>(p, s);
  if (d == 128 && b == 32) return launch_typed<TQ, TC, 128, 32>(p, s);
  if (d == 64 && b == 16) return launch_typed<TQ, TC, 64, 16>(p, s);
  if (d == 64 && b == 32) return launch_typed<TQ, TC, 64, 32>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace

SplitPlan plan_decode_splits(int64_t num_seqs, int32_t hkv, int32_t head_chunks, int64_t max_ctx,
                             int32_t num_cus) {
  // Aim for about 8 work-groups per compute unit in total; never split below
  // 256 tokens; split lengths are whole multiples of 4 waves x 32 tokens.
  // PKV_DECODE_SPLIT_LEN (a positive multiple of 128) forces the split length.
  if (const char* env = getenv("PKV_DECODE_SPLIT_LEN")) {
    const long forced = atol(env);
    if (forced >= 128 && forced % 128 == 0) {
      int64_t splits = (max_ctx + forced - 1) / forced;
      return SplitPlan{(int32_t)(splits < 1 ? 1 : splits), (int32_t)forced};
    }
  }
  const int64_t units = num_seqs * hkv * head_chunks;
  const int64_t target = 8LL * (num_cus > 0 ? num_cus : 256);
  int64_t splits = units > 0 ? (target + units - 1) / units : 1;
  const int64_t max_splits = (max_ctx + 255) / 256;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t len = (max_ctx + splits - 1) / splits;
  len = ((len + 127) / 128) * 128;
  if (len < 128) len = 128;
  splits = (max_ctx + len - 1) / len;
  if (splits < 1) splits = 1;
  return SplitPlan{(int32_t)splits, (int32_t)len};
}

hipError_t launch_decode(const DecodeParams& p, DT q_dt, DT cache_dt, int d, int b, hipStream_t s) {
  if (q_dt == DT::F32 && cache_dt == DT::F32) return launch_shape<float, float>(p, d, b, s);
  if (q_dt == DT::F16 && cache_dt == DT::F16) return launch_shape<f16_t, f16_t>(p, d, b, s);
  if (q_dt == DT::BF16 && cache_dt == DT::BF16) return launch_shape<bf16_t, bf16_t>(p, d, b, s);
  if (q_dt == DT::F16 && cache_dt == DT::FP8) return launch_shape<f16_t, uint8_t>(p, d, b, s);
  if (q_dt == DT::BF16 && cache_dt == DT::FP8) return launch_shape<bf16_t, uint8_t>(p, d, b, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv
