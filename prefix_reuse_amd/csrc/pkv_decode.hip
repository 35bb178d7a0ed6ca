// Paged decode attention for gfx950.
//
// What it computes (page "KV Cache에 대해 알아보자 (Feat. Attention)" §1 and
// §3; page "PagedAttention과 RadixAttention으로 LLM KV 캐시 최적화" §02): for
// each sequence s and query head h, out[s,h] = softmax(scale * q[s,h] K^T) V
// over the context_lens[s] cached tokens, whose rows are found through the
// block table, with query head h reading KV head h / G.
//
// Design (decode is bound by reading the KV cache from HBM):
//  * Balanced, persistent partition. Every 32-token chunk of every sequence
//    is one unit of work; for each KV head (and group of up to 16 query heads)
//    a fixed number of one-wave work-groups - as many as the chip holds at
//    once - each take an equal, contiguous range of the chunks in sequence
//    order. A wave keeps its softmax state across the chunks of a sequence and
//    writes a result only when it leaves the sequence: the final output if it
//    saw the whole sequence, else an unnormalised partial (O, m, l) that a
//    small combine kernel merges in wave order. Lengths that differ by 8x
//    therefore cost nothing in balance, and no wave idles on an empty split.
//  * The whole GQA group (up to 16 query heads) is served from one read of K
//    and V. Both products run on the matrix cores with operands loaded
//    straight from global memory in 16-byte pieces, all of a chunk's loads
//    issued before the first product:
//      S^T[token][head] = K[token][:] . Q[head][:]     (A = K rows, B = Q^T)
//      O^T[dim][head]  += V^T[dim][token] . P^T[token][head]
//    The second product needs V with tokens contiguous, which is why the V
//    cache stores each (block, head) tile as [d][B]. K rows are loaded in a
//    permuted order so that the score tile leaves each lane holding 8
//    consecutive tokens of one head: exactly the B operand of the PV product,
//    and exactly 8 contiguous tokens of a V^T row.
//  * Online softmax in base 2 with the scale folded into one multiplier; the
//    running max is made uniform across the wave with two lane exchanges.
//  * Results are bitwise deterministic; arithmetic order depends only on
//    logical positions and on the partition, never on timing.
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

#include <math.h>
#include <stdlib.h>
#include <type_traits>

namespace pkv {
namespace {

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

// Chunk bookkeeping of the balanced partition: every 32-token chunk of every
// sequence, in sequence order, is one unit of work; wave w of a KV head takes
// units [w * per_wave, (w + 1) * per_wave).
struct Partition {
  int total;     // chunks of all sequences
  int per_wave;  // ceil(total / waves per head)
};

__device__ __forceinline__ int ctx_of(const DecodeParams& p, int s, int cap) {
  int c = p.context_lens[s];
  return c < 0 ? 0 : (c > cap ? cap : c);
}

// Cascade decode: tokens of sequence s before this one belong to its group's
// shared prefix (whole blocks, cut to its context); 0 for a plain decode.
template <int BLK>
__device__ __forceinline__ int shared_of(const DecodeParams& p, int s, int ctx) {
  if (!p.shared_lens) return 0;
  int l = p.shared_lens[s];
  l = l < 0 ? 0 : l;
  l -= l % BLK;  // whole blocks, then cut to the context (a short sequence ends inside them)
  return l > ctx ? ctx : l;
}

// tokens the decode kernel covers: all of them, or those after the shared prefix
template <int BLK>
__device__ __forceinline__ int own_of(const DecodeParams& p, int s, int cap) {
  const int c = ctx_of(p, s, cap);
  return c - shared_of<BLK>(p, s, c);
}

// Wave-wide inclusive scan of one value per lane.
__device__ __forceinline__ int wave_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

template <typename TQ, typename TC, int D, int BLK>
__global__ __launch_bounds__(64, 3) void decode_kernel(DecodeParams p) {
  typedef typename QFrag<TQ, TC, D>::T QT;
  typedef ChunkRegs<TC, D> R;
  constexpr int QS = QFrag<TQ, TC, D>::kSteps;
  constexpr int NT = D / 16;  // output dim tiles
  constexpr bool kSplitP = std::is_same<TQ, bf16_t>::value;  // bf16 P as hi + lo

  const int logical = xcd_remap(blockIdx.x, p.total_wgs);
  const int hkc = logical / p.waves_per_head;  // kv head * head_chunks + chunk
  const int w = logical % p.waves_per_head;
  const int hk = hkc / p.head_chunks;
  const int hchunk = hkc % p.head_chunks;
  const int lane = threadIdx.x;
  const int g = lane / 16, c16 = lane % 16;
  const int cap = p.max_blocks * BLK;
  const int nh = min(16, p.group - hchunk * 16);

  // ---- partition: total chunks, this wave's range, its first sequence ----
  int total = 0;
  for (int b = 0; b < p.num_seqs; b += 64) {
    const int s = b + lane;
    int ch = s < p.num_seqs ? (own_of<BLK>(p, s, cap) + kChunk - 1) / kChunk : 0;
    total += __shfl(wave_scan(ch, lane), 63);
  }
  total = __builtin_amdgcn_readfirstlane(total);
  if (total == 0) return;
  const int per_wave = (total + p.waves_per_head - 1) / p.waves_per_head;
  const int c0 = w * per_wave;
  const int c1 = min(c0 + per_wave, total);
  // per-sequence partition info, written once for the combine kernel
  if (logical == 0) {
    int run = 0;
    for (int b = 0; b < p.num_seqs; b += 64) {
      const int s = b + lane;
      int ch = s < p.num_seqs ? (own_of<BLK>(p, s, cap) + kChunk - 1) / kChunk : 0;
      const int incl = run + wave_scan(ch, lane);
      const int first = incl - ch;
      if (s < p.num_seqs) {
        p.seq_info[2 * s] = ch > 0 ? first / per_wave : 0;                                // first wave
        p.seq_info[2 * s + 1] = ch > 0 ? (incl - 1) / per_wave - first / per_wave + 1 : 0;  // waves
      }
      run = __shfl(incl, 63);
    }
  }
  if (c0 >= c1) return;
  // first sequence of the range: the one whose chunks contain c0
  int s_cur = 0, s_first_chunk = 0;
  {
    int run = 0;
    for (int b = 0; b < p.num_seqs; b += 64) {
      const int s = b + lane;
      int ch = s < p.num_seqs ? (own_of<BLK>(p, s, cap) + kChunk - 1) / kChunk : 0;
      const int incl = run + wave_scan(ch, lane);
      const unsigned long long hit = __ballot(s < p.num_seqs && incl > c0);
      if (hit) {
        const int l0 = __builtin_ctzll(hit);
        s_cur = b + l0;
        s_first_chunk = __shfl(incl - ch, l0);
        break;
      }
      run = __shfl(incl, 63);
    }
  }
  s_cur = __builtin_amdgcn_readfirstlane(s_cur);
  s_first_chunk = __builtin_amdgcn_readfirstlane(s_first_chunk);

  const TC* kbase = reinterpret_cast<const TC*>(p.k_cache);
  const TC* vbase = reinterpret_cast<const TC*>(p.v_cache);
  const bool hvalid = c16 < nh;
  const int qh_lane = hk * p.group + hchunk * 16 + (hvalid ? c16 : 0);

  QT qf[QS];
  f32x4 acc[NT];
  float m_run, l_run;
  // ctx counts this kernel's tokens of s_cur; bt starts at the first of them
  auto table_of = [&](int s) {
    return p.block_tables + (int64_t)s * p.bt_s0 + shared_of<BLK>(p, s, ctx_of(p, s, cap)) / BLK;
  };
  int ctx = own_of<BLK>(p, s_cur, cap);
  int tb = (c0 - s_first_chunk) * kChunk;
  const int32_t* bt = table_of(s_cur);

  auto start_seq = [&]() {
    load_q<TQ, TC, D>(qf, reinterpret_cast<const TQ*>(p.q) + s_cur * p.q_s0 + qh_lane * p.q_s1, hvalid, g);
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
  };

  // write this wave's result for s_cur: final output if it saw the whole
  // sequence, else an unnormalised partial in slot (w + s_cur)
  auto finish_seq = [&](bool whole) {
    float l = l_run + __shfl_xor(l_run, 16);
    l += __shfl_xor(l, 32);
    if (!hvalid) return;
    const int qh = hk * p.group + hchunk * 16 + c16;
    if (whole) {
      const float inv = p.v_scale / l;
      TQ* o = reinterpret_cast<TQ*>(p.out) + s_cur * p.o_s0 + qh * p.o_s1;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        typedef __attribute__((__vector_size__(4 * sizeof(TQ)))) TQ TQx4;
        TQx4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = from_f32<TQ>(acc[n][i] * inv);
        *reinterpret_cast<TQx4*>(o + 16 * n + 4 * g) = v;
      }
    } else {
      const int64_t row = (int64_t)(w + s_cur) * p.hq + qh;
#pragma unroll
      for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4*>(p.ws_o + row * D + 16 * n + 4 * g) = acc[n];
      if (g == 0) { p.ws_ml[row * 2] = m_run; p.ws_ml[row * 2 + 1] = l; }
    }
  };

  start_seq();
  int seq_start = s_first_chunk;  // global index of s_cur's first chunk
  for (int c = c0; c < c1; ++c) {
    // ---- load the chunk ----
    const int jb = tb / BLK;
    int b0 = bt[jb], b1 = b0;
    if constexpr (BLK == 16) {
      if ((jb + 1) * BLK < ctx) b1 = bt[jb + 1];  // only entries that hold live tokens
    }
    b0 = min(max(b0, 0), p.num_blocks - 1);
    b1 = min(max(b1, 0), p.num_blocks - 1);
    R r;
    load_chunk<TC, D, BLK>(r, kbase, vbase, b0, b1, hk, p.hkv, c16, g);

    // ---- scores S^T for 32 tokens: two 16-token tiles ----
    float sc[8];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      f32x4 sv = score_tile<TQ, TC, D>(r, a, qf);
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * a + i] = sv[i] * p.qk_scale_log2;
    }
    // lane (g, c16) holds tokens tb + 8g + j, j = 0..7, of head c16
    const int nvalid = min(max(ctx - (tb + 8 * g), 0), 8);
    const bool tail = tb + kChunk > ctx;
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

    // ---- advance ----
    tb += kChunk;
    if (tb >= ctx || c + 1 == c1) {
      const int nch = (ctx + kChunk - 1) / kChunk;
      finish_seq(!p.shared_lens && seq_start >= c0 && seq_start + nch <= c1);  // cascade: always a partial
      if (c + 1 == c1) break;
      seq_start += nch;
      do {  // next non-empty sequence
        ++s_cur;
        ctx = own_of<BLK>(p, s_cur, cap);
      } while (ctx == 0);
      tb = 0;
      bt = table_of(s_cur);
      start_seq();
    }
  }
}

// Merge the partials of the sequences that several waves shared, in wave
// order. One work-group per (sequence, pair of query heads), so that even a
// handful of long sequences spreads over many work-groups; each thread owns 4
// consecutive dims of one head. Sequences that one wave covered entirely
// already hold their output; empty sequences get zero rows here.
constexpr int kCombineHeads = 2;

template <typename TQ, int D, int BLK>
__global__ __launch_bounds__(kCombineHeads * D / 4) void decode_combine_kernel(DecodeParams p) {
  const int groups = (p.hq + kCombineHeads - 1) / kCombineHeads;
  const int seq = blockIdx.x / groups;
  const int qh = (blockIdx.x % groups) * kCombineHeads + threadIdx.x / (D / 4);
  const int d0 = (threadIdx.x % (D / 4)) * 4;
  if (qh >= p.hq) return;
  const int cap = p.max_blocks * BLK;
  TQ* out = reinterpret_cast<TQ*>(p.out) + seq * p.o_s0 + qh * p.o_s1 + d0;
  typedef __attribute__((__vector_size__(4 * sizeof(TQ)))) TQ TQx4;
  const int ctx = ctx_of(p, seq, cap);
  if (ctx == 0) {
    TQx4 z;
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = from_f32<TQ>(0.f);
    *reinterpret_cast<TQx4*>(out) = z;
    return;
  }
  const int first = p.seq_info[2 * seq];
  int n = p.seq_info[2 * seq + 1];
  if (!p.shared_lens && n <= 1) return;
  if (own_of<BLK>(p, seq, cap) == 0) n = 0;  // cascade, nothing after the shared prefix
  const int64_t row0 = (int64_t)(first + seq) * p.hq + qh;  // slot of wave `first`
  float M = -INFINITY, L = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  // cascade: the shared prefix's partials (one per key chunk that reaches
  // into this sequence's shared tokens) join the merge first
  constexpr int kMaxSplits = 16;
  f32x2 sml[kMaxSplits];
  f32x4 so[kMaxSplits];
  int nsh = 0;
  if (p.shared_lens) {
    const int sh = shared_of<BLK>(p, seq, ctx);
    int lr = p.shared_lens[seq];
    lr = lr < 0 ? 0 : lr;
    lr -= lr % BLK;
    const int chunk = cascade_chunk(lr, p.sh_splits);
    nsh = chunk > 0 ? min((sh + chunk - 1) / chunk, min(p.sh_splits, kMaxSplits)) : 0;
  }
#pragma unroll
  for (int i = 0; i < kMaxSplits; ++i) {
    sml[i] = f32x2{-INFINITY, 0.f};
    so[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < nsh) {
      const int64_t srow = ((int64_t)i * p.num_seqs + seq) * p.hq + qh;
      sml[i] = *reinterpret_cast<const f32x2*>(p.sh_ml + srow * 2);
      so[i] = *reinterpret_cast<const f32x4*>(p.sh_o + srow * D + d0);
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxSplits; ++i) M = fmaxf(M, sml[i][0]);
  // one round of loads for up to kFew partials, then a general loop
  constexpr int kFew = 8;
  const int nf = n < kFew ? n : kFew;
  f32x2 ml[kFew];
  f32x4 o[kFew];
#pragma unroll
  for (int i = 0; i < kFew; ++i) {
    const int64_t row = row0 + (int64_t)i * p.hq;
    ml[i] = i < nf ? *reinterpret_cast<const f32x2*>(p.ws_ml + row * 2) : f32x2{-INFINITY, 0.f};
    o[i] = i < nf ? *reinterpret_cast<const f32x4*>(p.ws_o + row * D + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < kFew; ++i) M = fmaxf(M, ml[i][0]);
#pragma unroll
  for (int i = 0; i < kMaxSplits; ++i) {
    const float f = i < nsh ? exp2f(sml[i][0] - M) : 0.f;
    L += sml[i][1] * f;
    O += so[i] * f;
  }
#pragma unroll
  for (int i = 0; i < kFew; ++i) {
    const float f = i < nf ? exp2f(ml[i][0] - M) : 0.f;
    L += ml[i][1] * f;
    O += o[i] * f;
  }
  // further partials (long contexts spread over many waves) in batches of
  // kFew, each loaded in one round and merged under a running maximum
  for (int i0 = kFew; i0 < n; i0 += kFew) {
#pragma unroll
    for (int i = 0; i < kFew; ++i) {
      const int64_t row = row0 + (int64_t)(i0 + i) * p.hq;
      const bool ok = i0 + i < n;
      ml[i] = ok ? *reinterpret_cast<const f32x2*>(p.ws_ml + row * 2) : f32x2{-INFINITY, 0.f};
      o[i] = ok ? *reinterpret_cast<const f32x4*>(p.ws_o + row * D + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < kFew; ++i) Mb = fmaxf(Mb, ml[i][0]);
    const float r = exp2f(M - Mb);  // M is finite: the first round held a partial
    L *= r;
    O *= r;
    M = Mb;
#pragma unroll
    for (int i = 0; i < kFew; ++i) {
      const float f = i0 + i < n ? exp2f(ml[i][0] - M) : 0.f;
      L += ml[i][1] * f;
      O += o[i] * f;
    }
  }
  const float inv = p.v_scale / L;
  TQx4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = from_f32<TQ>(O[i] * inv);
  *reinterpret_cast<TQx4*>(out) = v;
}

template <typename TQ, typename TC, int D, int BLK>
hipError_t launch_typed(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<TQ, TC, D, BLK>), dim3(p.total_wgs), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int groups = (p.hq + kCombineHeads - 1) / kCombineHeads;
  hipLaunchKernelGGL((decode_combine_kernel<TQ, D, BLK>), dim3(p.num_seqs * groups), dim3(kCombineHeads * D / 4), 0,
                     stream, p);
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

DecodePlan plan_decode(int64_t num_seqs, int32_t hkv, int32_t head_chunks, int32_t num_cus) {
  // One wave per work-group, 8 waves per compute unit in total (2 per SIMD:
  // enough loads in flight to keep HBM busy, few enough that each wave's run
  // is long), split evenly over the (KV head, head chunk) pairs.
  // PKV_DECODE_WAVES (a positive integer) forces the total.
  int64_t waves = 8LL * (num_cus > 0 ? num_cus : 256);
  if (const char* env = getenv("PKV_DECODE_WAVES")) {
    const long forced = atol(env);
    if (forced > 0) waves = forced;
  }
  const int64_t units = (int64_t)hkv * head_chunks;
  int64_t per_head = waves / units;
  if (per_head < 1) per_head = 1;
  (void)num_seqs;
  return DecodePlan{(int32_t)per_head, (int32_t)(per_head * units)};
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
