// Device code of the paged decode (one wave per unit of the balanced
// partition), shared by the decode kernel and the cascade kernel.
#pragma once
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

#include <math.h>
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

// K rows at or past the chunk's `live` tokens are not read (their scores are
// masked): a sequence's last block is read only as far as it holds tokens.
template <typename TC, int D, int BLK>
__device__ __forceinline__ void load_chunk(ChunkRegs<TC, D>& r, const TC* kbase, const TC* vbase,
                                           int blk0, int blk1, int hk, int hkv, int c16, int g, int live) {
  typedef ChunkRegs<TC, D> R;
  const int64_t tile = (int64_t)BLK * D;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int tok = 8 * (c16 / 4) + 4 * a + (c16 % 4);  // chunk-relative token of this A row
    const int blk = (BLK == 32 || tok < 16) ? blk0 : blk1;
    const TC* krow = kbase + ((int64_t)blk * hkv + hk) * tile + (int64_t)(tok % BLK) * D + g * R::E;
    if (tok < live) {
#pragma unroll
      for (int c = 0; c < R::KN; ++c) r.k[a][c] = load_u32x4(krow + c * 4 * R::E);
    } else {
#pragma unroll
      for (int c = 0; c < R::KN; ++c) r.k[a][c] = u32x4{0u, 0u, 0u, 0u};
    }
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

// Decode step: the chunk's token jn (0..31, uniform) is the sequence's newest
// one. Its K and V come from the step's rows instead of the cache, converted
// exactly as pkv_append converts them (bit copy; for fp8, e4m3fn(x / scale)).
// fetch_new_token issues their loads before the chunk's own (both arrive in
// one round trip), place_new_token swaps the values into the chunk registers,
// and store_new_token writes them to the cache slot that the chunk load read
// (once the wave's range is done), so the cache ends as an append would
// leave it.
template <typename TQ, typename TC, int D>
struct NewToken {
  static constexpr bool kFp8 = std::is_same<TC, uint8_t>::value;
  typedef typename std::conditional<kFp8, TQ, TC>::type TR;  // dtype of the step's rows
  static constexpr int KN = ChunkRegs<TC, D>::KN;
  static constexpr int NT = ChunkRegs<TC, D>::NT;
  u32x4 k[KN][kFp8 ? 2 : 1];  // this lane's K pieces as raw row bytes (fp8: 16 row values each)
  TR v[NT];                   // this lane's V values (dims c16 + 16n)
  uint32_t vbits[NT];         // the same as the cache stores them
  int a;                      // which A row of the lane is token jn (-1: none)
  int jv;                     // element of the lane's V pieces that is token jn (-1: none)
};

template <typename TQ, typename TC, int D>
__device__ __forceinline__ void fetch_new_token(NewToken<TQ, TC, D>& nt, const DecodeParams& p, int s, int jn, int hk,
                                                int c16, int g) {
  typedef NewToken<TQ, TC, D> N;
  typedef typename N::TR TR;
  constexpr int E = ChunkRegs<TC, D>::E;
  const TR* knew = reinterpret_cast<const TR*>(p.k_new) + (int64_t)s * p.kn_s0 + (int64_t)hk * p.kn_s1;
  const TR* vnew = reinterpret_cast<const TR*>(p.v_new) + (int64_t)s * p.vn_s0 + (int64_t)hk * p.vn_s1;
  nt.a = -1;
#pragma unroll
  for (int a = 0; a < 2; ++a)
    if (8 * (c16 / 4) + 4 * a + (c16 % 4) == jn) nt.a = a;
  if (nt.a >= 0) {
#pragma unroll
    for (int c = 0; c < N::KN; ++c) {
      const TR* src = knew + g * E + c * 4 * E;
#pragma unroll
      for (int h = 0; h < (N::kFp8 ? 2 : 1); ++h) nt.k[c][h] = load_u32x4(src + h * (16 / sizeof(TR)));
    }
  }
  nt.jv = jn - 8 * g;
  if (nt.jv < 0 || nt.jv >= 8) nt.jv = -1;
  if (nt.jv >= 0) {
#pragma unroll
    for (int n = 0; n < N::NT; ++n) nt.v[n] = vnew[c16 + 16 * n];
  }
}

// Converts the fetched values in place (nt.k to the cache's K bytes, nt.v to
// the cache's V values as raw bits) and swaps them into the chunk registers.
template <typename TQ, typename TC, int D>
__device__ __forceinline__ void place_new_token(ChunkRegs<TC, D>& r, NewToken<TQ, TC, D>& nt,
                                                const DecodeParams& p) {
  typedef ChunkRegs<TC, D> R;
  typedef NewToken<TQ, TC, D> N;
  typedef typename N::TR TR;
  if (nt.a >= 0) {
#pragma unroll
    for (int c = 0; c < R::KN; ++c) {
      u32x4 w;
      if constexpr (N::kFp8) {
        typedef __attribute__((__vector_size__(8 * sizeof(TR)))) TR TR8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const TR8 x = __builtin_bit_cast(TR8, nt.k[c][q / 2]);
          uint32_t word = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) word |= f32_to_e4m3fn(to_f32(x[4 * (q % 2) + j]) / p.k_quant) << (8 * j);
          w[q] = word;
        }
      } else {
        w = nt.k[c][0];
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
        if (a == nt.a) r.k[a][c] = w;
      nt.k[c][0] = w;
    }
  }
  if (nt.jv < 0) return;
  constexpr int kBits = 8 * sizeof(TC);
  constexpr int kPerWord = 32 / kBits;
  constexpr uint32_t kMask = kBits == 32 ? 0xffffffffu : ((1u << kBits) - 1u);
#pragma unroll
  for (int n = 0; n < R::NT; ++n) {
    uint32_t bits;
    if constexpr (N::kFp8) bits = f32_to_e4m3fn(to_f32(nt.v[n]) / p.v_quant);
    else if constexpr (kBits == 16) bits = __builtin_bit_cast(uint16_t, nt.v[n]);
    else bits = __builtin_bit_cast(uint32_t, nt.v[n]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // static register indices; one of them is jv
      if (j != nt.jv) continue;
      const int sh = kBits * (j % kPerWord);
      r.v[n][j / kPerWord] = (r.v[n][j / kPerWord] & ~(kMask << sh)) | (bits << sh);
    }
    nt.vbits[n] = bits;
  }
}

// Writes the placed values to the newest token's cache slot. Issued after the
// wave's range (the chunk's own loads of those lines have long returned).
template <typename TQ, typename TC, int D, int BLK>
__device__ __forceinline__ void store_new_token(const NewToken<TQ, TC, D>& nt, const DecodeParams& p, int jn,
                                                TC* kbase, TC* vbase, int blk0, int blk1, int hk, int c16, int g) {
  typedef ChunkRegs<TC, D> R;
  const int64_t tile = (int64_t)BLK * D;
  if (nt.a >= 0) {
    const int blk = (BLK == 32 || jn < 16) ? blk0 : blk1;
    TC* kdst = kbase + ((int64_t)blk * p.hkv + hk) * tile + (int64_t)(jn % BLK) * D + g * R::E;
#pragma unroll
    for (int c = 0; c < R::KN; ++c) *reinterpret_cast<u32x4*>(kdst + c * 4 * R::E) = nt.k[c][0];
  }
  if (nt.jv < 0) return;
  const int tokv = 8 * g;
  const int blkv = (BLK == 32 || tokv < 16) ? blk0 : blk1;
  TC* vt = vbase + ((int64_t)blkv * p.hkv + hk) * tile + (tokv % BLK) + (int64_t)c16 * BLK;
  constexpr int kBits = 8 * sizeof(TC);
  typedef typename std::conditional<kBits == 8, uint8_t,
                                    typename std::conditional<kBits == 16, uint16_t, uint32_t>::type>::type UT;
#pragma unroll
  for (int n = 0; n < R::NT; ++n) reinterpret_cast<UT*>(vt)[(int64_t)16 * n * BLK + nt.jv] = (UT)nt.vbits[n];
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

// One wave of the decode: logical wave index `logical` of the partition, on
// lane `lane` (0..63) of a wave that runs nothing else.
// kIdsAhead: each chunk's block ids are fetched while the chunk before it in
// the same sequence loads. Measured on the Llama-shaped batch, this makes the
// step form 1.3 us faster and the cascade's decode waves ~2 us faster, but the
// plain decode 2.1-2.7 us slower, so the plain decode keeps fetching them in turn.
// kSeqLanes: lane i keeps what the range walk needs of sequence i < 64 (its own
// tokens, shared prefix, chunks and their running sum) from the first pass, so
// that finding the first sequence and moving to the next read no memory. It
// makes the decode and step forms ~0.6 us faster and the cascade ~0.4 us slower
// (its kernel is already short of registers), so the cascade goes without.
template <typename TQ, typename TC, int D, int BLK, bool kStep = false, bool kIdsAhead = false,
          bool kSeqLanes = false>
__device__ __forceinline__ void decode_wave(const DecodeParams& p, const int logical, const int lane) {
  typedef typename QFrag<TQ, TC, D>::T QT;
  typedef ChunkRegs<TC, D> R;
  constexpr int QS = QFrag<TQ, TC, D>::kSteps;
  constexpr int NT = D / 16;  // output dim tiles
  constexpr bool kSplitP = std::is_same<TQ, bf16_t>::value;  // bf16 P as hi + lo

  const int hkc = logical / p.waves_per_head;  // kv head * head_chunks + chunk
  const int w = logical % p.waves_per_head;
  const int hk = hkc / p.head_chunks;
  const int hchunk = hkc % p.head_chunks;
  const int g = lane / 16, c16 = lane % 16;
  const int cap = p.max_blocks * BLK;
  const int nh = min(16, p.group - hchunk * 16);

  // ---- partition: total chunks, this wave's range, its first sequence ----
  int total = 0, own64 = 0, sh64 = 0, ch64 = 0, incl64 = 0;
  for (int b = 0; b < p.num_seqs; b += 64) {
    const int s = b + lane;
    int own = 0, sh = 0;
    if (s < p.num_seqs) {
      const int cx = ctx_of(p, s, cap);
      sh = shared_of<BLK>(p, s, cx);
      own = cx - sh;
    }
    const int ch = (own + kChunk - 1) / kChunk;
    const int incl = wave_scan(ch, lane);
    if (kSeqLanes && b == 0) {
      own64 = own;
      sh64 = sh;
      ch64 = ch;
      incl64 = incl;
    }
    total += __shfl(incl, 63);
  }
  // own and shared-prefix tokens of sequence s, from the lanes when kept there
  auto own_at = [&](int s) {
    return kSeqLanes && s < 64 ? __builtin_amdgcn_readlane(own64, s) : own_of<BLK>(p, s, cap);
  };
  auto shared_at = [&](int s) {
    return kSeqLanes && s < 64 ? __builtin_amdgcn_readlane(sh64, s) : shared_of<BLK>(p, s, ctx_of(p, s, cap));
  };
  total = __builtin_amdgcn_readfirstlane(total);
  if (total == 0) return;
  const int per_wave = (total + p.waves_per_head - 1) / p.waves_per_head;
  const int c0 = w * per_wave;
  const int c1 = min(c0 + per_wave, total);
  // per-sequence partition info, written once for the combine kernel, by wave 0
  // after its own range (its stores would otherwise hold up its first loads)
  auto write_partition_info = [&]() {
    if (logical != 0) return;
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
  };
  if (c0 >= c1) {
    write_partition_info();
    return;
  }
  // first sequence of the range: the one whose chunks contain c0
  int s_cur = 0, s_first_chunk = 0;
  if (kSeqLanes && p.num_seqs <= 64) {
    // c0 < total, so some lane's running sum passes c0
    const int l0 = __builtin_ctzll(__ballot(lane < p.num_seqs && incl64 > c0));
    s_cur = l0;
    s_first_chunk = __shfl(incl64 - ch64, l0);
  } else {
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
  auto table_of = [&](int s) { return p.block_tables + (int64_t)s * p.bt_s0 + shared_at(s) / BLK; };
  int ctx = own_at(s_cur);
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
  // A result of a sequence the range leaves before its end is kept in
  // registers and written once the next one is complete (or the range is
  // done): a store counts in the vector-memory counter with the loads, so one
  // issued before the next sequence's loads would make their wait cover it.
  f32x4 pend_acc[NT];
  float pend_m = 0.f, pend_l = 0.f;
  int pend_s = -1;
  bool pend_whole = false;
  auto write_result = [&](const f32x4* a, float m, float l, int s, bool whole) {
    if (!hvalid) return;
    const int qh = hk * p.group + hchunk * 16 + c16;
    if (whole) {
      const float inv = p.v_scale / l;
      TQ* o = reinterpret_cast<TQ*>(p.out) + s * p.o_s0 + qh * p.o_s1;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        typedef __attribute__((__vector_size__(4 * sizeof(TQ)))) TQ TQx4;
        TQx4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = from_f32<TQ>(a[n][i] * inv);
        *reinterpret_cast<TQx4*>(o + 16 * n + 4 * g) = v;
      }
    } else {
      const int64_t row = (int64_t)(w + s) * p.hq + qh;
#pragma unroll
      for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4*>(p.ws_o + row * D + 16 * n + 4 * g) = a[n];
      if (g == 0) { p.ws_ml[row * 2] = m; p.ws_ml[row * 2 + 1] = l; }
    }
  };
  auto finish_seq = [&](bool whole, bool last) {
    float l = l_run + __shfl_xor(l_run, 16);
    l += __shfl_xor(l, 32);
    if (pend_s >= 0) {
      write_result(pend_acc, pend_m, pend_l, pend_s, pend_whole);
      pend_s = -1;
    }
    if (last) {
      write_result(acc, m_run, l, s_cur, whole);
      return;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) pend_acc[n] = acc[n];
    pend_m = m_run;
    pend_l = l;
    pend_s = s_cur;
    pend_whole = whole;
  };

  start_seq();
  int seq_start = s_first_chunk;  // global index of s_cur's first chunk
  // Decode step: the stores of the newest token's K and V wait until the
  // wave's range is done (or until the next sequence's newest token comes).
  // Stores count in the same vector-memory counter as loads, so a store
  // issued mid-range would make the wait for the next chunk's loads wait for
  // it too.
  NewToken<TQ, TC, D> pend;
  int pend_jn = -1, pend_b0 = 0, pend_b1 = 0;
  int nb0 = 0, nb1 = 0;   // block ids of the next chunk, fetched during this one
  bool have_next = false;  // (when it lies in the same sequence)
  for (int c = c0; c < c1; ++c) {
    // ---- load the chunk ----
    const int jb = tb / BLK;
    int b0, b1;
    if (kIdsAhead && have_next) {
      b0 = nb0;
      b1 = nb1;
    } else {
      b0 = bt[jb];
      b1 = b0;
      if constexpr (BLK == 16) {
        if ((jb + 1) * BLK < ctx) b1 = bt[jb + 1];  // only entries that hold live tokens
      }
    }
    b0 = min(max(b0, 0), p.num_blocks - 1);
    b1 = min(max(b1, 0), p.num_blocks - 1);
    R r;
    const int jn = ctx - 1 - tb;  // decode step: the newest token, if this chunk holds it
    NewToken<TQ, TC, D> nt;
    if constexpr (kStep) {
      if (jn < kChunk) fetch_new_token<TQ, TC, D>(nt, p, s_cur, jn, hk, c16, g);
    }
    load_chunk<TC, D, BLK>(r, kbase, vbase, b0, b1, hk, p.hkv, c16, g, ctx - tb);
    // the next chunk's block ids, if it is in this sequence: fetched now, so
    // that its loads need not wait for them
    have_next = kIdsAhead && tb + kChunk < ctx && c + 1 < c1;
    if (have_next) {
      const int jn2 = (tb + kChunk) / BLK;
      nb0 = bt[jn2];
      nb1 = nb0;
      if constexpr (BLK == 16) {
        if ((jn2 + 1) * BLK < ctx) nb1 = bt[jn2 + 1];
      }
    }
    if constexpr (kStep) {
      if (jn < kChunk) place_new_token<TQ, TC, D>(r, nt, p);
    }

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

    if constexpr (kStep) {
      if (jn < kChunk && hchunk == 0) {
        if (pend_jn >= 0)
          store_new_token<TQ, TC, D, BLK>(pend, p, pend_jn, const_cast<TC*>(kbase), const_cast<TC*>(vbase), pend_b0,
                                          pend_b1, hk, c16, g);
        pend = nt;
        pend_jn = jn;
        pend_b0 = b0;
        pend_b1 = b1;
      }
    }

    // ---- advance ----
    tb += kChunk;
    if (tb >= ctx || c + 1 == c1) {
      const int nch = (ctx + kChunk - 1) / kChunk;
      finish_seq(!p.shared_lens && seq_start >= c0 && seq_start + nch <= c1, c + 1 == c1);  // cascade: always a partial
      if (c + 1 == c1) break;
      seq_start += nch;
      do {  // next non-empty sequence
        ++s_cur;
        ctx = own_at(s_cur);
      } while (ctx == 0);
      tb = 0;
      bt = table_of(s_cur);
      start_seq();
    }
  }
  if constexpr (kStep) {
    if (pend_jn >= 0)
      store_new_token<TQ, TC, D, BLK>(pend, p, pend_jn, const_cast<TC*>(kbase), const_cast<TC*>(vbase), pend_b0,
                                      pend_b1, hk, c16, g);
  }
  write_partition_info();
}

}  // namespace
}  // namespace pkv
