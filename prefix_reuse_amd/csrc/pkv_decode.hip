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
//    once - each take a contiguous range of ceil(total / waves) of the chunks
//    in sequence order (the last waves of a head may get fewer, or none). A
//    wave keeps its softmax state across the chunks of a sequence and writes
//    a result only when it leaves the sequence: the final output if it saw the
//    whole sequence, else an unnormalised partial (O, m, l) that a small
//    combine kernel merges in wave order. Lengths that differ by 8x therefore
//    cost nothing in balance.
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
#include "pkv_decode_body.hpp"

#include <stdlib.h>

namespace pkv {
namespace {

// kStep: the decode step's form, which also appends each sequence's newest
// token (DecodeParams::k_new). The partition runs two waves per SIMD, so
// every form may use the registers of two (several need more than the 168
// that three would leave).
// Work-group i is logical wave i: the hardware hands consecutive work-groups
// to the eight XCDs in turn, so XCD k runs waves w = k (mod 8) of every KV
// head. (Remapping so that each XCD took one KV head measured 1.1 % slower on
// the Llama-shaped batch; outputs do not depend on the placement.)
template <typename TQ, typename TC, int D, int BLK, bool kStep>
__global__ __launch_bounds__(64, 2) void decode_kernel(DecodeParams p) {
  decode_wave<TQ, TC, D, BLK, kStep, kStep, true>(p, blockIdx.x, threadIdx.x);
}

// Merge the partials of the sequences that several waves shared, in wave
// order. One work-group per (sequence, group of eight query heads); each
// thread owns 4 consecutive dims of one head, so a long sequence's merge
// still spreads over H_q * d / 4 threads. (Two, four and sixteen heads per
// work-group measured 0.2-0.8 us slower on the Llama-shaped batch, eight
// equal on the shared-prefix one.) Sequences that one wave covered entirely
// already hold their output; empty sequences get zero rows here.
constexpr int kCombineHeads = 8;

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
  // the loads that do not depend on each other go out together: context
  // length, partition info, shared length and the first shared partial (its
  // slot exists for every sequence, so it is read before it is known to count)
  const int ctx = ctx_of(p, seq, cap);
  const int first = p.seq_info[2 * seq];
  int n = p.seq_info[2 * seq + 1];
  constexpr int kMaxSplits = 16;
  // the first shared partial; a shared prefix cut into several key chunks has
  // more, merged further down in batches
  f32x2 sml0 = f32x2{-INFINITY, 0.f};
  f32x4 so0 = f32x4{0.f, 0.f, 0.f, 0.f};
  int lr = 0;
  if (p.shared_lens) {
    lr = p.shared_lens[seq];
    const int64_t srow = (int64_t)seq * p.hq + qh;
    sml0 = *reinterpret_cast<const f32x2*>(p.sh_ml + srow * 2);
    so0 = *reinterpret_cast<const f32x4*>(p.sh_o + srow * D + d0);
  }
  if (ctx == 0) {
    TQx4 z;
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = from_f32<TQ>(0.f);
    *reinterpret_cast<TQx4*>(out) = z;
    return;
  }
  if (!p.shared_lens && n <= 1) return;
  if (own_of<BLK>(p, seq, cap) == 0) n = 0;  // cascade, nothing after the shared prefix
  const int64_t row0 = (int64_t)(first + seq) * p.hq + qh;  // slot of wave `first`
  float M = -INFINITY, L = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  // cascade: the shared prefix's partials (one per key chunk that reaches
  // into this sequence's shared tokens) join the merge first
  int nsh = 0;
  if (p.shared_lens) {
    const int sh = shared_of<BLK>(p, seq, ctx);
    lr = lr < 0 ? 0 : lr;
    lr -= lr % BLK;
    const int chunk = cascade_chunk(lr, p.sh_splits);
    nsh = chunk > 0 ? min((sh + chunk - 1) / chunk, min(p.sh_splits, kMaxSplits)) : 0;
  }
  if (nsh < 1) {
    sml0 = f32x2{-INFINITY, 0.f};
    so0 = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  M = sml0[0];
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
  if (nsh >= 1) {
    const float f = exp2f(sml0[0] - M);
    L += sml0[1] * f;
    O += so0 * f;
  }
#pragma unroll
  for (int i = 0; i < kFew; ++i) {
    const float f = i < nf ? exp2f(ml[i][0] - M) : 0.f;
    L += ml[i][1] * f;
    O += o[i] * f;
  }
  // further partials in batches of kFew, each loaded in one round and merged
  // under a running maximum: the other shared chunks, then the partials of a
  // long context spread over many waves. A batch only moves the maximum up
  // (r = 1 while both are still -inf: nothing has been added yet).
  for (int i0 = 1; i0 < nsh; i0 += kFew) {
#pragma unroll
    for (int i = 0; i < kFew; ++i) {
      const int64_t srow = ((int64_t)(i0 + i) * p.num_seqs + seq) * p.hq + qh;
      const bool ok = i0 + i < nsh;
      ml[i] = ok ? *reinterpret_cast<const f32x2*>(p.sh_ml + srow * 2) : f32x2{-INFINITY, 0.f};
      o[i] = ok ? *reinterpret_cast<const f32x4*>(p.sh_o + srow * D + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < kFew; ++i) Mb = fmaxf(Mb, ml[i][0]);
    const float r = M == Mb ? 1.f : exp2f(M - Mb);
    L *= r;
    O *= r;
    M = Mb;
#pragma unroll
    for (int i = 0; i < kFew; ++i) {
      const float f = i0 + i < nsh ? exp2f(ml[i][0] - M) : 0.f;
      L += ml[i][1] * f;
      O += o[i] * f;
    }
  }
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
    const float r = M == Mb ? 1.f : exp2f(M - Mb);
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

template <typename TQ, int D, int BLK>
hipError_t launch_combine_typed(const DecodeParams& p, hipStream_t stream) {
  const int groups = (p.hq + kCombineHeads - 1) / kCombineHeads;
  hipLaunchKernelGGL((decode_combine_kernel<TQ, D, BLK>), dim3(p.num_seqs * groups), dim3(kCombineHeads * D / 4), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename TQ, typename TC, int D, int BLK>
hipError_t launch_typed(const DecodeParams& p, hipStream_t stream, bool combine_only) {
  if (!combine_only) {
    if (p.k_new)
      hipLaunchKernelGGL((decode_kernel<TQ, TC, D, BLK, true>), dim3(p.total_wgs), dim3(64), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_kernel<TQ, TC, D, BLK, false>), dim3(p.total_wgs), dim3(64), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_combine_typed<TQ, D, BLK>(p, stream);
}

template <typename TQ, typename TC>
hipError_t launch_shape(const DecodeParams& p, int d, int b, hipStream_t s, bool combine_only) {
  if (d == 128 && b == 16) return launch_typed<TQ, TC, 128, 16>(p, s, combine_only);
  if (d == 128 && b == 32) return launch_typed<TQ, TC, 128, 32>(p, s, combine_only);
  if (d == 64 && b == 16) return launch_typed<TQ, TC, 64, 16>(p, s, combine_only);
  if (d == 64 && b == 32) return launch_typed<TQ, TC, 64, 32>(p, s, combine_only);
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

namespace {
hipError_t launch_any(const DecodeParams& p, DT q_dt, DT cache_dt, int d, int b, hipStream_t s, bool combine_only) {
  if (q_dt == DT::F32 && cache_dt == DT::F32) return launch_shape<float, float>(p, d, b, s, combine_only);
  if (q_dt == DT::F16 && cache_dt == DT::F16) return launch_shape<f16_t, f16_t>(p, d, b, s, combine_only);
  if (q_dt == DT::BF16 && cache_dt == DT::BF16) return launch_shape<bf16_t, bf16_t>(p, d, b, s, combine_only);
  if (q_dt == DT::F16 && cache_dt == DT::FP8) return launch_shape<f16_t, uint8_t>(p, d, b, s, combine_only);
  if (q_dt == DT::BF16 && cache_dt == DT::FP8) return launch_shape<bf16_t, uint8_t>(p, d, b, s, combine_only);
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_decode(const DecodeParams& p, DT q_dt, DT cache_dt, int d, int b, hipStream_t s) {
  return launch_any(p, q_dt, cache_dt, d, b, s, false);
}

hipError_t launch_decode_combine(const DecodeParams& p, DT q_dt, DT cache_dt, int d, int b, hipStream_t s) {
  return launch_any(p, q_dt, cache_dt, d, b, s, true);
}

}  // namespace pkv
