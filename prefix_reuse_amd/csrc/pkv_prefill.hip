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
//    tile's causal diagonal spans few tokens. A work-group of 8 waves (one
//    per CU, two per SIMD) owns 256 rows of one (request, KV head); each wave
//    owns 32 rows, whose Q^T stays in registers.
//  * Keys are consumed 64 per stage through a ring of four LDS buffers per
//    operand. 16-bit K and V tiles go from global memory straight to LDS
//    (global_load_lds, one 1 KB load per wave lying inside a single cache
//    block, addressed by a scalar block base plus a fixed lane offset), three
//    stages ahead of use; fp8 tiles are staged through registers and
//    converted exactly. V^T tiles keep the cache's own [d][B] block layout in
//    LDS. Both LDS layouts are XOR-swizzled so that the matrix-core operand
//    reads are free of bank conflicts. Block ids come from scalar loads.
//  * Per wave and 32-key sub-tile, on v_mfma_f32_32x32x16:
//      S^T[key][row] = K[key][:] . Q[row][:]
//      O^T[dim][row] += V^T[dim][keys] . P^T[keys][row]
//    K rows are read in a permuted order so that each lane ends up holding 16
//    consecutive keys of one row: the B operand of the PV product. The score
//    product runs two sub-tiles ahead of the value product; each step reads
//    its operands from LDS first, computes a softmax while they arrive, then
//    issues its 24 (16) products back to back.
//  * Precision of P in the PV product: with f16 operands P is rounded to f16
//    (11 bits; P stays in [0, 2^10] thanks to the lazy rescale below). With bf16
//    operands P would carry only 8 bits - too few for 2e-3 on short contexts -
//    so P goes in as bf16(P) + bf16(P - bf16(P)): two products on the matrix
//    cores. fp8 V is converted exactly to f16 while staging.
//  * Online softmax in base 2 with the scale folded into one FMA per score and
//    the raw v_exp_f32 (results below 2^-126 flush to 0); the running max moves
//    only when a row's max grows by more than 2^8 (lazy rescale), so the
//    output accumulators are rarely rescaled. The bf16 cache's fast pass takes
//    no row max in its full steps at all: it checks P's row sums after the
//    exponentials and moves a row's max only once one of its P values passes
//    2^6 (an infinite P sends the work-group to the exact pass). The causal mask is applied only
//    on key tiles that reach past the wave's first token.
//  * Key-split form (prefill_split_kernel + prefill_merge_kernel), for
//    batches whose row tiles would leave most CUs idle (one conversation's
//    next turn): each row tile's keys are spread over several work-groups,
//    the parts' partials merged by log-sum-exp in a second launch.
#include "pkv_prefill_body.hpp"

namespace pkv {
namespace {

template <typename TQ, typename TC, int D, int BLK>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes<D>];
  attend_tile<TQ, TC, D, BLK, false>(p, lds, blockIdx.x);
}

// Key-split form (few rows, long prefixes: a plain launch would leave most
// CUs idle). Parts 0 .. key_splits-2 of a row tile take chunks of the
// prefix's whole stages, the last part the keys after them; each writes an
// unnormalised partial, and prefill_merge_kernel merges them.
template <typename TQ, typename TC, int D, int BLK>
__global__ __launch_bounds__(kThreads, 1) void prefill_split_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes<D>];
  attend_tile<TQ, TC, D, BLK, false, true>(p, lds, blockIdx.x);
}

// Merge of the key-split parts: one work-group per (suffix token, group of
// eight query heads), each thread owning 4 consecutive dims of one head. The
// token's request is found as the prefill finds it (64 requests per round,
// lengths clamped the same way); the parts that hold keys are the last one
// and the prefix chunks that reach into the request's prefix, merged by
// log-sum-exp under a running maximum, eight at a time.
constexpr int kMergeHeads = 8;

template <typename TQ, int D, int BLK>
__global__ __launch_bounds__(kMergeHeads * D / 4) void prefill_merge_kernel(PrefillParams p) {
  const int groups = (p.hq + kMergeHeads - 1) / kMergeHeads;
  const int64_t t = blockIdx.x / groups;  // packed suffix token
  const int qh = (blockIdx.x % groups) * kMergeHeads + (int)threadIdx.x / (D / 4);
  const int d0 = ((int)threadIdx.x % (D / 4)) * 4;
  const int ln = (int)threadIdx.x % 64;
  int r = -1;
  int64_t rows_before = 0;
  for (int r0 = 0; r0 < p.num_reqs; r0 += 64) {  // uniform over the work-group
    const int rr = r0 + ln;
    int64_t s = 0;
    if (rr < p.num_reqs) s = p.suffix_lens[rr];
    s = s < 0 ? 0 : (s > p.total_rows ? p.total_rows : s);
    int64_t incl = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t u = __shfl_up(incl, off);
      if (ln >= off) incl += u;
    }
    const int64_t rb = min(rows_before + (incl - s), p.total_rows);
    const int64_t re = min(rows_before + incl, p.total_rows);
    const uint64_t hit = __ballot(rr < p.num_reqs && t >= rb && t < re);
    if (hit) {
      r = r0 + __builtin_ctzll(hit);
      break;
    }
    rows_before = min(rows_before + __shfl(incl, 63), p.total_rows);
  }
  if (r < 0 || qh >= p.hq) return;  // a row no request covers is left as the plain kernel leaves it
  const int cap = p.max_blocks * BLK;
  int P = p.prefix_lens[r];
  P = P < 0 ? 0 : (P > cap ? cap : P);
  const int nsplit = p.key_splits - 1;
  const int Ps = split_prefix_keys(P);
  const int chunk = cascade_chunk(Ps, nsplit);
  const int nk = chunk > 0 ? min((Ps + chunk - 1) / chunk, nsplit) : 0;
  // The last part holds keys (at least the first one after the chunks) unless
  // the prefix filled the table's capacity and that capacity is a whole
  // number of stages: then every key is in the chunks, the last part's
  // work-group found nothing to do and its slot was never written.
  const int skip = (P == cap && Ps == P) ? 1 : 0;
  const int np = nk + 1 - skip;
  // part list: the last part (when it holds keys), then the prefix chunks
  // 0 .. nk-1
  constexpr int kFew = 8;
  float M = -INFINITY, L = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < np; j0 += kFew) {
    f32x2 ml[kFew];
    f32x4 o[kFew];
#pragma unroll
    for (int j = 0; j < kFew; ++j) {
      const int q = j0 + j + skip;
      const int part = q == 0 ? nsplit : q - 1;
      const int64_t srow = ((int64_t)part * p.total_rows + t) * p.hq + qh;
      const bool ok = j0 + j < np;
      ml[j] = ok ? *reinterpret_cast<const f32x2*>(p.ws_ml + srow * 2) : f32x2{-INFINITY, 0.f};
      o[j] = ok ? *reinterpret_cast<const f32x4*>(p.ws_o + srow * D + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float Mb = M;
#pragma unroll
    for (int j = 0; j < kFew; ++j) Mb = fmaxf(Mb, ml[j][0]);
    const float rs = M == Mb ? 1.f : exp2f(M - Mb);
    L *= rs;
    O *= rs;
    M = Mb;
#pragma unroll
    for (int j = 0; j < kFew; ++j) {
      const float f = j0 + j < np ? exp2f(ml[j][0] - M) : 0.f;
      L += ml[j][1] * f;
      O += o[j] * f;
    }
  }
  const float inv = p.v_scale / L;
  typedef __attribute__((__vector_size__(4 * sizeof(TQ)))) TQ TQx4;
  TQx4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = from_f32<TQ>(O[i] * inv);
  *reinterpret_cast<TQx4*>(reinterpret_cast<TQ*>(p.out) + t * p.o_s0 + (int64_t)qh * p.o_s1 + d0) = v;
}

template <typename TQ, typename TC, int D, int BLK>
hipError_t launch_typed(const PrefillParams& p, hipStream_t stream, bool split) {
  const int64_t wgs = (int64_t)p.hkv * p.tiles_per_head;
  if (wgs == 0) return hipSuccess;
  if (!split) {
    hipLaunchKernelGGL((prefill_kernel<TQ, TC, D, BLK>), dim3((unsigned)wgs), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((prefill_split_kernel<TQ, TC, D, BLK>), dim3((unsigned)wgs), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t mwgs = p.total_rows * ((p.hq + kMergeHeads - 1) / kMergeHeads);
  hipLaunchKernelGGL((prefill_merge_kernel<TQ, D, BLK>), dim3((unsigned)mwgs), dim3(kMergeHeads * D / 4), 0, stream,
                     p);
  return hipGetLastError();
}

template <typename TQ, typename TC>
hipError_t launch_shape(const PrefillParams& p, int d, int b, hipStream_t s, bool split) {
  if (d == 128 && b == 16) return launch_typed<TQ, TC, 128, 16>(p, s, split);
  if (d == 128 && b == 32) return launch_typed<TQ, TC, 128, 32>(p, s, split);
  if (d == 64 && b == 16) return launch_typed<TQ, TC, 64, 16>(p, s, split);
  if (d == 64 && b == 32) return launch_typed<TQ, TC, 64, 32>(p, s, split);
  return hipErrorInvalidValue;
}

hipError_t launch_any(const PrefillParams& p, DT q_dt, DT cache_dt, int d, int b, hipStream_t s, bool split) {
  if (q_dt == DT::F16 && cache_dt == DT::F16) return launch_shape<f16_t, f16_t>(p, d, b, s, split);
  if (q_dt == DT::BF16 && cache_dt == DT::BF16) return launch_shape<bf16_t, bf16_t>(p, d, b, s, split);
  if (q_dt == DT::F16 && cache_dt == DT::FP8) return launch_shape<f16_t, uint8_t>(p, d, b, s, split);
  if (q_dt == DT::BF16 && cache_dt == DT::FP8) return launch_shape<bf16_t, uint8_t>(p, d, b, s, split);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, DT q_dt, DT cache_dt, int d, int b, hipStream_t s) {
  return launch_any(p, q_dt, cache_dt, d, b, s, false);
}

hipError_t launch_prefill_split(const PrefillParams& p, DT q_dt, DT cache_dt, int d, int b, hipStream_t s) {
  if (p.key_splits < 2 || p.ws_o == nullptr || p.ws_ml == nullptr) return hipErrorInvalidValue;
  return launch_any(p, q_dt, cache_dt, d, b, s, true);
}

}  // namespace pkv
