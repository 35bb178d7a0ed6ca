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
#include "pkv_prefill_body.hpp"

namespace pkv {
namespace {

template <typename TQ, typename TC, int D, int BLK>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes<D>];
  attend_tile<TQ, TC, D, BLK, false>(p, lds, blockIdx.x);
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
