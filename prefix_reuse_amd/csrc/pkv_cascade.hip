// Cascade decode for groups of sequences that share a prompt prefix, for
// gfx950 (page "PagedAttention과 RadixAttention으로 LLM KV 캐시 최적화"
// §03-§04: the shared prefix is cached once and reused by every request that
// starts with it). Attention over a whole context equals the log-sum-exp
// merge of the attention over the shared keys and over the remaining ones.
//
// One launch of cascade_kernel does both parts of the attention:
//  * Work-groups [0, shared_wgs): the shared part. Each takes one row tile of
//    a group's (sequence, head) query rows and a chunk of the group's shared
//    keys, runs the suffix-prefill work-group on the matrix cores (non-causal,
//    each row limited to its own context) and writes unnormalised partials.
//    The shared keys are read once per row tile instead of once per sequence.
//  * The remaining work-groups: eight decode waves each, over every
//    sequence's own tokens after its shared prefix (the balanced partition of
//    the decode kernel, sized to the compute units the shared part leaves).
// The shared work-groups come first in the grid, so the hardware places them
// first; each holds a whole CU (128 KiB of LDS), and the decode waves fill the
// other CUs and stream their tokens beside them. One launch avoids the
// cross-queue waits two streams would need. The decode's combine kernel then
// merges every sequence's partials.
#include "pkv_decode_body.hpp"
#include "pkv_prefill_body.hpp"

namespace pkv {
namespace {

template <typename TQ, typename TC, int D, int BLK>
__global__ __launch_bounds__(kThreads, 1) void cascade_kernel(PrefillParams sp, DecodeParams dp, int shared_wgs) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes<D>];
  const int wg = blockIdx.x;
  if (wg < shared_wgs) {  // shared_wgs is a multiple of 8: the decode part starts on XCD 0
    if (wg < sp.hkv * sp.tiles_per_head) attend_tile<TQ, TC, D, BLK, true>(sp, lds, wg);
    return;
  }
  const int dwg = xcd_remap(wg - shared_wgs, (int)gridDim.x - shared_wgs);
  const int v = dwg * kWaves + __builtin_amdgcn_readfirstlane((int)threadIdx.x / 64);
  if (v < dp.total_wgs) decode_wave<TQ, TC, D, BLK, false, true>(dp, v, (int)threadIdx.x % 64);
}

template <typename TQ, typename TC, int D, int BLK>
hipError_t launch_typed(const PrefillParams& sp, const DecodeParams& dp, int shared_wgs, hipStream_t stream) {
  const int64_t grid = (int64_t)shared_wgs + (dp.total_wgs + kWaves - 1) / kWaves;
  hipLaunchKernelGGL((cascade_kernel<TQ, TC, D, BLK>), dim3((unsigned)grid), dim3(kThreads), 0, stream, sp, dp,
                     shared_wgs);
  return hipGetLastError();
}

template <typename TQ, typename TC>
hipError_t launch_shape(const PrefillParams& sp, const DecodeParams& dp, int shared_wgs, int d, int b,
                        hipStream_t s) {
  if (d == 128 && b == 16) return launch_typed<TQ, TC, 128, 16>(sp, dp, shared_wgs, s);
  if (d == 128 && b == 32) return launch_typed<TQ, TC, 128, 32>(sp, dp, shared_wgs, s);
  if (d == 64 && b == 16) return launch_typed<TQ, TC, 64, 16>(sp, dp, shared_wgs, s);
  if (d == 64 && b == 32) return launch_typed<TQ, TC, 64, 32>(sp, dp, shared_wgs, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_cascade(const PrefillParams& sp, const DecodeParams& dp, int shared_wgs, DT q_dt, DT cache_dt,
                          int d, int b, hipStream_t s) {
  if (shared_wgs % 8 != 0 || (int64_t)sp.hkv * sp.tiles_per_head > shared_wgs) return hipErrorInvalidValue;
  hipError_t e = hipErrorInvalidValue;
  if (q_dt == DT::F16 && cache_dt == DT::F16) e = launch_shape<f16_t, f16_t>(sp, dp, shared_wgs, d, b, s);
  else if (q_dt == DT::BF16 && cache_dt == DT::BF16) e = launch_shape<bf16_t, bf16_t>(sp, dp, shared_wgs, d, b, s);
  else if (q_dt == DT::F16 && cache_dt == DT::FP8) e = launch_shape<f16_t, uint8_t>(sp, dp, shared_wgs, d, b, s);
  else if (q_dt == DT::BF16 && cache_dt == DT::FP8) e = launch_shape<bf16_t, uint8_t>(sp, dp, shared_wgs, d, b, s);
  if (e != hipSuccess) return e;
  return launch_decode_combine(dp, q_dt, cache_dt, d, b, s);
}

}  // namespace pkv
