// Second pass of split-K decode: merge each (sequence, query head)'s split
// partials by log-sum-exp (course README "Build an LLM Inference Engine From
// Scratch", curriculum S12 and claim s12: the split variants agree with the
// plain softmax). M = max_s lse_s, w_s = exp(lse_s - M),
// out = sum_s w_s o_s / sum_s w_s, lse = M + log sum_s w_s.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

// One wavefront per (sequence, query head): merge that pair's split partials.
template <int D>
__global__ __launch_bounds__(256) void lse_combine_kernel(CombineParams p) {
  constexpr int DPL = D / kWave;  // dims per lane
  const int lane = threadIdx.x & 63;
  const int pair = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (pair >= p.batch * p.num_q_heads) return;
  const int b = pair / p.num_q_heads;
  const int h = pair % p.num_q_heads;
  const int ns = p.nsplits[b];
  float* out = p.out + static_cast<size_t>(pair) * D + lane * DPL;
  const bool bad = ns < 1 || ns > p.max_ns;
  const size_t row0 = static_cast<size_t>(b) * p.max_ns * p.num_q_heads + h;

  float M = neg_inf();
  bool nan = false;
  if (!bad) {
    for (int s = lane; s < ns; s += kWave) {
      const float x = p.lse_part[row0 + static_cast<size_t>(s) * p.num_q_heads];
      nan = nan || (x != x);
      M = fmaxf(M, x);
    }
  }
  M = wave_max(M);
  nan = wave_any(nan);
  float L = 0.f;
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  if (!bad && !nan && M != neg_inf()) {
#pragma unroll 4
    for (int s = 0; s < ns; ++s) {
      const size_t row = row0 + static_cast<size_t>(s) * p.num_q_heads;
      const float x = p.lse_part[row];
      const float wt = __builtin_amdgcn_exp2f((x - M) * kLog2e);  // -inf -> 0
      L += wt;
      const float* o = p.o_part + row * D + lane * DPL;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = fmaf(wt, o[e], acc[e]);
    }
  }
  float lse;
  if (bad || nan) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) out[e] = qnan();
    lse = qnan();
  } else if (L > 0.f) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) out[e] = acc[e] / L;
    lse = M + logf(L);
  } else {
#pragma unroll
    for (int e = 0; e < DPL; ++e) out[e] = 0.f;
    lse = neg_inf();
  }
  if (lane == 0 && p.out_lse != nullptr) p.out_lse[pair] = lse;
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t st) {
  const int pairs = p.batch * p.num_q_heads;
  const dim3 grid((pairs + 3) / 4);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(lse_combine_kernel<64>, grid, dim3(256), 0, st, p); break;
    case 128: hipLaunchKernelGGL(lse_combine_kernel<128>, grid, dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
