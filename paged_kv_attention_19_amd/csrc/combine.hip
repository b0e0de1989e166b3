// Second pass of split-K decode: merge each (sequence, query head)'s split
// partials by log-sum-exp (course README "Build an LLM Inference Engine From
// Scratch", curriculum S12 and claim s12: the split variants agree with the
// plain softmax). M = max_s lse_s, w_s = exp(lse_s - M),
// out = sum_s w_s o_s / sum_s w_s, lse = M + log sum_s w_s.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

// NW = 4: one workgroup of 4 wavefronts per (sequence, query head).
// Wavefront w merges splits w, w + 4, w + 8, ... against its own reference
// max; the four states (M_w, L_w, acc_w) then merge through LDS, each
// rescaled by exp(M_w - M). So the partials of a pair are read by four chains
// of loads in parallel, not one. NW = 1: one wavefront per pair, four pairs
// per workgroup, for pairs of a few splits, where the other three wavefronts
// would have nothing to read.
//
// With NW = 4 a wavefront takes its splits kChunk at a time. Every row of the
// partials below max_ns lies inside the caller's arrays, so the loads of a
// chunk (the lse values, one per lane, and the kChunk rows of o; a split past
// max_ns reads the last row instead) go out together, before the split count
// and the maxima they are weighed with arrive; splits at or past the
// sequence's own count are masked afterwards. Lane k holds the lse of the
// chunk's split k, and its weight reaches the other lanes by readlane. With
// NW = 1 (fewer than 8 splits) a first pass takes the max over the lse values
// (a lane per split), then a second the weighted rows. Measured on MI355X
// (head_dim 128, 16 query heads): 8 x 32k tokens in 64 splits 2.98 us against
// 3.46 us with the two passes; the mixed step's decode rows (at most 4
// splits) 2.64 us with the two passes against 3.0 us in one chunk.
constexpr int kChunk = 16;
// Workgroup i runs on XCD i % 8. The workgroups are renumbered so that each
// XCD merges one contiguous range of (sequence, query head) pairs: the same
// sequences whose partials the decode launch just wrote from that XCD (its
// work items are renumbered the same way), so the rows are read from that
// XCD's L2. Measured on MI355X (whole steps): 8 x 32k tokens in 64 splits,
// 165.6-165.7 against 167.0-167.1 us; the mixed step's int8 decode rows,
// 106.0-106.4 against 106.5-106.6 us.
constexpr int kXcdsM = 8;

template <int D, int NW>
__global__ __launch_bounds__(256) void lse_combine_kernel(CombineParams p) {
  constexpr int DPL = D / kWave;  // dims per lane
  __shared__ float s_acc[NW][D];
  __shared__ float s_m[NW], s_l[NW];
  __shared__ int s_nan[NW];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = NW == 1 ? 0 : wid;   // this wavefront's first split
  const int nwg = gridDim.x;   // a multiple of kXcdsM
  const int wg = (blockIdx.x % kXcdsM) * (nwg / kXcdsM) + blockIdx.x / kXcdsM;
  const int pair = NW == 1 ? wg * 4 + wid : wg;
  if (pair >= p.batch * p.num_q_heads) return;
  const int b = pair / p.num_q_heads;
  const int h = pair % p.num_q_heads;
  const size_t row0 = static_cast<size_t>(b) * p.max_ns * p.num_q_heads + h;
  // a scalar load: the vector loads below do not wait for it
  const int ns = p.nsplits[b];
  const bool bad = ns < 1 || ns > p.max_ns;

  float Mw = neg_inf(), Lw = 0.f;
  bool nan = false;
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  if constexpr (NW == 1) {
    // this wavefront's splits: their max lse (and whether any is NaN)
    if (!bad) {
      for (int s = lane; s < ns; s += kWave) {
        const float x = p.lse_part[row0 + static_cast<size_t>(s) * p.num_q_heads];
        nan = nan || (x != x);
        Mw = fmaxf(Mw, x);
      }
    }
    Mw = wave_max(Mw);
    nan = wave_any(nan);
    if (!bad && !nan && Mw != neg_inf()) {
#pragma unroll 4
      for (int s = 0; s < ns; ++s) {
        const size_t row = row0 + static_cast<size_t>(s) * p.num_q_heads;
        const float x = p.lse_part[row];
        const float wt = __builtin_amdgcn_exp2f((x - Mw) * kLog2e);  // -inf -> 0
        Lw += wt;
        const float* o = p.o_part + row * D + lane * DPL;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = fmaf(wt, o[e], acc[e]);
      }
    }
  } else {
    for (int c0 = 0; NW * c0 < p.max_ns; c0 += kChunk) {
      // the chunk's loads, all issued before any is used
      const int sl = w + NW * (c0 + lane);   // lane's split
      float x = neg_inf();
      if (lane < kChunk) x = p.lse_part[row0 + static_cast<size_t>(min(sl, p.max_ns - 1)) * p.num_q_heads];
      float o[kChunk][DPL];
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        const int s = min(w + NW * (c0 + k), p.max_ns - 1);
        const float* src = p.o_part + (row0 + static_cast<size_t>(s) * p.num_q_heads) * D + lane * DPL;
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[k][e] = src[e];
      }
      if (bad) break;
      if (NW * c0 + w >= ns) break;   // none of this chunk's splits is the sequence's
      const bool valid = lane < kChunk && sl < ns;
      if (!valid) x = neg_inf();
      nan = nan || wave_any(valid && x != x);
      const float Mn = fmaxf(Mw, wave_max(x));
      if (Mn == neg_inf()) continue;   // no finite lse yet
      const float corr = (Mw == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f((Mw - Mn) * kLog2e);
      Mw = Mn;
      Lw *= corr;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] *= corr;
      const float wl = (x == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f((x - Mw) * kLog2e);
      Lw += group_sum<kWave>(wl);
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        if (NW * (c0 + k) + w < ns) {   // uniform: split k of the chunk is the sequence's
          const float wt = __int_as_float(readlane(__float_as_int(wl), k));
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[e] = fmaf(wt, o[k][e], acc[e]);
        }
      }
    }
  }
  float M, L;
  bool any_nan;
  float f[NW];
  if constexpr (NW == 1) {
    M = Mw;
    L = Lw;
    any_nan = nan;
    f[0] = 1.f;
  } else {
#pragma unroll
    for (int e = 0; e < DPL; ++e) s_acc[w][lane * DPL + e] = acc[e];
    if (lane == 0) {
      s_m[w] = Mw;
      s_l[w] = Lw;
      s_nan[w] = nan;
    }
    __syncthreads();
    if (w != 0) return;
    M = s_m[0];
    any_nan = s_nan[0] != 0;
#pragma unroll
    for (int i = 1; i < NW; ++i) {
      M = fmaxf(M, s_m[i]);
      any_nan = any_nan || (s_nan[i] != 0);
    }
    L = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      f[i] = (s_m[i] == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f((s_m[i] - M) * kLog2e);
      L += s_l[i] * f[i];
    }
  }
  float* out = p.out + static_cast<size_t>(pair) * D + lane * DPL;
  float lse;
  if (bad || any_nan) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) out[e] = qnan();
    lse = qnan();
  } else if (L > 0.f) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      float y;
      if constexpr (NW == 1) {
        y = acc[e];
      } else {
        y = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) y = fmaf(s_acc[i][lane * DPL + e], f[i], y);
      }
      out[e] = y / L;
    }
    lse = M + logf(L);
  } else {
#pragma unroll
    for (int e = 0; e < DPL; ++e) out[e] = 0.f;
    lse = neg_inf();
  }
  if (lane == 0 && p.out_lse != nullptr) p.out_lse[pair] = lse;
}

}  // namespace

// Four wavefronts per pair from this many splits on (p.max_ns: the host's
// bound on every sequence's split count). Measured on MI355X (traced, head_dim
// 128, 16 query heads): 8 x 32k tokens in 64 splits, 6.7 us with one
// wavefront per pair against 3.9 us with four (eight, or a deeper unroll, were
// within noise of four); the mixed step's decode rows (at most 4 splits), 3.4
// us either way.
constexpr int kCombineWideSplits = 8;

template <int D>
hipError_t launch_combine_d(const CombineParams& p, hipStream_t st) {
  const int pairs = p.batch * p.num_q_heads;
  if (p.max_ns >= kCombineWideSplits) {
    hipLaunchKernelGGL((lse_combine_kernel<D, 4>), dim3((pairs + kXcdsM - 1) / kXcdsM * kXcdsM), dim3(256), 0, st, p);
  } else {
    hipLaunchKernelGGL((lse_combine_kernel<D, 1>), dim3(((pairs + 3) / 4 + kXcdsM - 1) / kXcdsM * kXcdsM), dim3(256),
                       0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t st) {
  switch (head_dim) {
    case 64: return launch_combine_d<64>(p, st);
    case 128: return launch_combine_d<128>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
