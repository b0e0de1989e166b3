// Split-K paged decode for gfx950: the partial pass and the log-sum-exp merge.
//
// What is computed (course README "Build an LLM Inference Engine From
// Scratch", curriculum S06 PagedAttention and S12 FlashAttention; claims s06
// and s12 in section "The code asserts its own claims"): for every sequence b
// and query head h, softmax(scale * q_h . k_t) weighted values over the
// sequence's tokens t < n_b, the K/V rows read through the block table. The
// tokens are cut into num_splits[b] block-aligned ranges; each range is
// reduced with an online softmax to (o_s, lse_s), and the ranges are merged by
// log-sum-exp.
//
// Work mapping. One workgroup of NW wavefronts per (split, kv head, sequence).
// The split's 16-token blocks are dealt to the wavefronts round-robin. A
// wavefront reads one (block, kv head) K tile -- 16 rows of head_dim elements,
// contiguous in HBM -- with 16-byte loads, 1 KiB per load instruction, and
// the V tile the same way. Lane l holds the 16 bytes at offset 16 l of each
// KiB: LPT consecutive lanes cover one token row, so one load instruction
// covers TPI = 64 / LPT tokens. The K/V tile stays in registers and serves
// all G query heads of the GQA group, so every KV byte is read from HBM once.
// QK dot products are lane-partial sums reduced across the LPT lanes with DPP
// moves; each of the TPI token slots keeps its own running max / sum /
// accumulator (base-2 exponentials), merged across slots with lane shuffles
// and across wavefronts through LDS at the end.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

template <int KV, int QT, int D, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_partial_kernel(DecodeParams p) {
  using Geo = KvGeom<KV>;
  constexpr int EPL = Geo::kEpl;
  constexpr int LPT = D / EPL;          // lanes per token row
  constexpr int TPI = kWave / LPT;      // tokens per load instruction
  constexpr int IPB = kBlock / TPI;     // load instructions per block tile
  constexpr bool kDot2 = (KV == PKV_BF16 && QT == PKV_BF16);
  constexpr int kTileBytes = kBlock * D * Geo::kEsize;
  constexpr bool kI8 = (KV == PKV_I8);
  static_assert(TPI * LPT == kWave && IPB * TPI == kBlock, "geometry");

  __shared__ float s_acc[NW][G][D];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];
  __shared__ int s_bad[NW];

  const int s = blockIdx.x;
  const int kh = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tslot = lane / LPT;
  const int c = lane % LPT;

  const int n = p.ctx[b];
  const int ns = p.direct ? 1 : p.nsplits[b];
  if (ns < 1 || s >= ns) return;  // not a split of this sequence (the merge checks ns)

  const bool bad_n = (n < 0) || (static_cast<int64_t>(n) > static_cast<int64_t>(p.max_blocks) * kBlock);
  int t0 = 0, t1 = 0;
  if (!bad_n && n > 0) {
    const int per = (n + ns - 1) / ns;
    const int tps = ((per + kBlock - 1) / kBlock) * kBlock;
    const int64_t a = static_cast<int64_t>(s) * tps;
    t0 = a < n ? static_cast<int>(a) : n;
    t1 = (static_cast<int64_t>(t0) + tps) < n ? t0 + tps : n;
  }
  const int blk_lo = t0 / kBlock;
  const int nblk = (t1 - t0 + kBlock - 1) / kBlock;
  const int nb_w = nblk > w ? (nblk - w + NW - 1) / NW : 0;

  // ---- the G query rows of this group, in the lane's EPL dims ----
  const int h0 = kh * G;
  float qf[G][EPL];
  uint32_t q2[G][EPL / 2];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const size_t base = (static_cast<size_t>(b) * p.num_q_heads + h0 + g) * D + c * EPL;
    if constexpr (kDot2) {
      const uint32_t* qp = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.q) + base);
#pragma unroll
      for (int e = 0; e < EPL / 2; ++e) q2[g][e] = qp[e];
    } else if constexpr (QT == PKV_BF16) {
      const uint16_t* qp = static_cast<const uint16_t*>(p.q) + base;
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[g][e] = __uint_as_float(static_cast<uint32_t>(qp[e]) << 16);
    } else {
      const float* qp = static_cast<const float*>(p.q) + base;
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[g][e] = qp[e];
    }
  }

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = neg_inf();
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  // ---- block ids: lane j of a 64-entry chunk holds the id of this wave's
  //      block (chunk*64 + j); ids outside the pool poison the result ----
  const int32_t* trow = p.tables + static_cast<size_t>(b) * p.max_blocks + blk_lo + w;
  int id_chunk = -1;
  int ids = 0;
  bool bad = bad_n;
  auto block_id = [&](int it) -> int {
    const int ch = it >> 6;
    if (ch != id_chunk) {
      id_chunk = ch;
      const int j = (ch << 6) + lane;
      int v = 0;
      bool lane_bad = false;
      if (j < nb_w) {
        v = trow[static_cast<size_t>(j) * NW];
        lane_bad = static_cast<unsigned>(v) >= static_cast<unsigned>(p.num_blocks);
        if (lane_bad) v = 0;
      }
      ids = v;
      bad = bad || wave_any(lane_bad);
    }
    return readlane(ids, it & 63);
  };

  const char* kbase = static_cast<const char*>(p.k) + lane * 16;
  const char* vbase = static_cast<const char*>(p.v) + lane * 16;
  auto load_block = [&](int it, uint4* kb, uint4* vb, float* ksc, float* vsc) {
    const int id = block_id(it);
    const size_t tile = static_cast<size_t>(id) * p.num_kv_heads + kh;
    const char* kt = kbase + tile * kTileBytes;
    const char* vt = vbase + tile * kTileBytes;
#pragma unroll
    for (int i = 0; i < IPB; ++i) kb[i] = *reinterpret_cast<const uint4*>(kt + i * 1024);
#pragma unroll
    for (int i = 0; i < IPB; ++i) vb[i] = *reinterpret_cast<const uint4*>(vt + i * 1024);
    if constexpr (kI8) {
#pragma unroll
      for (int i = 0; i < IPB; ++i) {
        ksc[i] = p.k_scale[tile * kBlock + i * TPI + tslot];
        vsc[i] = p.v_scale[tile * kBlock + i * TPI + tslot];
      }
    }
  };

  auto process = [&](const uint4* kb, const uint4* vb, const float* ksc, const float* vsc, int it) {
    const int tok0 = t0 + (w + it * NW) * kBlock;
    const bool full = tok0 + kBlock <= t1;
    float sc[IPB][G];
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      float kf[EPL];
      if constexpr (!kDot2) unpack16<KV>(kb[i], kf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.f;
        if constexpr (kDot2) {
          const uint32_t kw[4] = {kb[i].x, kb[i].y, kb[i].z, kb[i].w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q2[g][e]),
                                                __builtin_bit_cast(bf16x2_t, kw[e]), d, false);
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) d = fmaf(qf[g][e], kf[e], d);
        }
        d = group_sum<LPT>(d);
        if constexpr (kI8) d *= ksc[i] * p.scale_log2;
        else d *= p.scale_log2;
        if (!full && tok0 + i * TPI + tslot >= t1) d = neg_inf();
        sc[i][g] = d;
      }
    }
    // online softmax update of this lane's token slot
    float mnew[G];
    bool need = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float bm = sc[0][g];
#pragma unroll
      for (int i = 1; i < IPB; ++i) bm = fmaxf(bm, sc[i][g]);
      mnew[g] = fmaxf(m[g], bm);
      need = need || (mnew[g] > m[g]);
    }
    if (wave_any(need)) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float corr = (mnew[g] == neg_inf()) ? 1.f : __builtin_amdgcn_exp2f(m[g] - mnew[g]);
        l[g] *= corr;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= corr;
        m[g] = mnew[g];
      }
    }
    float pr[IPB][G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mu = (m[g] == neg_inf()) ? 0.f : m[g];
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < IPB; ++i) {
        pr[i][g] = __builtin_amdgcn_exp2f(sc[i][g] - mu);
        sum += pr[i][g];
      }
      l[g] += sum;
    }
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      float vf[EPL];
      unpack16<KV>(vb[i], vf);
      // rows past the context (and their int8 scales) may hold NaN: masked
      // tokens contribute by select, never as 0 * NaN
      const bool valid = full || (tok0 + i * TPI + tslot < t1);
      if (!valid) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pw = kI8 ? (valid ? pr[i][g] * vsc[i] : 0.f) : pr[i][g];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(pw, vf[e], acc[g][e]);
      }
    }
  };

  // ---- stream the wave's blocks, one block of K/V prefetched ahead ----
  uint4 ka[IPB], va[IPB], kb[IPB], vb[IPB];
  float ksa[IPB], vsa[IPB], ksb[IPB], vsb[IPB];
  if (nb_w > 0) load_block(0, ka, va, ksa, vsa);
  for (int it = 0; it < nb_w; it += 2) {
    if (it + 1 < nb_w) load_block(it + 1, kb, vb, ksb, vsb);
    process(ka, va, ksa, vsa, it);
    if (it + 2 < nb_w) load_block(it + 2, ka, va, ksa, vsa);
    if (it + 1 < nb_w) process(kb, vb, ksb, vsb, it + 1);
  }

  // ---- merge the TPI token slots of the wave ----
#pragma unroll
  for (int msk = LPT; msk < kWave; msk <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], msk);
      const float lo = __shfl_xor(l[g], msk);
      const float M = fmaxf(m[g], mo);
      const float a = (m[g] == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f(m[g] - M);
      const float bw = (mo == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f(mo - M);
      l[g] = l[g] * a + lo * bw;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = acc[g][e] * a + __shfl_xor(acc[g][e], msk) * bw;
      m[g] = M;
    }
  }

  // ---- merge the wavefronts through LDS and write ----
  if (lane < LPT) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[w][g][c * EPL + e] = acc[g][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      s_m[w][g] = m[g];
      s_l[w][g] = l[g];
    }
    s_bad[w] = bad ? 1 : 0;
  }
  __syncthreads();

  bool any_bad = false;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) any_bad = any_bad || (s_bad[ww] != 0);

  for (int idx = threadIdx.x; idx < G * D; idx += NW * kWave) {
    const int g = idx / D;
    const int d = idx % D;
    float M = neg_inf();
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, s_m[ww][g]);
    float L = 0.f, O = 0.f;
    if (M != neg_inf()) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float mw = s_m[ww][g];
        const float wt = (mw == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L += s_l[ww][g] * wt;
        O += s_acc[ww][g][d] * wt;
      }
    }
    float o, lse;
    if (any_bad) {
      o = qnan();
      lse = qnan();
    } else if (L > 0.f) {
      o = O / L;
      lse = (M + log2f(L)) * kLn2;
    } else {
      o = 0.f;
      lse = neg_inf();
    }
    const int h = h0 + g;
    const size_t row = p.direct ? static_cast<size_t>(b) * p.num_q_heads + h
                                : (static_cast<size_t>(b) * p.max_ns + s) * p.num_q_heads + h;
    p.o[row * D + d] = o;
    if (d == 0 && p.lse != nullptr) p.lse[row] = lse;
  }
}

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

constexpr int kDecodeWaves = 4;

template <int KV, int QT, int D, int G>
hipError_t launch_partial_t(const DecodeParams& p, int batch, hipStream_t st) {
  const dim3 grid(p.direct ? 1 : p.max_ns, p.num_kv_heads, batch);
  hipLaunchKernelGGL((decode_partial_kernel<KV, QT, D, G, kDecodeWaves>), grid, dim3(kDecodeWaves * kWave),
                     0, st, p);
  return hipGetLastError();
}

template <int KV, int QT, int D>
hipError_t launch_partial_g(const DecodeParams& p, int group, int batch, hipStream_t st) {
  switch (group) {
    case 1: return launch_partial_t<KV, QT, D, 1>(p, batch, st);
    case 2: return launch_partial_t<KV, QT, D, 2>(p, batch, st);
    case 4: return launch_partial_t<KV, QT, D, 4>(p, batch, st);
    case 8: return launch_partial_t<KV, QT, D, 8>(p, batch, st);
    default: return hipErrorInvalidValue;
  }
}

template <int KV, int QT>
hipError_t launch_partial_d(const DecodeParams& p, int head_dim, int group, int batch, hipStream_t st) {
  switch (head_dim) {
    case 64: return launch_partial_g<KV, QT, 64>(p, group, batch, st);
    case 128: return launch_partial_g<KV, QT, 128>(p, group, batch, st);
    default: return hipErrorInvalidValue;
  }
}

template <int KV>
hipError_t launch_partial_q(const DecodeParams& p, int q_dtype, int head_dim, int group, int batch,
                            hipStream_t st) {
  switch (q_dtype) {
    case PKV_F32: return launch_partial_d<KV, PKV_F32>(p, head_dim, group, batch, st);
    case PKV_BF16: return launch_partial_d<KV, PKV_BF16>(p, head_dim, group, batch, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_partial(const DecodeParams& p, int kv_dtype, int q_dtype, int head_dim,
                                 int group, int batch, hipStream_t st) {
  switch (kv_dtype) {
    case PKV_F32: return launch_partial_q<PKV_F32>(p, q_dtype, head_dim, group, batch, st);
    case PKV_BF16: return launch_partial_q<PKV_BF16>(p, q_dtype, head_dim, group, batch, st);
    case PKV_I8: return launch_partial_q<PKV_I8>(p, q_dtype, head_dim, group, batch, st);
    default: return hipErrorInvalidValue;
  }
}

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
