// Split-K paged decode, partial pass: the kernel template. Instantiated per
// KV element type in decode_f32.hip, decode_bf16.hip and decode_i8.hip.
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
// (block, kv head) K tile -- 16 rows of head_dim elements -- is contiguous in
// HBM; a wavefront reads it with 16-byte loads in which LPT consecutive lanes
// cover a contiguous 16*LPT-byte run of one token row (128 bytes, a whole
// cache line, for bf16 head_dim 128) and each lane holds CPL such chunks of
// its row. The V tile is read the same way. The tile stays in registers and
// serves all G query heads of the GQA group, so every KV byte is read from
// HBM once. A lane's partial q.k is reduced over its LPT lanes with DPP moves;
// each of the TPI token slots of a wavefront keeps its own running max / sum /
// accumulator (base-2 exponentials), merged across slots with lane shuffles
// and across wavefronts through LDS at the end. The running max is only moved
// when a block's max exceeds it by more than kRescaleSlack (weights then stay
// below 2^kRescaleSlack), which spares the accumulator rescale on almost every
// block; the result is the same softmax, normalised by the same reference.
#pragma once

#include <type_traits>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, one L2 each

template <int KV, int QT, int D, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_partial_kernel(DecodeParams p) {
  using Geo = KvGeom<KV>;
  constexpr int EPL = Geo::kEpl;                   // elements per 16-byte chunk
  constexpr int ROWB = D * Geo::kEsize;            // bytes per token row
  constexpr int ROWC = ROWB / 16;                  // chunks per token row
  constexpr int CPL = ROWC >= 16 ? 2 : 1;          // chunks of a row per lane
  constexpr int LPT = ROWC / CPL;                  // lanes per token row
  constexpr int TPI = kWave / LPT;                 // tokens per load group
  constexpr int IPB = kBlock / TPI;                // load groups per block tile
  constexpr int NE = CPL * EPL;                    // row elements per lane
  constexpr int kTileBytes = kBlock * ROWB;
  constexpr bool kDot2 = (KV == PKV_BF16 && QT == PKV_BF16);
  constexpr bool kI8 = (KV == PKV_I8);
  constexpr float kRescaleSlack = 8.0f;
  static_assert(TPI * LPT == kWave && IPB * TPI == kBlock && IPB * CPL * 1024 == kTileBytes, "geometry");

  // cross-slot merge through LDS when the (wave, slot) states fit in 64 KiB
  constexpr bool kLdsMerge = NW * TPI * G * D * 4 <= 65536;
  constexpr int kSlots = kLdsMerge ? TPI : 1;
  __shared__ float s_part[NW][kSlots][G][D];
  __shared__ float s_lp[NW][kSlots][G];
  __shared__ float s_m[NW][G];
  __shared__ int s_bad[NW];

  // Workgroup i runs on XCD i % 8. Renumber so that each XCD gets one
  // contiguous range of work items, with the kv heads of a (sequence, split)
  // adjacent: they share the sequence's block-table entries and context length
  // in that XCD's L2.
  const int nwg = gridDim.x;
  const int item = (blockIdx.x % kXcds) * (nwg / kXcds) + blockIdx.x / kXcds;
  const int S = p.direct ? 1 : p.max_ns;
  if (item >= p.batch * S * p.num_kv_heads) return;  // grid padding
  const int kh = item % p.num_kv_heads;
  const int s = (item / p.num_kv_heads) % S;
  const int b = item / (p.num_kv_heads * S);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tslot = lane / LPT;
  const int lc = lane % LPT;
  const int lane_off = tslot * ROWB + lc * 16;     // byte offset of the lane's first chunk in a tile

  // ---- the G query rows of this group, on the lane's NE dims ----
  const int h0 = kh * G;
  float qf[G][NE];
  uint32_t q2[G][NE / 2];
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const size_t base = (static_cast<size_t>(b) * p.num_q_heads + h0 + g) * D + (j * LPT + lc) * EPL;
      if constexpr (kDot2) {
        const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + base);
        q2[g][4 * j + 0] = x.x;
        q2[g][4 * j + 1] = x.y;
        q2[g][4 * j + 2] = x.z;
        q2[g][4 * j + 3] = x.w;
      } else if constexpr (QT == PKV_BF16) {
        const uint16_t* qp = static_cast<const uint16_t*>(p.q) + base;
#pragma unroll
        for (int e = 0; e < EPL; ++e) qf[g][j * EPL + e] = __uint_as_float(static_cast<uint32_t>(qp[e]) << 16);
      } else {
        const float* qp = static_cast<const float*>(p.q) + base;
#pragma unroll
        for (int e = 0; e < EPL; ++e) qf[g][j * EPL + e] = qp[e];
      }
    }
  }

  // Split 0 always starts at block 0, so its first table entries can be read
  // in the same round trip as q and the context length (entries past the
  // context are discarded once n is known; the row has max_blocks entries).
  int early_ids = 0;
  if (s == 0) {
    const int j = w + NW * lane;
    if (j < p.max_blocks) early_ids = p.tables[static_cast<size_t>(b) * p.max_blocks + j];
  }
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

  float m[G], l[G], acc[G][NE];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = neg_inf();
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[g][e] = 0.f;
  }

  // ---- block ids: lane j of a 64-entry chunk holds the id of this wave's
  //      block (chunk*64 + j); ids outside the pool poison the result ----
  const int32_t* trow = p.tables + static_cast<size_t>(b) * p.max_blocks + blk_lo + w;
  int id_chunk = -1;
  int ids = 0;
  bool bad = bad_n;
  auto fetch_ids = [&](int ch) {
    const int j = (ch << 6) + lane;
    int v = 0;
    bool lane_bad = false;
    if (j < nb_w) {
      v = trow[static_cast<size_t>(j) * NW];
      lane_bad = static_cast<unsigned>(v) >= static_cast<unsigned>(p.num_blocks);
      if (lane_bad) v = 0;
    }
    ids = v;
    id_chunk = ch;
    bad = bad || wave_any(lane_bad);
  };
  auto block_id = [&](int it) -> int {
    if ((it >> 6) != id_chunk) fetch_ids(it >> 6);
    return readlane(ids, it & 63);
  };
  if (s == 0 && nb_w > 0) {  // blk_lo == 0: the early read holds this wave's first 64 ids
    const bool lane_bad = lane < nb_w && static_cast<unsigned>(early_ids) >= static_cast<unsigned>(p.num_blocks);
    ids = lane_bad ? 0 : early_ids;
    id_chunk = 0;
    bad = bad || wave_any(lane_bad);
  }

  struct Tile {
    uint4 k[IPB][CPL];
    uint4 v[IPB][CPL];
    float ks[IPB];
    float vs[IPB];
  };

  auto load_block = [&](int it, Tile& t) {
    const int id = block_id(it);
    const size_t tile = static_cast<size_t>(id) * p.num_kv_heads + kh;
    // K/V are streamed once per call: non-temporal loads keep them from
    // evicting the block tables, context lengths and q from the caches
    const char* kt = static_cast<const char*>(p.k) + tile * kTileBytes;  // uniform base
    const char* vt = static_cast<const char*>(p.v) + tile * kTileBytes;
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
#pragma unroll
      for (int j = 0; j < CPL; ++j)
        t.k[i][j] = load_nt16(kt + lane_off + i * TPI * ROWB + j * LPT * 16);
    }
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
#pragma unroll
      for (int j = 0; j < CPL; ++j)
        t.v[i][j] = load_nt16(vt + lane_off + i * TPI * ROWB + j * LPT * 16);
    }
    if constexpr (kI8) {
#pragma unroll
      for (int i = 0; i < IPB; ++i) {
        t.ks[i] = p.k_scale[tile * kBlock + i * TPI + tslot];
        t.vs[i] = p.v_scale[tile * kBlock + i * TPI + tslot];
      }
    }
  };

  auto process = [&](const Tile& t, int it, auto full_tag) {
    constexpr bool kFull = decltype(full_tag)::value;
    const int tok0 = t0 + (w + it * NW) * kBlock;
    float sc[IPB][G];
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      float kf[NE];
      if constexpr (!kDot2) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) unpack16<KV>(t.k[i][j], kf + j * EPL);
      }
      const bool valid = kFull || (tok0 + i * TPI + tslot < t1);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.f;
        if constexpr (kDot2) {
#pragma unroll
          for (int j = 0; j < CPL; ++j) {
            const uint32_t kw[4] = {t.k[i][j].x, t.k[i][j].y, t.k[i][j].z, t.k[i][j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q2[g][4 * j + e]),
                                                  __builtin_bit_cast(bf16x2_t, kw[e]), d, false);
          }
        } else {
#pragma unroll
          for (int e = 0; e < NE; ++e) d = fmaf(qf[g][e], kf[e], d);
        }
        d = group_sum<LPT>(d);
        if constexpr (kI8) d *= t.ks[i] * p.scale_log2;
        else d *= p.scale_log2;
        if constexpr (!kFull) d = valid ? d : neg_inf();
        sc[i][g] = d;
      }
    }
    // online softmax: move the reference max only when a block exceeds it by
    // more than the slack (or the slot had no finite score yet)
    bool need = false;
    float bm[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      bm[g] = sc[0][g];
#pragma unroll
      for (int i = 1; i < IPB; ++i) bm[g] = fmaxf(bm[g], sc[i][g]);
      need = need || (bm[g] > m[g] + kRescaleSlack);
    }
    if (wave_any(need)) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (bm[g] > m[g] + kRescaleSlack) {
          const float corr = __builtin_amdgcn_exp2f(m[g] - bm[g]);  // m = -inf -> 0
          l[g] *= corr;
#pragma unroll
          for (int e = 0; e < NE; ++e) acc[g][e] *= corr;
          m[g] = bm[g];
        }
      }
    }
    float pr[IPB][G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mu = (m[g] == neg_inf()) ? 0.f : m[g];
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < IPB; ++i) {
        pr[i][g] = __builtin_amdgcn_exp2f(sc[i][g] - mu);  // -inf -> 0
        sum += pr[i][g];
      }
      l[g] += sum;
    }
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      float vf[NE];
#pragma unroll
      for (int j = 0; j < CPL; ++j) unpack16<KV>(t.v[i][j], vf + j * EPL);
      // rows past the context (and their int8 scales) may hold NaN: masked
      // tokens contribute by select, never as 0 * NaN
      const bool valid = kFull || (tok0 + i * TPI + tslot < t1);
      if constexpr (!kFull) {
#pragma unroll
        for (int e = 0; e < NE; ++e) vf[e] = valid ? vf[e] : 0.f;
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float pw = pr[i][g];
        if constexpr (kI8) pw = (kFull || valid) ? pw * t.vs[i] : 0.f;
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[g][e] = fmaf(pw, vf[e], acc[g][e]);
      }
    }
  };

  auto run = [&](const Tile& t, int it) {
    const int tok0 = t0 + (w + it * NW) * kBlock;
    if (tok0 + kBlock <= t1) process(t, it, std::true_type{});
    else process(t, it, std::false_type{});
  };

  // ---- stream the wave's blocks, two blocks of K/V in flight ahead ----
  Tile ta, tb, tc;
  if (nb_w > 0) load_block(0, ta);
  if (nb_w > 1) load_block(1, tb);
  for (int it = 0; it < nb_w; it += 3) {
    if (it + 2 < nb_w) load_block(it + 2, tc);
    run(ta, it);
    if (it + 3 < nb_w) load_block(it + 3, ta);
    if (it + 1 < nb_w) run(tb, it + 1);
    if (it + 4 < nb_w) load_block(it + 4, tb);
    if (it + 2 < nb_w) run(tc, it + 2);
  }

  // ---- merge: bring the wave's token slots to one reference max ----
  float M[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mm = m[g];
#pragma unroll
    for (int msk = LPT; msk < kWave; msk <<= 1) mm = fmaxf(mm, __shfl_xor(mm, msk));
    M[g] = mm;
    const float a = (m[g] == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f(m[g] - mm);
    l[g] *= a;
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[g][e] *= a;
  }
  if constexpr (kLdsMerge) {
    // every (wave, slot) state goes to LDS; the output threads sum them
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_part[w][tslot][g][(j * LPT + lc) * EPL + e] = acc[g][j * EPL + e];
      }
      if (lc == 0) s_lp[w][tslot][g] = l[g];
    }
  } else {
    // sum the slots with lane shuffles first, then one state per wave
#pragma unroll
    for (int msk = LPT; msk < kWave; msk <<= 1) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        l[g] += __shfl_xor(l[g], msk);
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[g][e] += __shfl_xor(acc[g][e], msk);
      }
    }
    if (lane < LPT) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) s_part[w][0][g][(j * LPT + lc) * EPL + e] = acc[g][j * EPL + e];
        }
        if (lc == 0) s_lp[w][0][g] = l[g];
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) s_m[w][g] = M[g];
    s_bad[w] = bad ? 1 : 0;
  }
  __syncthreads();

  bool any_bad = false;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) any_bad = any_bad || (s_bad[ww] != 0);

  for (int idx = threadIdx.x; idx < G * D; idx += NW * kWave) {
    const int g = idx / D;
    const int d = idx % D;
    float Mx = neg_inf();
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) Mx = fmaxf(Mx, s_m[ww][g]);
    float L = 0.f, O = 0.f;
    if (Mx != neg_inf()) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float mw = s_m[ww][g];
        const float wt = (mw == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f(mw - Mx);
        float ls = 0.f, os = 0.f;
#pragma unroll
        for (int t = 0; t < kSlots; ++t) {
          ls += s_lp[ww][t][g];
          os += s_part[ww][t][g][d];
        }
        L += ls * wt;
        O += os * wt;
      }
    }
    float o, lse;
    if (any_bad) {
      o = qnan();
      lse = qnan();
    } else if (L > 0.f) {
      o = O / L;
      lse = (Mx + log2f(L)) * kLn2;
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

// Host-side dispatch over the compile-time shape parameters of one KV type.
template <int KV, int QT, int D, int G, int NW>
hipError_t launch_partial_t(const DecodeParams& p, hipStream_t st) {
  const int items = p.batch * (p.direct ? 1 : p.max_ns) * p.num_kv_heads;
  const int grid = (items + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((decode_partial_kernel<KV, QT, D, G, NW>), dim3(grid), dim3(NW * kWave), 0, st, p);
  return hipGetLastError();
}

template <int KV, int QT, int D, int G>
hipError_t launch_partial_w(const DecodeParams& p, int waves, hipStream_t st) {
  switch (waves) {
    case 2: return launch_partial_t<KV, QT, D, G, 2>(p, st);
    case 4: return launch_partial_t<KV, QT, D, G, 4>(p, st);
    case 8: return launch_partial_t<KV, QT, D, G, 8>(p, st);
    default: return hipErrorInvalidValue;
  }
}

template <int KV, int QT, int D>
hipError_t launch_partial_g(const DecodeParams& p, int group, int waves, hipStream_t st) {
  switch (group) {
    case 1: return launch_partial_w<KV, QT, D, 1>(p, waves, st);
    case 2: return launch_partial_w<KV, QT, D, 2>(p, waves, st);
    case 4: return launch_partial_w<KV, QT, D, 4>(p, waves, st);
    case 8: return launch_partial_w<KV, QT, D, 8>(p, waves, st);
    default: return hipErrorInvalidValue;
  }
}

template <int KV>
hipError_t launch_partial_kv(const DecodeParams& p, int q_dtype, int head_dim, int group, int waves,
                             hipStream_t st) {
  if (q_dtype == PKV_F32) {
    if (head_dim == 64) return launch_partial_g<KV, PKV_F32, 64>(p, group, waves, st);
    if (head_dim == 128) return launch_partial_g<KV, PKV_F32, 128>(p, group, waves, st);
  } else if (q_dtype == PKV_BF16) {
    if (head_dim == 64) return launch_partial_g<KV, PKV_BF16, 64>(p, group, waves, st);
    if (head_dim == 128) return launch_partial_g<KV, PKV_BF16, 128>(p, group, waves, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
