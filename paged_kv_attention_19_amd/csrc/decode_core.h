// Per-wavefront decode machinery shared by the split-K and the balanced
// decode kernels: the lane layout of a KV tile, the loads, the QK / online
// softmax / PV update of one 16-token block, and the merges of a wavefront's
// token slots.
//
// Lane layout. A (block, kv head) K tile -- 16 rows of head_dim elements --
// is contiguous in HBM. A wavefront reads it with 16-byte loads in which LPT
// consecutive lanes cover a contiguous 16*LPT-byte run of one token row (128
// bytes, a whole cache line, for bf16 head_dim 128) and each lane holds CPL
// such chunks of its row; one load group covers TPI = 64 / LPT tokens. The V
// tile is read the same way. The tile stays in registers and serves all G
// query heads of the GQA group, so every KV byte is read from HBM once. A
// lane's partial q.k is reduced over its LPT lanes with DPP moves; each of the
// TPI token slots keeps its own running max / sum / accumulator (base-2
// exponentials). The running max is only moved when a block's max exceeds it
// by more than kRescaleSlack (weights then stay below 2^kRescaleSlack), which
// spares the accumulator rescale on almost every block; the result is the
// same softmax, normalised by the same reference.
#pragma once

#include <type_traits>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, one L2 each

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// kCausal: the G rows are query rows at different positions of one
// sequence (several new rows per sequence, each with its GQA heads), and row g
// sees only tokens t <= lim[g]; every tile then carries its first token index.
template <int KV, int QT, int D, int G, bool kCausal = false>
struct WaveDecoder {
  using Geo = KvGeom<KV>;
  static constexpr int EPL = Geo::kEpl;                 // elements per 16-byte chunk
  static constexpr int ROWB = D * Geo::kEsize;          // bytes per token row
  static constexpr int ROWC = ROWB / 16;                // chunks per token row
  static constexpr int CPL = ROWC >= 16 ? 2 : 1;        // chunks of a row per lane
  static constexpr int LPT = ROWC / CPL;                // lanes per token row
  static constexpr int TPI = kWave / LPT;               // tokens per load group
  static constexpr int IPB = kBlock / TPI;              // load groups per block tile
  static constexpr int NE = CPL * EPL;                  // row elements per lane
  static constexpr int kTileBytes = kBlock * ROWB;
  static constexpr bool kDot2 = (KV == PKV_BF16 && QT == PKV_BF16);
  // int8 K with bf16 q: q . k as two-wide fp16 dot products over the codes
  // biased into fp16 (1152 + c, exact), q scaled by a power of two per lane
  // into fp16 range (exact for bf16 values), the bias removed once per score
  static constexpr bool kDot2I8 = (KV == PKV_I8 && QT == PKV_BF16);
  static constexpr bool kScaled = is_scaled_kv(KV);   // int8 / fp8 code + scale per row
  static constexpr float kRescaleSlack = 8.0f;
  static_assert(TPI * LPT == kWave && IPB * TPI == kBlock && IPB * CPL * 1024 == kTileBytes, "geometry");

  struct Tile {
    uint4 k[IPB][CPL];
    uint4 v[IPB][CPL];
    float ks[IPB];
    float vs[IPB];
    int rows;   // token rows of the tile that are read (0 .. 16)
    int tok0;   // kCausal: sequence index of the tile's first token
  };

  int lane, tslot, lc, lane_off;
  float qf[G][NE];
  uint32_t q2[G][NE / 2];
  // kDot2I8: q2 holds q's bf16 pairs until the first reduction after load_q
  // turns them, in place, into fp16 pairs scaled by 2^sh (q_ready); qbias is
  // 1152 times the sum of those values and qinv is 2^-sh
  float qbias[G], qinv[G];
  bool q_ready;
  float m[G], l[G], acc[G][NE];
  int lim[G];   // kCausal: row g sees tokens t <= lim[g] (set by the caller)

  __device__ __forceinline__ void init_lane() {
    lane = threadIdx.x & 63;
    tslot = lane / LPT;
    lc = lane % LPT;
    lane_off = tslot * ROWB + lc * 16;   // byte offset of the lane's first chunk in a tile
  }

  // The G query rows of group kh of sequence b, on the lane's NE dims.
  __device__ __forceinline__ void load_q(const void* q, int num_q_heads, int b, int h0) {
    q_ready = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const size_t base = (static_cast<size_t>(b) * num_q_heads + h0 + g) * D + (j * LPT + lc) * EPL;
        if constexpr (kDot2 || kDot2I8) {
          // the chunk's EPL bf16 values, 8 per 16-byte load
#pragma unroll
          for (int u = 0; u < EPL / 8; ++u) {
            const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) + base + 8 * u);
            q2[g][j * (EPL / 2) + 4 * u + 0] = x.x;
            q2[g][j * (EPL / 2) + 4 * u + 1] = x.y;
            q2[g][j * (EPL / 2) + 4 * u + 2] = x.z;
            q2[g][j * (EPL / 2) + 4 * u + 3] = x.w;
          }
        } else if constexpr (QT == PKV_BF16) {
          const uint16_t* qp = static_cast<const uint16_t*>(q) + base;
#pragma unroll
          for (int e = 0; e < EPL; ++e) qf[g][j * EPL + e] = __uint_as_float(static_cast<uint32_t>(qp[e]) << 16);
        } else {
          const float* qp = static_cast<const float*>(q) + base;
#pragma unroll
          for (int e = 0; e < EPL; ++e) qf[g][j * EPL + e] = qp[e];
        }
      }
    }
  }

  // kCausal: the G query rows at element offsets off[g] of q (bf16); rows
  // with live[g] false are zeros.
  __device__ __forceinline__ void load_q_rows(const void* q, const int64_t (&off)[G], const bool (&live)[G]) {
    static_assert(QT == PKV_BF16, "multi-row decode takes bf16 q");
    q_ready = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int64_t base = off[g] + (j * LPT + lc) * EPL;
        if constexpr (kDot2 || kDot2I8) {
#pragma unroll
          for (int u = 0; u < EPL / 8; ++u) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (live[g]) x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) + base + 8 * u);
            q2[g][j * (EPL / 2) + 4 * u + 0] = x.x;
            q2[g][j * (EPL / 2) + 4 * u + 1] = x.y;
            q2[g][j * (EPL / 2) + 4 * u + 2] = x.z;
            q2[g][j * (EPL / 2) + 4 * u + 3] = x.w;
          }
        } else {
          const uint16_t* qp = static_cast<const uint16_t*>(q) + base;
#pragma unroll
          for (int e = 0; e < EPL; ++e) qf[g][j * EPL + e] = live[g] ? __uint_as_float(static_cast<uint32_t>(qp[e]) << 16) : 0.f;
        }
      }
    }
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = neg_inf();
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[g][e] = 0.f;
    }
  }

  // Loads of the (block id, kv head) tile, of which the first `rows` token
  // rows (0 .. 16) are read; id must be a valid block when rows > 0. The
  // loads go through buffer descriptors sized to those rows: the rows past
  // them (the tail of a sequence's last block) read as 0 without touching
  // memory, and a tile with rows == 0 issues its loads with no traffic at
  // all. Every call therefore issues the same instructions, which lets a
  // ring of tiles be filled unconditionally.
  __device__ __forceinline__ void load_tile(const DecodeParams& p, int id, int kh, int rows, Tile& t) const {
    const size_t tile = static_cast<size_t>(id) * p.num_kv_heads + kh;
    const char* kt = static_cast<const char*>(p.k) + tile * kTileBytes;  // uniform bases
    const char* vt = static_cast<const char*>(p.v) + tile * kTileBytes;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kt, rows * ROWB);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(vt, rows * ROWB);
    t.rows = rows;
    // K/V are streamed once per call: non-temporal loads keep them from
    // evicting the block tables, context lengths and q from the caches
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) t.k[i][j] = buffer_load_nt16(kr, lane_off + i * TPI * ROWB + j * LPT * 16);
    }
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) t.v[i][j] = buffer_load_nt16(vr, lane_off + i * TPI * ROWB + j * LPT * 16);
    }
    if constexpr (kScaled) {
      const __amdgpu_buffer_rsrc_t ksr = buffer_rsrc(p.k_scale + tile * kBlock, rows * 4);
      const __amdgpu_buffer_rsrc_t vsr = buffer_rsrc(p.v_scale + tile * kBlock, rows * 4);
#pragma unroll
      for (int i = 0; i < IPB; ++i) {
        t.ks[i] = buffer_load_f32(ksr, (i * TPI + tslot) * 4);
        t.vs[i] = buffer_load_f32(vsr, (i * TPI + tslot) * 4);
      }
    }
  }

  // kDot2I8: q of each head in fp16 pairs. The lane's largest |q| is brought
  // to [2^14, 2^15) by a power of two (exact for bf16 q; a value more than
  // 2^28 below the largest may lose bits as an fp16 subnormal, far below the
  // float32 rounding of the sum).
  __device__ __forceinline__ void prepare_qh() {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = 0.f;
#pragma unroll
      for (int e = 0; e < NE / 2; ++e) mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(q2[g][e])), fabsf(bf16_hi(q2[g][e]))));
      const int sh = mx > 0.f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < NE / 2; ++e) {
        const _Float16 a = static_cast<_Float16>(__builtin_ldexpf(bf16_lo(q2[g][e]), sh));
        const _Float16 c = static_cast<_Float16>(__builtin_ldexpf(bf16_hi(q2[g][e]), sh));
        sum += static_cast<float>(a) + static_cast<float>(c);
        const f16x2_t v = {a, c};
        q2[g][e] = __builtin_bit_cast(uint32_t, v);
      }
      qbias[g] = 1152.0f * sum;
      qinv[g] = __builtin_ldexpf(1.0f, -sh);
    }
    q_ready = true;
  }

  // One block of t.rows tokens (the rest of the tile is masked). The masked
  // rows were read as 0 (K, V and the 8-bit caches' scales), so they add exact zeros:
  // their weights are exp2(-inf) = 0 and their values are finite.
  __device__ __forceinline__ void process(const Tile& t, float scale_log2) {
    if constexpr (kDot2I8) {
      if (!q_ready) prepare_qh();
    }
    float sc[IPB][G];
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      float kf[NE];
      uint32_t kh16[NE / 2];
      if constexpr (kDot2I8) {
        // codes with the sign bit flipped (c + 128) under the fp16 exponent
        // byte 0x64: the fp16 numbers 1024 + c + 128, two per word
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const uint32_t w[4] = {t.k[i][j].x ^ 0x80808080u, t.k[i][j].y ^ 0x80808080u, t.k[i][j].z ^ 0x80808080u,
                                 t.k[i][j].w ^ 0x80808080u};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kh16[j * 8 + 2 * e] = __builtin_amdgcn_perm(0x64646464u, w[e], 0x04010400u);
            kh16[j * 8 + 2 * e + 1] = __builtin_amdgcn_perm(0x64646464u, w[e], 0x04030402u);
          }
        }
      } else if constexpr (!kDot2) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) unpack16<KV>(t.k[i][j], kf + j * EPL);
      }
      const bool valid = i * TPI + tslot < t.rows;
      const int tok = kCausal ? t.tok0 + i * TPI + tslot : 0;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.f;
        if constexpr (kDot2I8) {
#pragma unroll
          for (int e = 0; e < NE / 2; ++e)
            d = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q2[g][e]), __builtin_bit_cast(f16x2_t, kh16[e]), d,
                                       false);
          d = (d - qbias[g]) * qinv[g];
        } else if constexpr (kDot2) {
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
        if constexpr (kScaled) d *= t.ks[i] * scale_log2;
        else d *= scale_log2;
        if constexpr (kCausal) sc[i][g] = (valid && tok <= lim[g]) ? d : neg_inf();
        else sc[i][g] = valid ? d : neg_inf();
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
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float pw = pr[i][g];
        if constexpr (kScaled) pw *= t.vs[i];
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[g][e] = fmaf(pw, vf[e], acc[g][e]);
      }
    }
  }

  // Stream `count` blocks of kv head kh of one sequence through a ring of
  // PD + 1 register tiles (PD blocks in flight while one is reduced). Block j
  // of the stream starts at token tok0 + j * stride * 16 and its id is
  // trow[j * stride]; t1 is the sequence's end (rows past it are masked).
  // Ids are read 64 at a time, one per lane, before their blocks stream; with
  // use_early the first 64 come from `early` (read by the caller beside q).
  // Ids outside the pool set `bad`. Every tile, also past the stream's end, is
  // issued by the same instructions (past the end with a zero-size
  // descriptor), so the compiler's wait counts cover exactly the block being
  // reduced.
  // first_loads() runs once, right after the first tiles' loads are issued:
  // loads that the reduction needs but the tile addresses do not (the q rows)
  // go out there, so the tile loads do not queue behind them (vector memory
  // counts retire in order, and the ids the tile addresses need are waited
  // for with vmcnt(0) at the head of the stream).
  template <int PD, typename FirstLoads>
  __device__ __forceinline__ void stream_blocks(const DecodeParams& p, int kh, const int32_t* trow, int stride,
                                                int tok0, int count, int t1, bool use_early, int early, bool& bad,
                                                FirstLoads&& first_loads) {
    Tile ring[PD + 1];
    for (int c0 = 0; c0 < count; c0 += kWave) {
      const int cn = min(kWave, count - c0);
      int v = 0;
      if (use_early && c0 == 0) v = early;
      else if (lane < cn) v = trow[static_cast<size_t>(c0 + lane) * stride];
      const bool lane_bad = lane < cn && static_cast<unsigned>(v) >= static_cast<unsigned>(p.num_blocks);
      bad = bad || wave_any(lane_bad);
      const int ids = (lane < cn && !lane_bad) ? v : 0;
      auto issue = [&](int it, Tile& t) {
        int rows = 0, id = 0;
        const int first = tok0 + (c0 + it) * stride * kBlock;
        if (it < cn) {
          rows = min(kBlock, t1 - first);
          id = readlane(ids, it);
        }
        load_tile(p, id, kh, rows, t);
        if constexpr (kCausal) t.tok0 = first;
      };
#pragma unroll
      for (int k = 0; k < PD; ++k) issue(k, ring[k]);
      if (c0 == 0) first_loads();
      for (int it = 0; it < cn; it += PD + 1) {
#pragma unroll
        for (int k = 0; k <= PD; ++k) {
          issue(it + k + PD, ring[(k + PD) % (PD + 1)]);
          if (it + k < cn) process(ring[k], p.scale_log2);
        }
      }
    }
  }

  // Bring the token slots to the wavefront's common reference max M.
  __device__ __forceinline__ void slots_to_common_max(float (&M)[G]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mm = m[g];
      mm = coset_reduce<LPT>(mm, OpMax{});
      M[g] = mm;
      const float a = (m[g] == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f(m[g] - mm);
      l[g] *= a;
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[g][e] *= a;
      m[g] = mm;
    }
  }

  // After slots_to_common_max: sum the slots, so every slot holds the
  // wavefront's total (l and acc); lanes 0 .. LPT-1 then hold all D dims.
  __device__ __forceinline__ void sum_slots() {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      l[g] = coset_reduce<LPT>(l[g], OpAdd{});
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[g][e] = coset_reduce<LPT>(acc[g][e], OpAdd{});
    }
  }

  // Dimension of element e of the lane's row chunk j.
  __device__ __forceinline__ int dim_of(int j, int e) const { return (j * LPT + lc) * EPL + e; }
};

}  // namespace pkv
