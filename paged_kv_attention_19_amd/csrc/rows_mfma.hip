// Chunks of a few rows (speculative verification: a handful of draft rows per
// sequence over a long paged history) on MFMA, with the decode's work mapping.
//
// What is computed (course README "Build an LLM Inference Engine From
// Scratch", curriculum S11 chunked prefill and S12 FlashAttention): row r of
// an L-row chunk of sequence b sits at position n_b - L + r and attends the
// cached tokens t <= n_b - L + r, with softmax(scale * q . k) weighted values,
// online over the sequence's 16-token blocks.
//
// Work mapping. One workgroup of 4 wavefronts per (sequence, kv head); the
// chunk's L rows times the G query heads of the group (at most 16) are the N
// side of 16x16 MFMAs, padded with dead rows. The sequence's blocks are dealt
// to the wavefronts round-robin, as in the decode, and each wavefront keeps
// its own online-softmax state; the four merge through LDS at the end. Per
// block, on each wavefront:
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16, four k-steps over head_dim 128.
//                 K comes from HBM straight into the A-operand layout: lane l
//                 holds token l % 16 and the 32 contiguous dims
//                 [32 (l / 16), +32) of that row (MFMA j takes the 8 dims
//                 32 (l / 16) + 8 j .. +7; q's rows use the same dim order,
//                 which leaves q . k unchanged). The result puts row l % 16 and
//                 tokens 4 (l / 16) .. +3 on lane l.
//   O^T += V^T P^T  v_mfma_f32_16x16x16_bf16, eight dim blocks. The weights
//                 P^T are exactly the S^T registers after the softmax (lane l:
//                 row l % 16, tokens 4 (l / 16) .. +3 is the B-operand layout),
//                 split into a bf16 high part and its bf16 residual (two
//                 products; one bf16 rounding of a weight is too coarse for
//                 rows that see few keys). V is turned to V^T through a
//                 per-wavefront LDS stage: lane l holds tokens 2 (l / 8),
//                 +1 of dims [16 (l % 8), +16) and writes one 4-byte word per
//                 dim (the two tokens' values); the A operand of dim block i
//                 is then one two-word read per lane.
// 8-bit caches convert codes to bf16 on the way (int8 integers and E4M3 values
// are exact in bf16); the K scale multiplies the score, the V scale the
// weight. Row max and denominator are per row: each row lives on the four
// lanes l % 16 = row, whose max is exchanged only when some score exceeds the
// running max by more than the slack (rarely after the first block).
#include <cstdlib>
#include <cstring>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kRowsN = 16;                // query rows per kv head (MFMA N)
constexpr int kVtStride = 9;              // words per dim of a staged V^T block (8 token pairs + 1 pad)
constexpr int kVtWords = kD * kVtStride;  // one stage: 1152 words
constexpr int kStages = 2;
constexpr float kSlack = 8.0f;
constexpr int kXcdsR = 8;

__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Codes B0, B0 + 1 of an 8-bit cache word -> two bf16 (exact).
template <int KV, int B0>
__device__ __forceinline__ uint32_t codes_to_bf16x2(uint32_t w) {
  if constexpr (KV == PKV_I8) {
    return bf16_pair(i8_at(w, B0), i8_at(w, B0 + 1));
  } else {
    const f32x2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), B0 == 2);
    return bf16_pair(f.x, f.y);
  }
}

// The four 8-bit codes of a word -> floats (exact)
template <int KV>
__device__ __forceinline__ void codes4(uint32_t w, float (&f)[4]) {
  if constexpr (KV == PKV_I8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = i8_at(w, i);
  } else {
    const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
    const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
    f[0] = lo.x;
    f[1] = lo.y;
    f[2] = hi.x;
    f[3] = hi.y;
  }
}

template <int KV>
struct RowsTile {
  static constexpr bool kScaled = is_scaled_kv(KV);
  static constexpr int kKLoads = kScaled ? 2 : 4;   // 16-byte loads per lane for K
  static constexpr int kVLoads = kScaled ? 2 : 4;
  uint4 k[kKLoads];
  uint4 v[kVLoads];
  float4 ks, vs;
  int rows;
  int tok0;
};

// NW wavefronts per workgroup, PD blocks of K/V in flight per wavefront while
// one is reduced.
template <int KV, int GQ, int NW, int PD>
__global__ __launch_bounds__(NW * 64) void rows_mfma_kernel(DecodeParams p) {
  constexpr int kNW = NW;
  constexpr bool kScaled = is_scaled_kv(KV);
  constexpr int kRowBytes = kScaled ? kD : 2 * kD;
  using Tile = RowsTile<KV>;
  __shared__ __attribute__((aligned(16))) uint32_t s_vt[kNW][kStages][kVtWords];
  __shared__ int s_bad[kNW];
  static_assert(sizeof(s_vt) >= kNW * kRowsN * (kD + 2) * sizeof(float), "merge area");

  const int nwg = gridDim.x;
  const int item = (blockIdx.x % kXcdsR) * (nwg / kXcdsR) + blockIdx.x / kXcdsR;
  if (item >= p.batch * p.num_kv_heads) return;   // grid padding
  const int kh = item % p.num_kv_heads;
  const int b = item / p.num_kv_heads;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Hq = p.num_q_heads;
  const int Hkv = p.num_kv_heads;

  // block ids of this wavefront's first 64 blocks, in the round trip of n
  int early = 0;
  {
    const int j = w + kNW * lane;
    if (j < p.max_blocks) early = p.tables[static_cast<size_t>(b) * p.max_blocks + j];
  }
  const int n = p.ctx[b];
  const int q0 = p.cu_q[b];
  const int L = p.cu_q[b + 1] - q0;
  if (L == 0) return;
  const bool bad_seq = L < 0 || L > p.max_q_len || L * GQ > kRowsN || n < L ||
                       static_cast<int64_t>(n) > static_cast<int64_t>(p.max_blocks) * kBlock;
  if (bad_seq) {
    for (int64_t idx = threadIdx.x; idx < static_cast<int64_t>(max(L, 0)) * GQ * kD; idx += kNW * 64) {
      const int64_t r = idx / (GQ * kD);
      const int gh = static_cast<int>((idx / kD) % GQ);
      const size_t row = static_cast<size_t>(q0 + r) * Hq + kh * GQ + gh;
      p.o[row * kD + idx % kD] = qnan();
      if (idx % kD == 0 && p.lse != nullptr) p.lse[row] = qnan();
    }
    return;
  }

  // this lane's query row (the MFMA's N index) and its causal limit
  const int row = lane & 15;
  const int rq = row / GQ;                          // row of the chunk
  const bool row_live = rq < L;
  const int lim = row_live ? n - L + rq : -1;       // sees tokens t <= lim
  const int quad = lane >> 4;                        // K dims [32 quad, +32); S^T tokens 4 quad .. +3

  // ---- per-lane load geometry ----
  const int k_off = row * kRowBytes + quad * (kRowBytes / 4);        // K: token `row`, a quarter of the row
  const int va = lane >> 3, vc = lane & 7;                           // V: tokens 2 va, 2 va + 1; dims [16 vc, +16)
  const int v_off0 = (2 * va) * kRowBytes + vc * (kRowBytes / 8);
  const int v_off1 = v_off0 + kRowBytes;
  const char* kpool = static_cast<const char*>(p.k);
  const char* vpool = static_cast<const char*>(p.v);
  const size_t tile_stride = static_cast<size_t>(kBlock) * kRowBytes;

  // Cache policy of the K/V loads. This kernel is bound by each block's
  // chain of latencies, not by bandwidth, and over a 16-bit cache the loads
  // with the default policy return sooner: measured on MI355X (32 sequences
  // of 128..384 tokens, 8 kv heads), 12.8 against 15.2 us at 4 x 2 rows per kv
  // head and 14.5 against 16.6 us at 16 x 1; over an int8 cache the
  // non-temporal loads stay ahead (11.6 against 11.8 us at 4 x 2). The decode
  // kernels, which stream at the bandwidth limit, are the other way round.
  auto ld16 = [](__amdgpu_buffer_rsrc_t r, int off) -> uint4 {
    if constexpr (kScaled) return buffer_load_nt16(r, off);
    else return buffer_load_plain16(r, off);
  };
  auto load_tile = [&](int id, int rows, int tok0, Tile& t) {
    const size_t tile = static_cast<size_t>(id) * Hkv + kh;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kpool + tile * tile_stride, rows * kRowBytes);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(vpool + tile * tile_stride, rows * kRowBytes);
    t.rows = rows;
    t.tok0 = tok0;
#pragma unroll
    for (int i = 0; i < Tile::kKLoads; ++i) t.k[i] = ld16(kr, k_off + 16 * i);
    if constexpr (kScaled) {
      t.v[0] = ld16(vr, v_off0);
      t.v[1] = ld16(vr, v_off1);
      const __amdgpu_buffer_rsrc_t ksr = buffer_rsrc(p.k_scale + tile * kBlock, rows * 4);
      const __amdgpu_buffer_rsrc_t vsr = buffer_rsrc(p.v_scale + tile * kBlock, rows * 4);
      const u32x4v_t a = __builtin_bit_cast(u32x4v_t, __builtin_amdgcn_raw_buffer_load_b128(ksr, 16 * quad, 0, 0));
      const u32x4v_t c = __builtin_bit_cast(u32x4v_t, __builtin_amdgcn_raw_buffer_load_b128(vsr, 16 * quad, 0, 0));
      t.ks = make_float4(__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z), __uint_as_float(a.w));
      t.vs = make_float4(__uint_as_float(c.x), __uint_as_float(c.y), __uint_as_float(c.z), __uint_as_float(c.w));
    } else {
      t.v[0] = ld16(vr, v_off0);
      t.v[1] = ld16(vr, v_off0 + 16);
      t.v[2] = ld16(vr, v_off1);
      t.v[3] = ld16(vr, v_off1 + 16);
    }
  };

  // ---- q rows as B operands (loaded after the first tiles' loads) ----
  bf16x8_t qb[4];
  auto load_q = [&]() {
    const int gh = row % GQ;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                           (static_cast<size_t>(q0 + (row_live ? rq : 0)) * Hq + kh * GQ + gh) * kD + 32 * quad;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (row_live) x = *reinterpret_cast<const uint4*>(qrow + 8 * j);
      qb[j] = __builtin_bit_cast(bf16x8_t, x);
    }
  };

  // K tile -> A operands of the four k-steps
  auto k_operand = [&](const Tile& t, int j) -> bf16x8_t {
    if constexpr (kScaled) {
      const uint4 c = t.k[j >> 1];
      const uint32_t w0 = (j & 1) ? c.z : c.x;
      const uint32_t w1 = (j & 1) ? c.w : c.y;
      const uint4 x = make_uint4(codes_to_bf16x2<KV, 0>(w0), codes_to_bf16x2<KV, 2>(w0), codes_to_bf16x2<KV, 0>(w1),
                                 codes_to_bf16x2<KV, 2>(w1));
      return __builtin_bit_cast(bf16x8_t, x);
    } else {
      return __builtin_bit_cast(bf16x8_t, t.k[j]);
    }
  };

  // V tile -> this wavefront's V^T stage: word (dim d, token pair va) at d * kVtStride + va
  uint32_t* vt_w[kStages];
#pragma unroll
  for (int s = 0; s < kStages; ++s) vt_w[s] = &s_vt[w][s][0];
  auto stage_v = [&](const Tile& t, int s) {
    uint32_t* dst = vt_w[s] + (16 * vc) * kVtStride + va;
    if constexpr (kScaled) {
      const uint32_t a[4] = {t.v[0].x, t.v[0].y, t.v[0].z, t.v[0].w};   // token 2 va, dims 16 vc + 4 u + byte
      const uint32_t c[4] = {t.v[1].x, t.v[1].y, t.v[1].z, t.v[1].w};   // token 2 va + 1
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float fa[4], fc[4];
        codes4<KV>(a[u], fa);
        codes4<KV>(c[u], fc);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(4 * u + i) * kVtStride] = bf16_pair(fa[i], fc[i]);
      }
    } else {
      const uint32_t a[8] = {t.v[0].x, t.v[0].y, t.v[0].z, t.v[0].w, t.v[1].x, t.v[1].y, t.v[1].z, t.v[1].w};
      const uint32_t c[8] = {t.v[2].x, t.v[2].y, t.v[2].z, t.v[2].w, t.v[3].x, t.v[3].y, t.v[3].z, t.v[3].w};
#pragma unroll
      for (int e = 0; e < 16; ++e)
        dst[e * kVtStride] = __builtin_amdgcn_perm(c[e >> 1], a[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
    }
  };
  // A operand of dim block i: dim 16 i + row, tokens 4 quad .. +3
  auto v_operand = [&](int s, int i) -> bf16x4_t {
    const uint32_t* src = vt_w[s] + (16 * i + row) * kVtStride + 2 * quad;
    const u32x2v_t x = {src[0], src[1]};
    return __builtin_bit_cast(bf16x4_t, x);
  };

  // ---- online softmax state of row `row` over this wavefront's tokens ----
  float m = neg_inf(), lsum = 0.f;
  f32x4_t o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const Tile& t, int s) {
    stage_v(t, s);
    f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand(t, j), qb[j], sc, 0, 0, 0);
    float x[4];
    const float ksv[4] = {t.ks.x, t.ks.y, t.ks.z, t.ks.w};
    float bm = neg_inf();
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int tt = 4 * quad + v;
      float xv;
      {
        // rounded here: the max and the exponent use the same value
#pragma clang fp contract(off)
        xv = kScaled ? sc[v] * (ksv[v] * p.scale_log2) : sc[v] * p.scale_log2;
      }
      x[v] = (tt < t.rows && t.tok0 + tt <= lim) ? xv : neg_inf();
      bm = fmaxf(bm, x[v]);
    }
    if (wave_any(bm > m + kSlack)) {
      const float bmr = coset_reduce<16>(bm, OpMax{});   // the row's max over its four lanes
      if (bmr > m + kSlack) {
        const float corr = __builtin_amdgcn_exp2f(m - bmr);   // m = -inf -> 0
        lsum *= corr;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] *= corr;
        m = bmr;
      }
    }
    const float mu = (m == neg_inf()) ? 0.f : m;
    const float vsv[4] = {t.vs.x, t.vs.y, t.vs.z, t.vs.w};
    float pw[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float e = __builtin_amdgcn_exp2f(x[v] - mu);   // -inf -> 0
      lsum += e;
      pw[v] = kScaled ? e * vsv[v] : e;
    }
    const uint32_t h01 = bf16_pair(pw[0], pw[1]), h23 = bf16_pair(pw[2], pw[3]);
    const uint32_t l01 = bf16_pair(pw[0] - __uint_as_float(h01 << 16), pw[1] - __uint_as_float(h01 & 0xffff0000u));
    const uint32_t l23 = bf16_pair(pw[2] - __uint_as_float(h23 << 16), pw[3] - __uint_as_float(h23 & 0xffff0000u));
    const bf16x4_t phi = __builtin_bit_cast(bf16x4_t, u32x2v_t{h01, h23});
    const bf16x4_t plo = __builtin_bit_cast(bf16x4_t, u32x2v_t{l01, l23});
    // the stage's words were written by other lanes of this wavefront: LDS
    // executes a wavefront's accesses in order, and the clobber keeps the
    // compiler from moving the reads above the writes
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16x4_t a = v_operand(s, i);
      o[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, phi, o[i], 0, 0, 0);
      o[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, plo, o[i], 0, 0, 0);
    }
    asm volatile("" ::: "memory");
  };

  // ---- stream this wavefront's blocks w, w + 4, ... ----
  const int nblk = (n + kBlock - 1) / kBlock;
  const int nb_w = nblk > w ? (nblk - w + kNW - 1) / kNW : 0;
  const int32_t* trow = p.tables + static_cast<size_t>(b) * p.max_blocks;
  bool bad = false;
  Tile ring[PD + 1];
  for (int c0 = 0; c0 < nb_w; c0 += 64) {
    const int cn = min(64, nb_w - c0);
    int v = 0;
    if (c0 == 0) v = early;
    else if (lane < cn) v = trow[w + kNW * (c0 + lane)];
    const bool lane_bad = lane < cn && static_cast<unsigned>(v) >= static_cast<unsigned>(p.num_blocks);
    bad = bad || wave_any(lane_bad);
    const int ids = (lane < cn && !lane_bad) ? v : 0;
    auto issue = [&](int it, Tile& t) {
      int rows = 0, id = 0;
      const int blk = w + kNW * (c0 + it);
      if (it < cn) {
        rows = min(kBlock, n - blk * kBlock);
        id = readlane(ids, it);
      }
      load_tile(id, rows, blk * kBlock, t);
    };
#pragma unroll
    for (int k = 0; k < PD; ++k) issue(k, ring[k]);
    if (c0 == 0) load_q();
    for (int it = 0; it < cn; it += PD + 1) {
#pragma unroll
      for (int k = 0; k <= PD; ++k) {
        issue(it + k + PD, ring[(k + PD) % (PD + 1)]);
        if (it + k < cn) process(ring[k], k & 1);
      }
    }
  }

  // ---- merge the four wavefronts' states through LDS ----
  lsum = coset_reduce<16>(lsum, OpAdd{});   // the row's denominator over its four lanes (l, l ^ 16, ...)
  if (lane == 0) s_bad[w] = bad ? 1 : 0;
  __syncthreads();   // every wavefront is done with its V^T stages
  float* mo = reinterpret_cast<float*>(&s_vt[0][0][0]);          // [w][row][kD] then [w][row][m, l]
  float* ml = mo + kNW * kRowsN * kD;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) mo[(w * kRowsN + row) * kD + 16 * i + 4 * quad + v] = o[i][v];
  }
  if (quad == 0) {
    ml[(w * kRowsN + row) * 2] = m;
    ml[(w * kRowsN + row) * 2 + 1] = lsum;
  }
  __syncthreads();
  int bad_or = 0;   // no short-circuit: the flags' reads go out together
#pragma unroll
  for (int ww = 0; ww < kNW; ++ww) bad_or |= s_bad[ww];
  const bool any_bad = bad_or != 0;
  for (int idx = threadIdx.x; idx < kRowsN * kD; idx += kNW * 64) {
    const int rr = idx / kD, d = idx % kD;
    const int r = rr / GQ;
    if (r >= L) continue;
    // no branch on the maxima: every read can go out at once (weight 0 for a
    // wavefront with no finite score)
    float M = neg_inf();
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) M = fmaxf(M, ml[(ww * kRowsN + rr) * 2]);
    float Lt = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) {
      const float mw = ml[(ww * kRowsN + rr) * 2];
      const float a = (mw == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      Lt += ml[(ww * kRowsN + rr) * 2 + 1] * a;
      O += mo[(ww * kRowsN + rr) * kD + d] * a;
    }
    const size_t orow = static_cast<size_t>(q0 + r) * Hq + kh * GQ + rr % GQ;
    p.o[orow * kD + d] = any_bad ? qnan() : O * norm_inv(Lt);
    if (d == 0 && p.lse != nullptr) p.lse[orow] = any_bad ? qnan() : norm_lse2(M, Lt);
  }
}

template <int KV, int NW, int PD>
hipError_t launch_cfg(const DecodeParams& p, int group, hipStream_t st) {
  const int items = p.batch * p.num_kv_heads;
  const int grid = (items + kXcdsR - 1) / kXcdsR * kXcdsR;
  switch (group) {
    case 1: hipLaunchKernelGGL((rows_mfma_kernel<KV, 1, NW, PD>), dim3(grid), dim3(NW * 64), 0, st, p); break;
    case 2: hipLaunchKernelGGL((rows_mfma_kernel<KV, 2, NW, PD>), dim3(grid), dim3(NW * 64), 0, st, p); break;
    case 4: hipLaunchKernelGGL((rows_mfma_kernel<KV, 4, NW, PD>), dim3(grid), dim3(NW * 64), 0, st, p); break;
    case 8: hipLaunchKernelGGL((rows_mfma_kernel<KV, 8, NW, PD>), dim3(grid), dim3(NW * 64), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Wavefronts per workgroup and blocks in flight per wavefront;
// PKV_ROWS_MFMA_CFG ("NW,PD" with NW in {4, 8}, PD in {1, 2}) overrides them,
// for tuning.
template <int KV>
hipError_t launch_kv(const DecodeParams& p, int group, hipStream_t st) {
  static const int cfg = [] {
    const char* e = std::getenv("PKV_ROWS_MFMA_CFG");
    if (e == nullptr) return 0;
    const int nw = std::atoi(e);
    const char* c = std::strchr(e, ',');
    const int pd = c ? std::atoi(c + 1) : 1;
    return ((nw == 4 || nw == 8) && (pd == 1 || pd == 2)) ? nw * 10 + pd : 0;
  }();
  switch (cfg ? cfg : 41) {
    case 42: return launch_cfg<KV, 4, 2>(p, group, st);
    case 81: return launch_cfg<KV, 8, 1>(p, group, st);
    case 82: return launch_cfg<KV, 8, 2>(p, group, st);
    default: return launch_cfg<KV, 4, 1>(p, group, st);
  }
}

}  // namespace

hipError_t launch_rows_mfma(const DecodeParams& p, int kv_dtype, int head_dim, int group, hipStream_t st) {
  if (head_dim != kD || p.max_q_len * group > kRowsN) return hipErrorInvalidValue;
  if (kv_dtype == PKV_BF16) return launch_kv<PKV_BF16>(p, group, st);
  if (kv_dtype == PKV_I8) return launch_kv<PKV_I8>(p, group, st);
  if (kv_dtype == PKV_FP8) return launch_kv<PKV_FP8>(p, group, st);
  return hipErrorInvalidValue;
}

}  // namespace pkv
