// Chunked prefill for gfx950: causal query chunks over a paged KV prefix,
// with bf16 MFMA for both contractions.
//
// What is computed (course README "Build an LLM Inference Engine From
// Scratch", curriculum S11 chunked prefill and S12 FlashAttention): the L new
// rows of a sequence whose cache now holds n tokens (the chunk's own K/V
// included) sit at positions n - L + r and attend keys t <= n - L + r;
// softmax(scale * q . k) weighted values, online over 64-token KV tiles.
//
// Work mapping. A workgroup of 4 wavefronts owns one (sequence, kv head,
// query tile): 128 query rows = (128 / G) positions x the G query heads of the
// GQA group, which all read the same K/V. Each wavefront owns 32 rows. Per
// 64-token KV tile, with v_mfma_f32_32x32x16_bf16 (lane l of a 32x32 result
// holds column l % 32 and rows 8(v/4) + 4(l/32) + v%4 of register v):
//   S^T = K Q^T  (A = K rows from LDS, B = the wavefront's q rows, kept in
//                 registers): every lane holds scores of ONE query row, so the
//                 row max, the causal mask and the softmax state are lane-local
//                 (the two lanes l, l^32 of a row hold its two token halves);
//   O^T = V^T P^T (A = V^T from LDS, B = P^T straight from the S^T registers,
//                 as a bf16 high part plus a bf16 residual, two MFMAs: one
//                 bf16 rounding of a weight (2^-9) is too coarse for rows that
//                 see few keys, the pair keeps ~2^-17): the output accumulator
//                 again holds one query row per lane, so the online rescale is
//                 lane-local.
// K rows are fed to the first product in an order that swaps bits 2 and 3 of
// the row index; with it, the token order of the S^T registers is exactly the
// k order the second product needs, so P never moves between lanes.
// K is staged row-major and V transposed in LDS (the token index must be the
// MFMA k dimension), both XOR-swizzled against bank conflicts, double
// buffered: the next tile's global loads are in flight while this tile's
// MFMAs run. An int8 cache is dequantized on its way to LDS (codes are exact in
// bf16): the K scale multiplies the score column, the V scale the weight.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kD = 128;            // head_dim built
constexpr int kRows = 128;         // query rows per workgroup
constexpr int kTile = 64;          // tokens per KV tile
constexpr int kThreads = 256;
constexpr int kXcdsC = 8;

// LDS byte offsets
constexpr int kKBytes = kTile * kD * 2;    // 16 KiB, row-major [token][dim], swizzled
constexpr int kVBytes = kD * kTile * 2;    // 16 KiB, transposed [dim][token], swizzled

__device__ __forceinline__ int k_addr(int t, int unit) { return t * 256 + ((unit ^ (t & 15)) << 4); }
__device__ __forceinline__ int vt_sw(int d) { return ((d >> 1) ^ (d >> 3)) & 7; }
__device__ __forceinline__ int vt_addr(int d, int unit) { return d * 128 + ((unit ^ vt_sw(d)) << 4); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// int8 code c (sign-extended) -> bfloat16 bits (exact: |c| <= 127).
__device__ __forceinline__ uint32_t i8pair_to_bf16x2(uint32_t w, int byte0) {
  const float a = i8_at(w, byte0), b = i8_at(w, byte0 + 1);
  return pack_bf16(a, b);
}

template <int KV, int G>
__global__ __launch_bounds__(kThreads, 1) void chunked_kernel(ChunkedParams p) {
  constexpr int P = kRows / G;               // positions per query tile
  constexpr bool kI8 = (KV == PKV_I8);
  constexpr float kSlack = 8.0f;
  __shared__ __attribute__((aligned(16))) char s_kv[2][kKBytes + kVBytes];
  __shared__ __attribute__((aligned(16))) float s_ks[2][kTile];
  __shared__ __attribute__((aligned(16))) float s_vs[2][kTile];
  constexpr int kIdsCached = 1024;          // block ids kept in LDS (16384 tokens)
  __shared__ __attribute__((aligned(16))) int s_ids[kIdsCached];

  // ---- work item: (sequence, kv head, query tile), XCD-contiguous ----
  const int QT = (p.max_q_len + P - 1) / P;
  const int nwg = gridDim.x;
  const int item = (blockIdx.x % kXcdsC) * (nwg / kXcdsC) + blockIdx.x / kXcdsC;
  if (item >= p.num_seqs * p.num_kv_heads * QT) return;
  const int qt = QT - 1 - item % QT;               // later (longer) tiles first
  const int kh = (item / QT) % p.num_kv_heads;
  const int seq = item / (QT * p.num_kv_heads);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;                          // which token half of a row this lane holds
  const int rrow = 32 * w + (lane & 31);            // row of the 128-row tile
  const int g = rrow / P;
  const int pi = qt * P + rrow % P;                 // row index within the chunk

  const int q0 = p.cu_q[seq];
  const int L = p.cu_q[seq + 1] - q0;
  const int n = p.ctx[seq];
  if (L <= 0 || qt * P >= L) {
    if (!(L > p.max_q_len && qt == QT - 1)) return;
  }
  const bool bad_seq = L > n || L > p.max_q_len || n < 0 ||
                       static_cast<int64_t>(n) > static_cast<int64_t>(p.max_blocks) * kBlock;
  const int hq = kh * G + g;
  float* out_row = p.out + (static_cast<size_t>(q0 + pi) * p.num_q_heads + hq) * kD;
  if (bad_seq) {
    // rows this tile owns (and, for the last tile, any rows past the grid) become NaN
    const int rows_hi = (qt == QT - 1) ? L : min(L, (qt + 1) * P);
    for (int idx = tid; idx < (rows_hi - qt * P) * G * kD; idx += kThreads) {
      const int r = qt * P + idx / (G * kD);
      const int gg = (idx / kD) % G;
      const size_t o = (static_cast<size_t>(q0 + r) * p.num_q_heads + kh * G + gg) * kD + idx % kD;
      p.out[o] = qnan();
      if (idx % kD == 0 && p.lse != nullptr) p.lse[static_cast<size_t>(q0 + r) * p.num_q_heads + kh * G + gg] = qnan();
    }
    return;
  }
  const bool row_live = pi < L;
  const int pos = n - L + pi;                       // this row attends keys t <= pos

  // ---- q rows as MFMA B operands (k = dims 16 ks + 8 h .. +7) ----
  bf16x8_t qb[8];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                           (static_cast<size_t>(q0 + (row_live ? pi : 0)) * p.num_q_heads + hq) * kD;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (row_live) x = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * h);
      qb[ks] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  // ---- KV range of this query tile ----
  const int last_pi = min(L, (qt + 1) * P) - 1;
  const int kv_end = n - L + last_pi + 1;          // keys [0, kv_end) are visible to some row
  const int ntiles = (kv_end + kTile - 1) / kTile;
  const int first_diag = (n - L + qt * P) / kTile;   // tiles >= this one need the causal mask
  const int nblk_seq = (n + kBlock - 1) / kBlock;
  const int32_t* trow = p.tables + static_cast<size_t>(seq) * p.max_blocks;

  // staging registers for one tile: K 4 chunks, V 4 chunks per thread
  uint4 stk[4];
  uint4 stv[4];
  float sks = 0.f;
  int bad = 0;

  // K chunk i: token 16 i + tid / 16, unit tid % 16 (8 dims)
  // V chunk i: token 4 (tid / 16) + i, unit tid % 16
  // the block ids this tile range needs, read once into LDS (ids past what
  // LDS holds are read from the table when used)
  const int nblk_need = min(nblk_seq, ntiles * (kTile / kBlock));
  for (int j = tid; j < min(nblk_need, kIdsCached); j += kThreads) s_ids[j] = trow[j];
  __syncthreads();

  // Block ids of the 4 blocks of a tile (uniform), read before any of the
  // tile's loads are issued: a lookup between them would make every later
  // load wait for the earlier ones. ok bit bi: block bi exists and is valid.
  auto tile_ids = [&](int tile, int (&id)[4]) -> unsigned {
    const int blk0 = tile * (kTile / kBlock);
    if (blk0 + 4 <= kIdsCached) {
      const int4 x = *reinterpret_cast<const int4*>(&s_ids[blk0]);
      id[0] = x.x; id[1] = x.y; id[2] = x.z; id[3] = x.w;
    } else {
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) id[bi] = blk0 + bi < nblk_seq ? trow[blk0 + bi] : 0;
    }
    unsigned ok = 0;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      id[bi] = __builtin_amdgcn_readfirstlane(id[bi]);
      if (blk0 + bi < nblk_seq) {
        if (static_cast<unsigned>(id[bi]) < static_cast<unsigned>(p.num_blocks)) ok |= 1u << bi;
        else bad = 1;
      }
    }
    return ok;
  };

  auto gload = [&](int tile) {
    const int u = tid & 15;
    const int t0 = tile * kTile;
    constexpr int kRowBytes = kI8 ? kD : 2 * kD;
    int id[4];
    const unsigned ok = tile_ids(tile, id);
    // K chunk i sits in block i of the tile; V chunks of this wavefront in block w
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = t0 + 16 * i + (tid >> 4);
      stk[i] = make_uint4(0, 0, 0, 0);
      if (((ok >> i) & 1u) && tok < n) {
        const char* base = static_cast<const char*>(p.k) +
                           (static_cast<size_t>(id[i]) * p.num_kv_heads + kh) * kBlock * kRowBytes;
        const int off = (tid >> 4) * kRowBytes + u * (kRowBytes / 16);
        if constexpr (kI8) {
          const uint2 c = *reinterpret_cast<const uint2*>(base + off);
          stk[i] = make_uint4(c.x, c.y, 0, 0);
        } else {
          stk[i] = *reinterpret_cast<const uint4*>(base + off);
        }
      }
    }
    const int tg = tid >> 4;
    {
      // tokens 4 tg .. 4 tg + 3 lie in block tg / 4 == w
      const int wu = __builtin_amdgcn_readfirstlane(w);
      const int idw = wu == 0 ? id[0] : wu == 1 ? id[1] : wu == 2 ? id[2] : id[3];
      const bool okw = (ok >> wu) & 1u;
      const char* base = static_cast<const char*>(p.v) +
                         (static_cast<size_t>(idw) * p.num_kv_heads + kh) * kBlock * kRowBytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 4 * tg + i;
        stv[i] = make_uint4(0, 0, 0, 0);
        if (okw && tok < n) {
          const int off = (4 * (tg & 3) + i) * kRowBytes + u * (kRowBytes / 16);
          if constexpr (kI8) {
            const uint2 c = *reinterpret_cast<const uint2*>(base + off);
            stv[i] = make_uint4(c.x, c.y, 0, 0);
          } else {
            stv[i] = *reinterpret_cast<const uint4*>(base + off);
          }
        }
      }
    }
    if constexpr (kI8) {
      // one scale per token: threads 0..63 fetch the tile's K scales, 64..127
      // the V scales
      sks = 0.f;
      if (tid < 2 * kTile) {
        const int tt = tid & (kTile - 1);
        const int tok = t0 + tt;
        const int bi = tt >> 4;
        const int ids = bi == 0 ? id[0] : bi == 1 ? id[1] : bi == 2 ? id[2] : id[3];
        if (((ok >> bi) & 1u) && tok < n) {
          const size_t srow = (static_cast<size_t>(ids) * p.num_kv_heads + kh) * kBlock + (tt & 15);
          // raw scale: any arithmetic on it here would wait for all the tile's loads
          sks = (tid < kTile ? p.k_scale : p.v_scale)[srow];
        }
      }
    }
  };

  auto lstore = [&](int buf) {
    char* kb = s_kv[buf];
    char* vb = s_kv[buf] + kKBytes;
    const int u = tid & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 x = stk[i];
      if constexpr (kI8) {
        x = make_uint4(i8pair_to_bf16x2(stk[i].x, 0), i8pair_to_bf16x2(stk[i].x, 2), i8pair_to_bf16x2(stk[i].y, 0),
                       i8pair_to_bf16x2(stk[i].y, 2));
      }
      *reinterpret_cast<uint4*>(kb + k_addr(16 * i + (tid >> 4), u)) = x;
    }
    // transpose V: thread holds tokens 4 tg .. 4 tg + 3 of dims 8 u .. 8 u + 7
    uint32_t vw[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (kI8) {
        vw[i][0] = i8pair_to_bf16x2(stv[i].x, 0);
        vw[i][1] = i8pair_to_bf16x2(stv[i].x, 2);
        vw[i][2] = i8pair_to_bf16x2(stv[i].y, 0);
        vw[i][3] = i8pair_to_bf16x2(stv[i].y, 2);
      } else {
        vw[i][0] = stv[i].x;
        vw[i][1] = stv[i].y;
        vw[i][2] = stv[i].z;
        vw[i][3] = stv[i].w;
      }
    }
    const int tg = tid >> 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // dim 8 u + e of the 4 tokens: low or high half of word e / 2 of each token
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t lo = __builtin_amdgcn_perm(vw[1][e >> 1], vw[0][e >> 1], sel);
      const uint32_t hi = __builtin_amdgcn_perm(vw[3][e >> 1], vw[2][e >> 1], sel);
      const int d = 8 * u + e;
      *reinterpret_cast<uint2*>(vb + vt_addr(d, tg >> 1) + ((tg & 1) << 3)) = make_uint2(lo, hi);
    }
    if constexpr (kI8) {
      if (tid < kTile) s_ks[buf][tid] = sks * p.scale_log2;   // K scale x softmax scale
      else if (tid < 2 * kTile) s_vs[buf][tid - kTile] = sks;
    }
  };

  // ---- online softmax state of this lane's row ----
  float m = neg_inf(), l = 0.f;
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16_t{};

  // row r of an S^T block is K token sigma(r): bits 2 and 3 of r swapped
  const int ar = lane & 31;
  const int a_tok = (ar & 3) | ((ar & 4) << 1) | ((ar & 8) >> 1) | (ar & 16);

  gload(0);
  lstore(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < ntiles) gload(it + 1);
    const char* kb = s_kv[buf];
    const char* vb = s_kv[buf] + kKBytes;

    // S^T for the two 32-token halves of the tile
    f32x16_t sacc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      sacc[nb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(kb + k_addr(32 * nb + a_tok, 2 * ks + h));
        sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), qb[ks], sacc[nb], 0, 0, 0);
      }
    }

    // int8: the scales of this lane's 32 tokens, as runs of 8 (float4 reads)
    float ksv[2][16], vsv[2][16];
    if constexpr (kI8) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int t0 = 32 * nb + 8 * h + 16 * half;
#pragma unroll
          for (int q4 = 0; q4 < 2; ++q4) {
            const float4 a = *reinterpret_cast<const float4*>(&s_ks[buf][t0 + 4 * q4]);
            const float4 b = *reinterpret_cast<const float4*>(&s_vs[buf][t0 + 4 * q4]);
            const int v0 = 8 * half + 4 * q4;
            ksv[nb][v0] = a.x; ksv[nb][v0 + 1] = a.y; ksv[nb][v0 + 2] = a.z; ksv[nb][v0 + 3] = a.w;
            vsv[nb][v0] = b.x; vsv[nb][v0 + 1] = b.y; vsv[nb][v0 + 2] = b.z; vsv[nb][v0 + 3] = b.w;
          }
        }
      }
    }

    // scores: register v of half nb holds token 32 nb + (v % 8) + 8 h + 16 (v / 8) of the tile
    const int tbase = it * kTile;
    const bool diag = it >= first_diag;
    float tmax = neg_inf();
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tt = 32 * nb + (v & 7) + 8 * h + 16 * (v >> 3);
        float sv;
        if constexpr (kI8) sv = sacc[nb][v] * ksv[nb][v];   // k scale x softmax scale
        else sv = sacc[nb][v] * p.scale_log2;
        if (diag && tbase + tt > pos) sv = neg_inf();
        sacc[nb][v] = sv;
        tmax = fmaxf(tmax, sv);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    // move the reference max only when the tile exceeds it by more than the
    // slack: weights stay below 2^kSlack and O is rarely rescaled
    const bool need = tmax > m + kSlack;
    if (wave_any(need)) {
      const float mnew = need ? tmax : m;
      const float corr = __builtin_amdgcn_exp2f(m - mnew);   // m = -inf -> 0; unchanged -> 1
      l *= corr;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= corr;
      m = mnew;
    }
    const float mu = (m == neg_inf()) ? 0.f : m;
    float rsum = 0.f;
    bf16x8_t phi[4], plo[4];   // P^T as a bf16 high part and a bf16 residual (~2^-17 together)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        // k-step 2 nb + half of the PV product: registers 8 half .. 8 half + 7
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int v = 8 * half + j;
          float pv = __builtin_amdgcn_exp2f(sacc[nb][v] - mu);
          rsum += pv;
          if constexpr (kI8) pv *= vsv[nb][v];
          const __bf16 hi = static_cast<__bf16>(pv);
          phi[2 * nb + half][j] = hi;
          plo[2 * nb + half][j] = static_cast<__bf16>(pv - static_cast<float>(hi));
        }
      }
    }
    rsum += __shfl_xor(rsum, 32);
    l += rsum;

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(vb + vt_addr(32 * db + (lane & 31), 2 * ks + h));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), phi[ks], o[db], 0, 0, 0);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), plo[ks], o[db], 0, 0, 0);
      }
    }

    if (it + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- write: lane holds dims 32 db + 8 (v / 4) + 4 h + v % 4 of its row ----
  bad = __syncthreads_or(bad);
  if (!row_live) return;
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      float4 x = make_float4(o[db][4 * v4] * inv, o[db][4 * v4 + 1] * inv, o[db][4 * v4 + 2] * inv,
                             o[db][4 * v4 + 3] * inv);
      if (bad) x = make_float4(qnan(), qnan(), qnan(), qnan());
      *reinterpret_cast<float4*>(out_row + 32 * db + 8 * v4 + 4 * h) = x;
    }
  }
  if (h == 0 && p.lse != nullptr) {
    const float lse = bad ? qnan() : (l > 0.f ? (m + log2f(l)) * kLn2 : neg_inf());
    p.lse[static_cast<size_t>(q0 + pi) * p.num_q_heads + hq] = lse;
  }
}

template <int KV, int G>
hipError_t launch_t(const ChunkedParams& p, hipStream_t st) {
  constexpr int P = kRows / G;
  const int QT = (p.max_q_len + P - 1) / P;
  const int64_t items = static_cast<int64_t>(p.num_seqs) * p.num_kv_heads * QT;
  if (items > (int64_t(1) << 30)) return hipErrorInvalidValue;
  const int grid = static_cast<int>((items + kXcdsC - 1) / kXcdsC * kXcdsC);
  hipLaunchKernelGGL((chunked_kernel<KV, G>), dim3(grid), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

template <int KV>
hipError_t launch_g(const ChunkedParams& p, int group, hipStream_t st) {
  switch (group) {
    case 1: return launch_t<KV, 1>(p, st);
    case 2: return launch_t<KV, 2>(p, st);
    case 4: return launch_t<KV, 4>(p, st);
    case 8: return launch_t<KV, 8>(p, st);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

hipError_t launch_chunked(const ChunkedParams& p, int kv_dtype, int head_dim, int group, hipStream_t st) {
  if (head_dim != kD) return hipErrorNotSupported;
  if (kv_dtype == PKV_BF16) return launch_g<PKV_BF16>(p, group, st);
  if (kv_dtype == PKV_I8) return launch_g<PKV_I8>(p, group, st);
  return hipErrorNotSupported;
}

}  // namespace pkv
