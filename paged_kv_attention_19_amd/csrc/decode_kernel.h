// Decode kernels for gfx950: the split-K partial pass and the balanced
// single-launch decode. Instantiated per KV element type in decode_f32.hip,
// decode_bf16.hip and decode_i8.hip.
//
// What is computed (course README "Build an LLM Inference Engine From
// Scratch", curriculum S06 PagedAttention and S12 FlashAttention; claims s06
// and s12 in section "The code asserts its own claims"): for every sequence b
// and query head h, softmax(scale * q_h . k_t) weighted values over the
// sequence's tokens t < n_b, the K/V rows read through the block table.
//
// Split-K: the tokens are cut into num_splits[b] block-aligned ranges; one
// workgroup of NW wavefronts reduces each (split, kv head, sequence) with an
// online softmax to (o_s, lse_s), and the ranges are merged by log-sum-exp.
//
// Balanced: the (sequence, kv head, block) tiles of the whole batch, in that
// order, are dealt to the wavefronts of the grid in equal contiguous ranges,
// so every CU streams the same number of KV bytes whatever the context
// lengths. A (sequence, kv head) segment that falls inside one range is
// written directly; one that a range boundary cuts leaves a partial per
// contributing wavefront (agent-coherent stores), and the last contributor to
// finish (a device-atomic arrival counter) merges them by log-sum-exp, in the
// same launch.
#pragma once

#include "decode_core.h"
#include "quant_row.h"

namespace pkv {

// Append (split mode): one wavefront writes the new K and V rows of kv head
// kh of sequence b to slot p.slots[b] (skipped when the slot is outside the
// pool), with the same per-row arithmetic as reshape_and_cache. The rows are
// read as one 16-byte piece per lane (a row is at most 512 bytes, so K and V
// take at most 64 pieces):
//   scaled 8-bit caches: lanes [0, R) hold K's pieces, [R, 2R) V's, with
//                        R = D / (source elements per 16 bytes);
//   other caches       : the rows are copied as they are, K's pieces then V's.
// Every lane loads: lanes past the row's pieces load one of them again (the
// same lines, in bounds), so the load needs no branch and no merge of values
// that would make the wavefront wait for it on the spot.
template <int KV, int D>
__device__ __forceinline__ uint4 load_new_piece(const DecodeParams& p, int b, int kh, int lane) {
  const int64_t row = static_cast<int64_t>(b) * p.num_kv_heads + kh;
  if constexpr (is_scaled_kv(KV)) {
    const int esize = p.new_dtype == PKV_BF16 ? 2 : 4;
    const int R = D * esize / 16;
    const int i = lane % (2 * R);
    const bool isv = i >= R;
    return *reinterpret_cast<const uint4*>(static_cast<const char*>(isv ? p.v_new : p.k_new) + row * D * esize +
                                           (i % R) * 16);
  } else {
    constexpr int kRowBytes = D * KvGeom<KV>::kEsize;
    constexpr int kPieces = kRowBytes / 16;
    static_assert(2 * kPieces <= kWave, "K and V pieces of a row fit one wavefront");
    const int i = lane % (2 * kPieces);
    const bool isv = i >= kPieces;
    return *reinterpret_cast<const uint4*>(static_cast<const char*>(isv ? p.v_new : p.k_new) + row * kRowBytes +
                                           (i % kPieces) * 16);
  }
}

template <int SRC, int D, int KV>
__device__ __forceinline__ void store_quant(const DecodeParams& p, uint4 piece, int64_t dst_row, int lane) {
  constexpr int R = D / KvGeom<SRC>::kEpl;
  if (lane < 2 * R) {
    const bool isv = lane >= R;
    quantize_piece<SRC, D, KV>(piece, isv ? p.v_w : p.k_w, isv ? p.v_scale_w : p.k_scale_w, dst_row, lane % R);
  }
}

template <int KV, int D>
__device__ __forceinline__ void store_new_piece(const DecodeParams& p, uint4 piece, int64_t slot, int kh, int lane) {
  if (slot < 0 || slot >= p.num_slots) return;
  const int64_t dst_row = ((slot / kBlock) * p.num_kv_heads + kh) * kBlock + slot % kBlock;
  if constexpr (is_scaled_kv(KV)) {
    if (p.new_dtype == PKV_BF16) store_quant<PKV_BF16, D, KV>(p, piece, dst_row, lane);
    else store_quant<PKV_F32, D, KV>(p, piece, dst_row, lane);
  } else {
    constexpr int kRowBytes = D * KvGeom<KV>::kEsize;
    constexpr int kPieces = kRowBytes / 16;
    if (lane < 2 * kPieces) {
      const bool isv = lane >= kPieces;
      *reinterpret_cast<uint4*>(static_cast<char*>(isv ? p.v_w : p.k_w) + dst_row * kRowBytes +
                                (lane % kPieces) * 16) = piece;
    }
  }
}

template <int KV, int QT, int D, int G, int NW, int PD>
__global__ __launch_bounds__(NW * 64) void decode_partial_kernel(DecodeParams p) {
  using WD = WaveDecoder<KV, QT, D, G>;
  constexpr int LPT = WD::LPT, TPI = WD::TPI, CPL = WD::CPL, EPL = WD::EPL;

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
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  WD wd;
  wd.init_lane();
  const int lane = wd.lane;
  const int h0 = kh * G;

  // Split 0 always starts at block 0, so its first table entries can be read
  // in the same round trip as the context length (entries past the
  // context are discarded once n is known; the row has max_blocks entries).
  int early_ids = 0;
  if (s == 0) {
    const int j = w + NW * lane;
    if (j < p.max_blocks) early_ids = p.tables[static_cast<size_t>(b) * p.max_blocks + j];
  }
  const int n = p.ctx[b];
  const int ns = p.direct ? 1 : p.nsplits[b];
  // The step's new rows and their slot go out in the same round trip: which
  // wavefront writes them is known only once n is, and loading them then
  // would cost that wavefront a round trip more than the others. The empty
  // asm with a memory clobber keeps the compiler from sinking these loads
  // into the branch that uses them.
  uint4 new_piece{};
  int64_t new_slot = -1;
  if (p.k_new != nullptr) {
    new_piece = load_new_piece<KV, D>(p, b, kh, lane);
    new_slot = p.slots[b];
  }
  asm volatile("" ::: "memory");
  if (ns < 1 || s >= ns) return;  // not a split of this sequence (the merge checks ns)

  const bool bad_n = (n < 0) || (static_cast<int64_t>(n) > static_cast<int64_t>(p.max_blocks) * kBlock);
  int t0 = 0, t1 = 0, tps = 0;
  if (!bad_n && n > 0) {
    const int per = (n + ns - 1) / ns;
    tps = ((per + kBlock - 1) / kBlock) * kBlock;
    const int64_t a = static_cast<int64_t>(s) * tps;
    t0 = a < n ? static_cast<int>(a) : n;
    t1 = (static_cast<int64_t>(t0) + tps) < n ? t0 + tps : n;
  }
  const int blk_lo = t0 / kBlock;
  const int nblk = (t1 - t0 + kBlock - 1) / kBlock;
  const int nb_w = nblk > w ? (nblk - w + NW - 1) / NW : 0;

  // Append: the wavefront that reads the block of token n - 1 (in split
  // (n - 1) / tps, where the block is dealt to wavefront (its index in the
  // split) % NW; trailing splits may be empty) writes the new rows first and
  // waits for those stores to complete before it issues any tile load, so its
  // read of the block sees them. No other wavefront reads that block. With no
  // tokens to read, split 0's wavefront 0 writes them.
  if (p.k_new != nullptr) {
    const bool has_tail = !bad_n && n > 0;
    const int s_tail = has_tail ? (n - 1) / tps : 0;
    const int w_tail = has_tail ? ((n - 1) / kBlock - blk_lo) % NW : 0;
    if (s == s_tail && w == w_tail) {
      store_new_piece<KV, D>(p, new_piece, new_slot, kh, lane);
      // the row stores have completed before any tile load is issued (a
      // workgroup-scope fence does not wait for them); the memory clobbers
      // keep the compiler from moving the stores or the loads across the wait
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0);
      asm volatile("" ::: "memory");
    }
  }

  wd.reset();

  // ---- stream this wave's blocks: blocks w, w + NW, ... of the split ----
  bool bad = bad_n;
  // q is loaded after the first tiles' loads are issued (it is needed only
  // once the first tile is reduced; a wavefront with no blocks never needs it)
  wd.template stream_blocks<PD>(p, kh, p.tables + static_cast<size_t>(b) * p.max_blocks + blk_lo + w, NW,
                                t0 + w * kBlock, nb_w, t1, s == 0, early_ids, bad,
                                [&] { wd.load_q(p.q, p.num_q_heads, b, h0); });

  // ---- merge: bring the wave's token slots to one reference max ----
  float M[G];
  wd.slots_to_common_max(M);
  const int tslot = wd.tslot, lc = wd.lc;
  if constexpr (kLdsMerge) {
    // every (wave, slot) state goes to LDS; the output threads sum them
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_part[w][tslot][g][wd.dim_of(j, e)] = wd.acc[g][j * EPL + e];
      }
      if (lc == 0) s_lp[w][tslot][g] = wd.l[g];
    }
  } else {
    // sum the slots with lane shuffles first, then one state per wave
    wd.sum_slots();
    if (lane < LPT) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) s_part[w][0][g][wd.dim_of(j, e)] = wd.acc[g][j * EPL + e];
        }
        if (lc == 0) s_lp[w][0][g] = wd.l[g];
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) s_m[w][g] = M[g];
    s_bad[w] = bad ? 1 : 0;
  }
  __syncthreads();

  int bad_or = 0;   // no short-circuit: the flags' reads go out together
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) bad_or |= s_bad[ww];
  const bool any_bad = bad_or != 0;

  for (int idx = threadIdx.x; idx < G * D; idx += NW * kWave) {
    const int g = idx / D;
    const int d = idx % D;
    // No branch on the maxima: every LDS read of the merge can go out at
    // once. A wavefront with no finite score (mw = -inf) gets weight 0; with
    // none anywhere, L = 0.
    float Mx = neg_inf();
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) Mx = fmaxf(Mx, s_m[ww][g]);
    float L = 0.f, O = 0.f;
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
    float o, lse;
    if (any_bad) {
      o = qnan();
      lse = qnan();
    } else if (L > 0.f) {
      o = O / L;
      lse = (Mx + log2f(L)) * kLn2;
    } else if (L == 0.f) {
      o = 0.f;
      lse = neg_inf();
    } else {   // a NaN was read
      o = qnan();
      lse = qnan();
    }
    const int h = h0 + g;
    const size_t row = p.direct ? static_cast<size_t>(b) * p.num_q_heads + h
                                : (static_cast<size_t>(b) * p.max_ns + s) * p.num_q_heads + h;
    p.o[row * D + d] = o;
    if (d == 0 && p.lse != nullptr) p.lse[row] = lse;
  }
}

// Several new rows per sequence: the L_b rows of sequence b (chunk rows at
// positions n_b - L_b + r; speculative verification, or any chunk of a few
// rows) with the GQ query heads of kv head kh, R = L * GQ rows in all (padded
// to a power of two), share every K/V tile the wavefronts stream, as the GQA
// heads of one decode row do. Row r sees tokens t <= n_b - L_b + r (course
// README "Build an LLM Inference Engine From Scratch", curriculum S11 chunked
// prefill: a chunk's rows attend the cached prefix and the chunk's own earlier
// rows). One workgroup of NW wavefronts per (sequence, kv head) streams the
// whole sequence, blocks dealt round-robin, and merges through LDS.
template <int KV, int D, int GQ, int R, int NW>
__global__ __launch_bounds__(NW * 64) void decode_rows_kernel(DecodeParams p) {
  using WD = WaveDecoder<KV, PKV_BF16, D, R, true>;
  constexpr int LPT = WD::LPT, TPI = WD::TPI, CPL = WD::CPL, EPL = WD::EPL;
  static_assert(R % GQ == 0, "whole rows");
  constexpr bool kLdsMerge = NW * TPI * R * D * 4 <= 65536;
  constexpr int kSlots = kLdsMerge ? TPI : 1;
  __shared__ float s_part[NW][kSlots][R][D];
  __shared__ float s_lp[NW][kSlots][R];
  __shared__ float s_m[NW][R];
  __shared__ int s_bad[NW];

  const int nwg = gridDim.x;
  const int item = (blockIdx.x % kXcds) * (nwg / kXcds) + blockIdx.x / kXcds;
  if (item >= p.batch * p.num_kv_heads) return;   // grid padding
  const int kh = item % p.num_kv_heads;
  const int b = item / p.num_kv_heads;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Hq = p.num_q_heads;

  WD wd;
  wd.init_lane();
  const int lane = wd.lane;
  int early_ids = 0;
  {
    const int j = w + NW * lane;
    if (j < p.max_blocks) early_ids = p.tables[static_cast<size_t>(b) * p.max_blocks + j];
  }
  const int n = p.ctx[b];
  const int q0 = p.cu_q[b];
  const int L = p.cu_q[b + 1] - q0;
  if (L == 0) return;
  const bool bad_seq = L < 0 || L > p.max_q_len || L * GQ > R || n < L ||
                       static_cast<int64_t>(n) > static_cast<int64_t>(p.max_blocks) * kBlock;
  if (bad_seq) {
    // the chunk's rows of this kv head's query heads become NaN
    for (int64_t idx = threadIdx.x; idx < static_cast<int64_t>(max(L, 0)) * GQ * D; idx += NW * kWave) {
      const int64_t r = idx / (GQ * D);
      const int gh = static_cast<int>((idx / D) % GQ);
      const size_t row = static_cast<size_t>(q0 + r) * Hq + kh * GQ + gh;
      p.o[row * D + idx % D] = qnan();
      if (idx % D == 0 && p.lse != nullptr) p.lse[row] = qnan();
    }
    return;
  }

  int64_t off[R];
  bool live[R];
#pragma unroll
  for (int g = 0; g < R; ++g) {
    const int r = g / GQ;
    live[g] = r < L;
    off[g] = (static_cast<int64_t>(q0 + (live[g] ? r : 0)) * Hq + kh * GQ + g % GQ) * D;
    wd.lim[g] = n - L + r;
  }
  const int nblk = (n + kBlock - 1) / kBlock;
  const int nb_w = nblk > w ? (nblk - w + NW - 1) / NW : 0;
  wd.reset();
  bool bad = false;
  wd.template stream_blocks<1>(p, kh, p.tables + static_cast<size_t>(b) * p.max_blocks + w, NW, w * kBlock, nb_w, n,
                               true, early_ids, bad, [&] { wd.load_q_rows(p.q, off, live); });

  // merge the wave's token slots, then the wavefronts, as the split decode does
  float M[R];
  wd.slots_to_common_max(M);
  const int tslot = wd.tslot, lc = wd.lc;
  if constexpr (kLdsMerge) {
#pragma unroll
    for (int g = 0; g < R; ++g) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_part[w][tslot][g][wd.dim_of(j, e)] = wd.acc[g][j * EPL + e];
      }
      if (lc == 0) s_lp[w][tslot][g] = wd.l[g];
    }
  } else {
    wd.sum_slots();
    if (lane < LPT) {
#pragma unroll
      for (int g = 0; g < R; ++g) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) s_part[w][0][g][wd.dim_of(j, e)] = wd.acc[g][j * EPL + e];
        }
        if (lc == 0) s_lp[w][0][g] = wd.l[g];
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < R; ++g) s_m[w][g] = M[g];
    s_bad[w] = bad ? 1 : 0;
  }
  __syncthreads();

  int bad_or = 0;   // no short-circuit: the flags' reads go out together
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) bad_or |= s_bad[ww];
  const bool any_bad = bad_or != 0;

  for (int idx = threadIdx.x; idx < R * D; idx += NW * kWave) {
    const int g = idx / D;
    const int d = idx % D;
    const int r = g / GQ;
    if (r >= L) continue;
    // no branch on the maxima (as in the decode's merge): weight 0 for a
    // wavefront with no finite score
    float Mx = neg_inf();
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) Mx = fmaxf(Mx, s_m[ww][g]);
    float Ls = 0.f, O = 0.f;
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
      Ls += ls * wt;
      O += os * wt;
    }
    float o, lse;
    if (any_bad) {
      o = qnan();
      lse = qnan();
    } else {
      o = O * norm_inv(Ls);
      lse = norm_lse2(Mx, Ls);
    }
    const size_t row = static_cast<size_t>(q0 + r) * Hq + kh * GQ + g % GQ;
    p.o[row * D + d] = o;
    if (d == 0 && p.lse != nullptr) p.lse[row] = lse;
  }
}

template <int KV, int D, int GQ>
hipError_t launch_rows_g(const DecodeParams& p, hipStream_t st) {
  const int items = p.batch * p.num_kv_heads;
  const int grid = (items + kXcds - 1) / kXcds * kXcds;
  const int rows = p.max_q_len * GQ;   // query rows sharing each K/V tile
  if constexpr (GQ <= 2) {
    if (rows <= 2) {
      hipLaunchKernelGGL((decode_rows_kernel<KV, D, GQ, 2, 4>), dim3(grid), dim3(4 * kWave), 0, st, p);
      return hipGetLastError();
    }
  }
  if constexpr (GQ <= 4) {
    if (rows <= 4) {
      hipLaunchKernelGGL((decode_rows_kernel<KV, D, GQ, 4, 4>), dim3(grid), dim3(4 * kWave), 0, st, p);
      return hipGetLastError();
    }
  }
  if (rows > 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_rows_kernel<KV, D, GQ, 8, 4>), dim3(grid), dim3(4 * kWave), 0, st, p);
  return hipGetLastError();
}

template <int KV, int D>
hipError_t launch_rows_d(const DecodeParams& p, int group, hipStream_t st) {
  switch (group) {
    case 1: return launch_rows_g<KV, D, 1>(p, st);
    case 2: return launch_rows_g<KV, D, 2>(p, st);
    case 4: return launch_rows_g<KV, D, 4>(p, st);
    case 8: return launch_rows_g<KV, D, 8>(p, st);
    default: return hipErrorInvalidValue;
  }
}

template <int KV>
hipError_t launch_rows_kv(const DecodeParams& p, int head_dim, int group, hipStream_t st) {
  if (head_dim == 128) return launch_rows_d<KV, 128>(p, group, st);
  if (head_dim == 64) return launch_rows_d<KV, 64>(p, group, st);
  return hipErrorInvalidValue;
}

__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ int wave_incl_scan_i32(int x, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// Number of 16-token blocks of a context length, 0 for lengths the table
// cannot hold (those sequences are written by the empty-sequence pass).
__device__ __forceinline__ int blocks_of(int n, int max_blocks) {
  return (n > 0 && static_cast<int64_t>(n) <= static_cast<int64_t>(max_blocks) * kBlock) ? (n + kBlock - 1) / kBlock
                                                                                        : 0;
}

// Balanced single-launch decode (see the file comment). Four wavefronts per
// workgroup, each an independent worker; PD blocks of K/V in flight.
template <int KV, int QT, int D, int G, int PD>
__global__ __launch_bounds__(256) void decode_balanced_kernel(DecodeParams p) {
  using WD = WaveDecoder<KV, QT, D, G>;
  using Tile = typename WD::Tile;
  constexpr int LPT = WD::LPT, CPL = WD::CPL, EPL = WD::EPL;
  constexpr int kPart = G * (D + 1);   // floats of one partial: o[G][D] then lse[G]

  WD wd;
  wd.init_lane();
  const int lane = wd.lane;
  const int nw_grid = gridDim.x * 4;
  const int gw = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Hkv = p.num_kv_heads;
  const int Hq = p.num_q_heads;

  // ---- total tiles of the batch ----
  // the context lengths are read kRound * 64 at a time, every load of a
  // round issued before any is used (one round trip per 256 sequences)
  constexpr int kRound = 4;
  int64_t T = 0;
  for (int c0 = 0; c0 < p.batch; c0 += kRound * kWave) {
    int len[kRound];
#pragma unroll
    for (int u = 0; u < kRound; ++u) {
      const int bb = c0 + u * kWave + lane;
      len[u] = bb < p.batch ? p.ctx[bb] : 0;
    }
#pragma unroll
    for (int u = 0; u < kRound; ++u) T += wave_sum_i32(blocks_of(len[u], p.max_blocks));
  }
  T = uniform64(T) * Hkv;   // the same on every lane: scalar registers

  // ---- sequences without tiles: n == 0 -> (0, -inf); bad n -> NaN ----
  for (int bb = gw; bb < p.batch; bb += nw_grid) {
    const int n = p.ctx[bb];
    if (blocks_of(n, p.max_blocks) > 0) continue;
    const bool empty = (n == 0);
    float* out = p.o + static_cast<size_t>(bb) * Hq * D;
    for (int idx = lane; idx < Hq * D; idx += kWave) out[idx] = empty ? 0.f : qnan();
    if (p.lse != nullptr)
      for (int h = lane; h < Hq; h += kWave) p.lse[static_cast<size_t>(bb) * Hq + h] = empty ? neg_inf() : qnan();
  }
  if (T == 0) return;
  // tiles are dealt over min(wavefronts, T) workers, so that every worker
  // owns at least one tile and the workers that touch a segment are exactly
  // the consecutive ones between its first and its last tile's owner
  const int nw = static_cast<int>(T < nw_grid ? T : nw_grid);
  if (gw >= nw) return;
  const int64_t r0 = static_cast<int64_t>(gw) * T / nw;
  const int64_t r1 = static_cast<int64_t>(gw + 1) * T / nw;
  if (r0 >= r1) return;
  auto wave_of = [&](int64_t t) -> int { return static_cast<int>(((t + 1) * nw - 1) / T); };

  // ---- locate tile r0: sequence b, kv head kh, block blk ----
  int b = 0;
  int64_t base = 0;   // flat index of tile (b, kh = 0, blk = 0)
  bool found = false;
  for (int c0 = 0; c0 < p.batch && !found; c0 += kRound * kWave) {
    int len[kRound];
#pragma unroll
    for (int u = 0; u < kRound; ++u) {
      const int bb = c0 + u * kWave + lane;
      len[u] = bb < p.batch ? p.ctx[bb] : 0;
    }
#pragma unroll
    for (int u = 0; u < kRound; ++u) {
      if (!found) {
        const int tiles = Hkv * blocks_of(len[u], p.max_blocks);   // 0 past the batch
        const int incl = wave_incl_scan_i32(tiles, lane);
        const int total = __shfl(incl, kWave - 1);
        if (base + total > r0) {
          const uint64_t hit = __ballot(base + incl > r0);
          const int first = __builtin_ctzll(hit);
          b = c0 + u * kWave + first;
          base += __shfl(incl, first) - __shfl(tiles, first);
          found = true;
        } else {
          base += total;
        }
      }
    }
  }
  // the cursors are the same on every lane: keep them in scalar registers,
  // so the tile addresses built from them (buffer descriptors) are uniform
  b = __builtin_amdgcn_readfirstlane(b);
  base = uniform64(base);
  int n = __builtin_amdgcn_readfirstlane(p.ctx[b]);
  int nb = blocks_of(n, p.max_blocks);
  if (nb == 0) return;   // cannot happen for r0 < T; keeps the divisions below safe
  int kh = static_cast<int>((r0 - base) / nb);
  int blk = static_cast<int>((r0 - base) % nb);

  // the load cursor runs PD tiles ahead of the processing cursor
  int lb = b, lkh = kh, lblk = blk, lnb = nb, ln = n;
  int64_t lbase = base;
  auto advance = [&](int& cb, int& ckh, int& cblk, int& cnb, int64_t& cbase, int& cn) {
    if (++cblk < cnb) return;
    cblk = 0;
    if (++ckh < Hkv) return;
    ckh = 0;
    cbase += static_cast<int64_t>(Hkv) * cnb;
    do {
      ++cb;
      cn = cb < p.batch ? __builtin_amdgcn_readfirstlane(p.ctx[cb]) : kBlock;
      cnb = blocks_of(cn, p.max_blocks);
    } while (cnb == 0);
  };

  // block ids of the load cursor's sequence, 64 per fetch (lane j -> block c*64+j)
  int id_b = -1, id_chunk = -1, ids = 0;
  bool seg_bad = false;   // an id outside the pool: the current segment comes out NaN
  auto block_id = [&](int cb, int cblk) -> int {
    if (cb != id_b || (cblk >> 6) != id_chunk) {
      id_b = cb;
      id_chunk = cblk >> 6;
      const int j = (id_chunk << 6) + lane;
      int v = 0;
      if (j < max(1, blocks_of(p.ctx[cb], p.max_blocks))) v = p.tables[static_cast<size_t>(cb) * p.max_blocks + j];
      ids = v;
    }
    const int id = readlane(ids, cblk & 63);
    return id;
  };

  Tile ring[PD + 1];
  int ring_bad = 0;   // bit k: the id of ring[k] was outside the pool
  int64_t lpos = r0;
  auto issue = [&](int slot) {
    const int id = block_id(lb, lblk);
    const bool ok = static_cast<unsigned>(id) < static_cast<unsigned>(p.num_blocks);
    ring_bad = ok ? (ring_bad & ~(1 << slot)) : (ring_bad | (1 << slot));
    const int rows = min(kBlock, ln - lblk * kBlock);
    wd.load_tile(p, ok ? id : 0, lkh, rows, ring[slot]);
    advance(lb, lkh, lblk, lnb, lbase, ln);
    ++lpos;
  };

  wd.load_q(p.q, Hq, b, kh * G);
  wd.reset();
#pragma unroll
  for (int k = 0; k < PD; ++k)
    if (r0 + k < r1) issue(k);

  auto finish_segment = [&](int sb, int skh, int snb, int64_t sbase, int sn) {
    float M[G];
    wd.slots_to_common_max(M);
    wd.sum_slots();
    const bool sbad = wave_any(seg_bad);
    const int64_t seg_lo = sbase + static_cast<int64_t>(skh) * snb;
    const int64_t seg_hi = seg_lo + snb;
    const int h0 = skh * G;
    if (seg_lo >= r0 && seg_hi <= r1) {
      // the whole segment is this wavefront's: write the result
      if (lane < LPT) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float L = wd.l[g];
          const float inv = norm_inv(L);
          float* out = p.o + (static_cast<size_t>(sb) * Hq + h0 + g) * D;
#pragma unroll
          for (int j = 0; j < CPL; ++j) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) out[wd.dim_of(j, e)] = sbad ? qnan() : wd.acc[g][j * EPL + e] * inv;
          }
          if (lane == 0 && p.lse != nullptr)
            p.lse[static_cast<size_t>(sb) * Hq + h0 + g] =
                sbad ? qnan() : norm_lse2(M[g], L);
        }
      }
    } else {
      // A range boundary cuts the segment: leave a partial, the last one in
      // merges. The XCDs' L2s are not coherent with each other, and a
      // device-scope fence would write back / invalidate a whole L2; instead
      // the partials are written and read with agent-coherent (sc1) accesses,
      // and the counter is a device atomic, so only the exchanged bytes go
      // to the coherent level.
      const int slot = (seg_lo <= r0) ? 0 : 1;   // this wavefront's first segment, or its last
      float* part = p.part + (static_cast<size_t>(gw) * 2 + slot) * kPart;
      if (lane < LPT) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float L = wd.l[g];
          const float inv = norm_inv(L);
#pragma unroll
          for (int j = 0; j < CPL; ++j) {
#pragma unroll
            for (int e = 0; e < EPL; ++e)
              __hip_atomic_store(part + g * D + wd.dim_of(j, e), sbad ? qnan() : wd.acc[g][j * EPL + e] * inv,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          if (lane == 0)
            __hip_atomic_store(part + G * D + g, sbad ? qnan() : norm_lse2(M[g], L),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      // The arrival may be counted only once the partial's stores have
      // completed: the last arrival, in any workgroup on any XCD, reads the
      // partial as soon as it sees the count. This ordering is built from the
      // hardware's rules rather than from a release/acquire pair:
      //  - the partial stores are agent-scope atomic stores, which gfx950
      //    writes through to the device-coherent level (sc1), and a vector
      //    store is counted in vmcnt until that level has acknowledged it;
      //  - s_waitcnt vmcnt(0) therefore returns only once every partial word
      //    is visible device-wide, and the arrival atomic is issued after it;
      //  - the merging wavefront reads the partials with agent-scope atomic
      //    loads (sc1), which bypass any stale copy in its own XCD's L2.
      // The empty asm statements with a memory clobber keep the compiler from
      // moving any memory access across the wait. An agent-scope release on
      // the arrival and an agent-scope acquire before the merge express the
      // same ordering in HIP's memory model, but they write back and
      // invalidate the whole L2 of the XCD: measured on MI355X, the ragged
      // B=256 batch took 401 us against 291 us, and B=128 114 against 42 us.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0);
      asm volatile("" ::: "memory");
      int old = 0;
      int32_t* cnt = p.counters + static_cast<size_t>(sb) * Hkv + skh;
      if (lane == 0) old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      old = __shfl(old, 0);
      const int w_lo = wave_of(seg_lo);
      const int w_hi = wave_of(seg_hi - 1);
      if (old == w_hi - w_lo) {
        // compiler-level acquire: no load of the merge moves above the count
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        asm volatile("" ::: "memory");
        // Merge the C contributors' partials, lane-parallel: every round of
        // coherent loads is issued before any of it is used.
        const int C = w_hi - w_lo + 1;
        const int64_t start_lo = static_cast<int64_t>(w_lo) * T / nw;
        auto part_of = [&](int c) -> const float* {
          const int sl = (c == 0 && seg_lo > start_lo) ? 1 : 0;
          return p.part + (static_cast<size_t>(w_lo + c) * 2 + sl) * kPart;
        };
        auto ld = [](const float* a) { return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
        constexpr int kPerPass = kWave / G;                // contributors whose lse one pass loads
        constexpr int kElems = G * D / kWave;              // output elements per lane: idx = lane + 64 k
        constexpr int kChunk = 8;                          // contributors whose rows one round loads
        const int mg = lane % G;
        // 1. reference max of each head over the contributors
        float mx = neg_inf();
        bool nan = false;
        for (int c0 = 0; c0 < C; c0 += kPerPass) {
          const int c = c0 + lane / G;
          const float x = c < C ? ld(part_of(c) + G * D + mg) : neg_inf();
          nan = nan || (x != x);
          mx = fmaxf(mx, x);
        }
#pragma unroll
        for (int msk = G; msk < kWave; msk <<= 1) mx = fmaxf(mx, __shfl_xor(mx, msk));   // lane holds max of head lane % G
        nan = wave_any(nan);
        // 2. weights, denominators and weighted rows, kChunk contributors per round
        float Lh = 0.f;                     // denominator of head lane % G (summed over lanes below)
        float O[kElems];
#pragma unroll
        for (int k = 0; k < kElems; ++k) O[k] = 0.f;
        for (int c0 = 0; c0 < C; c0 += kChunk) {
          const int cw = c0 + lane / G;      // lanes 0 .. kChunk*G-1: contributor c0 + lane/G, head lane%G
          float wt = 0.f;
          if (lane < kChunk * G && cw < C && mx != neg_inf()) wt = __builtin_amdgcn_exp2f((ld(part_of(cw) + G * D + mg) - mx) * kLog2e);
          Lh += wt;
          float rows[kChunk][kElems];
#pragma unroll
          for (int cc = 0; cc < kChunk; ++cc) {
#pragma unroll
            for (int k = 0; k < kElems; ++k) rows[cc][k] = (c0 + cc < C) ? ld(part_of(c0 + cc) + lane + kWave * k) : 0.f;
          }
#pragma unroll
          for (int cc = 0; cc < kChunk; ++cc) {
#pragma unroll
            for (int k = 0; k < kElems; ++k) {
              const int gk = (lane + kWave * k) / D;
              O[k] = fmaf(__shfl(wt, cc * G + gk), rows[cc][k], O[k]);
            }
          }
        }
        // denominators: lanes with the same lane % G hold parts of the same head's sum
#pragma unroll
        for (int msk = G; msk < kWave; msk <<= 1) Lh += __shfl_xor(Lh, msk);
#pragma unroll
        for (int k = 0; k < kElems; ++k) {
          const int idx = lane + kWave * k;
          const int gk = idx / D;
          const float L = __shfl(Lh, gk);
          const float M = __shfl(mx, gk);
          const float o = nan ? qnan() : (L > 0.f ? O[k] / L : (L == 0.f ? 0.f : qnan()));
          p.o[(static_cast<size_t>(sb) * Hq + h0) * D + idx] = o;
          if (idx % D == 0 && p.lse != nullptr)
            p.lse[static_cast<size_t>(sb) * Hq + h0 + gk] = nan ? qnan() : (L > 0.f ? M + logf(L) : (L == 0.f ? neg_inf() : qnan()));
        }
        if (lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // ready for the next call
      }
    }
    wd.reset();
    seg_bad = false;
    (void)sn;
  };

  int64_t pos = r0;
  while (pos < r1) {
#pragma unroll
    for (int k = 0; k <= PD; ++k) {
      if (pos < r1) {
        if (lpos < r1) issue((k + PD) % (PD + 1));
        seg_bad = seg_bad || ((ring_bad >> k) & 1);
        wd.process(ring[k], p.scale_log2);
        ++pos;
        // leaving the segment (or the range): finish it
        const bool last_of_seg = (blk + 1 == nb);
        if (last_of_seg || pos == r1) {
          finish_segment(b, kh, nb, base, n);
          if (pos < r1) {
            advance(b, kh, blk, nb, base, n);
            wd.load_q(p.q, Hq, b, kh * G);
          }
        } else {
          ++blk;
        }
      }
    }
  }
}

// Host-side dispatch over the compile-time shape parameters of one KV type.
template <int KV, int QT, int D, int G, int NW, int PD>
hipError_t launch_partial_t(const DecodeParams& p, hipStream_t st) {
  const int items = p.batch * (p.direct ? 1 : p.max_ns) * p.num_kv_heads;
  const int grid = (items + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((decode_partial_kernel<KV, QT, D, G, NW, PD>), dim3(grid), dim3(NW * kWave), 0, st, p);
  return hipGetLastError();
}

template <int KV, int QT, int D, int G>
hipError_t launch_balanced_t(const DecodeParams& p, int workgroups, hipStream_t st) {
  hipLaunchKernelGGL((decode_balanced_kernel<KV, QT, D, G, 2>), dim3(workgroups), dim3(256), 0, st, p);
  return hipGetLastError();
}

// waves: wavefronts per workgroup. Each wavefront keeps one block of K/V in
// flight while it reduces the previous one, or two over a bf16 cache whose
// sequences are cut into kDeepRingSplits or more splits. Measured on MI355X
// (16/8 heads, head_dim 128), per step with one block ahead against two: the
// 32-sequence bf16 step of 128..384 tokens (one split each) 10.07 against
// 10.50 us, the mixed step's int8 rows (1024-token splits, up to 4 per
// sequence) 106.9 against 113.4 us, and 8 x 32k bf16 tokens in 64 splits
// 170.7 against 168.2 us. While every wavefront of the chip streams, HBM is
// oversubscribed and a deeper ring only lengthens the queues, except where
// each wavefront streams many blocks of a long context, which many splits
// per sequence mark (the table width does not: a wide table may hold short
// sequences). An 8-bit cache's blocks carry more VALU work per byte, and its
// wavefronts lose with the deeper ring even then.
constexpr int kDeepRingSplits = 8;

template <int KV, int QT, int D, int G>
hipError_t launch_partial_w(const DecodeParams& p, int waves, hipStream_t st) {
  if (waves < 0) return launch_balanced_t<KV, QT, D, G>(p, -waves, st);   // balanced: -workgroups
  switch (waves) {
    case 2: return launch_partial_t<KV, QT, D, G, 2, 1>(p, st);
    case 4:
      if constexpr (KV == PKV_BF16) {
        if (!p.direct && p.max_ns >= kDeepRingSplits) return launch_partial_t<KV, QT, D, G, 4, 2>(p, st);
      }
      return launch_partial_t<KV, QT, D, G, 4, 1>(p, st);
    case 8: return launch_partial_t<KV, QT, D, G, 8, 1>(p, st);
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
