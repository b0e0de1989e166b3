// Chunked prefill for gfx950: causal query chunks over a paged KV prefix,
// with MFMA for both contractions (bf16; the PV product in fp16 over int8 and
// fp8 caches).
//
// What is computed (course README "Build an LLM Inference Engine From
// Scratch", curriculum S11 chunked prefill and S12 FlashAttention): the L new
// rows of a sequence whose cache now holds n tokens (the chunk's own K/V
// included) sit at positions n - L + r and attend keys t <= n - L + r;
// softmax(scale * q . k) weighted values, online over 64-token KV tiles.
//
// Work mapping. A workgroup of 8 wavefronts owns one (sequence, kv head,
// query tile): 128 query rows = (128 / G) positions x the G query heads of the
// GQA group, which all read the same K/V. Wavefronts w and w + 4 own the same
// 32 rows and split every KV tile: w takes its first 32 tokens, w + 4 the
// other 32, each with its own online-softmax state; the two states merge once,
// at the end, through LDS. Two wavefronts share each SIMD, so one's softmax
// work issues while the other's MFMAs run. With v_mfma_f32_32x32x16_bf16
// (lane l of a 32x32 result holds column l % 32 and rows 8(v/4) + 4(l/32) +
// v%4 of register v), per 32-token half tile:
//   S^T = K Q^T  (A = K rows from LDS, B = the wavefront's q rows, kept in
//                 registers): every lane holds scores of ONE query row, so the
//                 row max, the causal mask and the softmax state are lane-local
//                 (the two lanes l, l^32 of a row hold its two token quarters);
//   O^T = V^T P^T (A = V^T from LDS, B = P^T straight from the S^T registers):
//                 the output accumulator again holds one query row per lane,
//                 so the online rescale is lane-local. A bf16 cache runs it
//                 twice, on a bf16 high part of P and on its bf16 residual:
//                 one bf16 rounding of a weight (2^-9) is too coarse for rows
//                 that see few keys, the pair keeps ~2^-17. An int8 or fp8
//                 cache stages V as fp16 instead (its codes are exact there)
//                 and runs it once on P rounded to fp16 (2^-12), with the V
//                 scale folded into P.
// K rows are fed to the first product in an order that swaps bits 2 and 3 of
// the row index; with it, the token order of the S^T registers is exactly the
// k order the second product needs, so P never moves between lanes.
//
// Pipeline. K is staged row-major and V transposed (the token index must be
// the MFMA k dimension), each in a ring of three LDS stages, XOR-swizzled
// against bank conflicts. Iteration j runs two phases, each written as slots of MFMAs
// and a share of the VALU / LDS work, fenced so the interleaving survives:
//   1. the softmax of tile j's scores  ||  S^T of tile j + 1 (MFMA);
//   2. O^T += V_j^T P_j^T (MFMA)       ||  tile j + 2: registers -> LDS.
// A tile's global loads are issued at the end of phase 2, one iteration
// before that tile is staged, into one register set (issuing them earlier in
// the phase measured slower). They are buffer loads whose range is the valid
// part of each block: rows past the context and blocks outside the table come
// back as zeros with no branch, so every tile issues the same loads. An int8
// or fp8 cache is dequantized on its way to LDS (int8 codes and E4M3 values
// are exact in bf16 and in fp16; K goes to bf16 beside the bf16 q rows, V to
// fp16): the K scale multiplies the score column, the V scale the weight.
#include <type_traits>
#include <utility>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

constexpr int kRows = 128;         // query rows per workgroup
constexpr int kTile = 64;          // tokens per KV tile
constexpr int kThreads = 512;
constexpr int kXcdsC = 8;
constexpr int kStages = 3;
constexpr int kIdsCached = 4096;           // block ids kept in LDS (65536 tokens)
constexpr int kRsrcWord3 = 0x00020000;     // buffer descriptor word 3 (gfx9 family): raw dwords

// Row order of the S^T product: bits 2 and 3 of the row index swapped.
__device__ __forceinline__ int sigma(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
// K row t (D dims, 2 D bytes), 16-byte unit u (8 dims). The XOR key sigma(t)
// makes the lanes of one operand read (rows sigma(0..15), one unit) hit
// different units.
template <int D>
__device__ __forceinline__ int k_off(int t, int u) { return t * (2 * D) + ((u ^ (sigma(t) & (D / 8 - 1))) << 4); }
// V^T row d (one dim: 64 tokens = 8 units of 8 tokens).
__device__ __forceinline__ int vt_sw(int d) { return (d ^ (d >> 3) ^ (d >> 6)) & 7; }
__device__ __forceinline__ int vt_off(int d, int u) { return d * 128 + ((u ^ vt_sw(d)) << 4); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// two floats -> fp16 pair, each rounded to nearest even (v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f16x2_t v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Byte B of two int8 code words -> fp16 pair (low half from w0), exact: the
// code c, offset to u = c + 128 by flipping its sign bit, becomes the low
// byte of the fp16 number 1024 + u (the numbers 1024 .. 2047 are spaced by
// 1), and subtracting 1152 leaves c.
template <int B>
__device__ __forceinline__ uint32_t i8pair_to_f16x2(uint32_t w0, uint32_t w1) {
  constexpr uint32_t sel = 0x0c000c00u | ((4u + B) << 16) | static_cast<uint32_t>(B);
  const uint32_t x = __builtin_amdgcn_perm(w1, w0, sel) ^ 0x64806480u;
  const f16x2_t v = __builtin_bit_cast(f16x2_t, x) - f16x2_t{static_cast<_Float16>(1152.0f), static_cast<_Float16>(1152.0f)};
  return __builtin_bit_cast(uint32_t, v);
}

// int8 code c (sign-extended) -> bfloat16 bits (exact: |c| <= 127).
__device__ __forceinline__ uint32_t i8pair_to_bf16x2(uint32_t w, int byte0) {
  const float a = i8_at(w, byte0), b = i8_at(w, byte0 + 1);
  return pack_bf16(a, b);
}

// Codes B0, B0 + 1 (B0 = 0 or 2) of a scaled 8-bit cache word -> two
// bfloat16: int8 integers, or OCP E4M3 values (gfx950's conversion decodes
// them exactly; at most 4 significant bits and exponents -9 .. 8, so the bf16
// packing is exact too).
template <int KV, int B0>
__device__ __forceinline__ uint32_t code_pair_to_bf16x2(uint32_t w) {
  static_assert(B0 == 0 || B0 == 2, "an aligned pair of bytes");
  if constexpr (KV == PKV_I8) {
    return i8pair_to_bf16x2(w, B0);
  } else {
    const f32x2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), B0 == 2);
    return pack_bf16(f.x, f.y);
  }
}

// Raw buffer over `bytes` bytes at `base`: loads at or past `bytes` return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes, kRsrcWord3);
}

typedef __attribute__((address_space(3))) char lds_char;

// LDS byte address of a shared-memory location
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_char*)p));
}
// A lane's LDS address, opaque to the compiler: accesses at it plus a
// compile-time stage offset (< 64 KiB) keep that offset in the instruction's
// immediate field, whatever the ring's own base, rather than adding it per
// lane or holding one more register per stage.
__device__ __forceinline__ uint32_t lane_address(uint32_t a) {
  asm volatile("" : "+v"(a));
  return a;
}
// max / sum of x over lanes l and l ^ 32, in every lane: gfx950's
// v_permlane32_swap exchanges the upper half of one register with the lower
// half of another, so with x in both each lane sees {x[l], x[l ^ 32]} (a VALU
// exchange, not an LDS round trip)
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint4 lds_read16(uint32_t a, int off) {
  const u32x4v_t x = *reinterpret_cast<const __attribute__((address_space(3))) u32x4v_t*>((const lds_char*)(uintptr_t)a + off);
  return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void lds_write16(uint32_t a, int off, uint4 x) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x4v_t*>((lds_char*)(uintptr_t)a + off) = u32x4v_t{x.x, x.y, x.z, x.w};
}
__device__ __forceinline__ void lds_write4(uint32_t a, int off, uint32_t x) {
  *reinterpret_cast<__attribute__((address_space(3))) uint32_t*>((lds_char*)(uintptr_t)a + off) = x;
}

// One tile's global loads for one thread, held in registers until they are
// stored to LDS. A thread stages part of its group's 32-token half of the
// tile: unit u = (thread % 256) % (D / 8) of K token tg + (2048 / D) i
// (chunk i, tg = (thread % 256) / (D / 8)), and of V tokens 2 tp, 2 tp + 1
// (tp = tg, for head_dim 64 only the first 128 threads).
struct Staged {
  uint4 k[2];      // K chunk i (head_dim 128: chunks 0, 1; 64: chunk 0), unit u (8-bit codes: 8 bytes)
  uint4 v[2];      // V: tokens 2 tp and 2 tp + 1 of the half, unit u
  float sc;        // 8-bit codes: the K (thread % 64 < 32) or V scale of token thread % 32 of the half
  bool sc_ok;      // that token exists
};

// kIdsInLds: every block id of the table fits the LDS copy (max_blocks <=
// kIdsCached), so the tile loop reads ids from LDS only. A global load of an
// id inside the loop would make the compiler wait for it with vmcnt(0), that
// is, for every tile load in flight as well (vector memory counts retire in
// order), and the loads issued for later tiles would lose their lead.
template <int KV, int G, bool kIdsInLds, int D>
__global__ __launch_bounds__(kThreads, 1) void chunked_kernel(ChunkedParams p) {
  constexpr int kD = D;                      // head_dim
  constexpr int kKS = D / 16;                // k-steps of the S^T product
  constexpr int kDB = D / 32;                // 32-dim blocks of O^T
  constexpr int kUnits = D / 8;              // 16-byte units (8 dims) of a staged row
  constexpr int kKC = D / 64;                // K chunks a thread stages per half tile
  constexpr int kKBytes = kTile * D * 2;     // a stage: K row-major [token][dim] or V^T [dim][token], swizzled
  constexpr int kMergeFloats = D / 2 + 2;    // per lane of a merging wavefront: o[D / 2], m, l
  constexpr int P = kRows / G;               // positions per query tile
  constexpr bool kScaled = is_scaled_kv(KV);   // int8 / fp8 codes + a scale per row
  constexpr float kSlack = 8.0f;
  // 8-bit caches: the fp16 weights are exp2(score - m - kP16Shift - lvs) x
  // V scale, where 2^lvs is a power of two at least twice every V scale the
  // workgroup reads (found once, before the loop). So they stay below
  // 2^(kSlack - kP16Shift - 1) = 8 whatever the magnitude of V, and the
  // weights that matter stay clear of fp16's subnormal range.
  constexpr float kP16Shift = 4.0f;
  constexpr int kRowBytes = kScaled ? kD : 2 * kD;   // bytes of one cached K or V row
  constexpr int kUnit = kRowBytes / kUnits;      // bytes of 8 dims of a cached row
  // stages 0 .. 2: K (row-major); stages 3 .. 5: V^T of the same tiles
  __shared__ __attribute__((aligned(16))) char s_kv[2 * kStages][kKBytes];
  __shared__ __attribute__((aligned(16))) float s_sc[kStages][2 * kTile];   // 8-bit codes: K scale x softmax scale, V scale
  __shared__ float s_vmax[kThreads / 64];   // 8-bit codes: largest V scale each wavefront saw
  __shared__ __attribute__((aligned(16))) int s_ids[kIdsCached];
  static_assert(2 * kStages * kKBytes >= 4 * kMergeFloats * 64 * 4, "merge area");

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
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int rb = wu & 3;                            // row block of this wavefront
  const int th = wu >> 2;                           // which 32-token half of each tile
  const int h = lane >> 5;                          // which token quarter of that half a lane holds
  const int rrow = 32 * rb + (lane & 31);           // row of the 128-row tile
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
  bf16x8_t qb[kKS];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                           (static_cast<size_t>(q0 + (row_live ? pi : 0)) * p.num_q_heads + hq) * kD;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
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
  const int nblk_need = min(nblk_seq, ntiles * (kTile / kBlock));   // the blocks of tiles < ntiles
  const int32_t* trow = p.tables + static_cast<size_t>(seq) * p.max_blocks;
  int bad = 0;

  // the block ids this tile range needs, read once into LDS (ids past what
  // LDS holds are read from the table when used)
  {
    // all of a thread's loads first, then the stores, so the loads overlap
    const int nfill = min(nblk_need, kIdsCached);
    int idv[kIdsCached / kThreads];
#pragma unroll
    for (int u = 0; u < kIdsCached / kThreads; ++u) {
      const int j = tid + u * kThreads;
      idv[u] = j < nfill ? trow[j] : 0;
    }
#pragma unroll
    for (int u = 0; u < kIdsCached / kThreads; ++u) {
      const int j = tid + u * kThreads;
      if (j < nfill) s_ids[j] = idv[u];
    }
  }
  __syncthreads();

  // Each group of 4 wavefronts (th = 0: wavefronts 0-3, th = 1: 4-7) loads
  // and stages only the 32-token half of every tile it computes on, so the
  // two groups share no staged data. Group-local thread tl: tg = tl / (D / 8),
  // u = tl % (D / 8); the V pair index tp = tg stages V only below 16.
  const int tl = tid & 255;
  const int un = tl % kUnits;
  const int tg = tl / kUnits;
  const int wl = wu & 3;                            // wavefront within its group
  // head_dim 64: K chunk 0 of wavefronts 2, 3 is in the group's second block;
  // V is staged by wavefronts 0 (block 0) and 1 (block 1) only
  const bool has_v = kD == 128 || wl < 2;
  const int vblk = kD == 128 ? (wl >> 1) : (wl & 1);
  const char* kpool = static_cast<const char*>(p.k);
  const char* vpool = static_cast<const char*>(p.v);

  // Where tile `tile`'s loads come from: buffer descriptors over the valid
  // rows of this wavefront's blocks (none for blocks the range does not
  // need) and this thread's scale. K chunk i comes from block 2 th + i
  // (head_dim 64: block 2 th + wl / 2), row tg % 16; V from block
  // 2 th + vblk. Any tile index is safe.
  struct TileSrc {
    __amdgpu_buffer_rsrc_t k[2];
    __amdgpu_buffer_rsrc_t v;
    const float* sc;
    bool sc_ok;
  };
  const float* sc_pool = (tl & 32) ? p.v_scale : p.k_scale;
  const size_t head_off = static_cast<size_t>(kh) * kBlock * kRowBytes;
  const size_t blk_stride = static_cast<size_t>(p.num_kv_heads) * kBlock * kRowBytes;
  // block blk of the sequence: its id (0 if the range does not need it, or
  // it is outside the pool, which poisons the output) and its valid rows
  auto block_src = [&](int blk, int& rows) -> int {
    int id = 0;
    rows = 0;
    if (blk < nblk_need) {
      id = (kIdsInLds || blk < kIdsCached) ? s_ids[blk] : trow[blk];
      id = __builtin_amdgcn_readfirstlane(id);
      if (static_cast<unsigned>(id) < static_cast<unsigned>(p.num_blocks)) {
        rows = min(kBlock, n - blk * kBlock);
      } else {
        bad = 1;
        id = 0;
      }
    }
    return id;
  };
  auto tile_src = [&](int tile, TileSrc& ts) {
    const int blk0 = tile * (kTile / kBlock) + 2 * th;   // this group's first block of the tile
    int rk0, rk1;
    const int id0 = block_src(blk0, rk0);
    const int id1 = block_src(blk0 + 1, rk1);
    if constexpr (kKC == 2) {
      ts.k[0] = rsrc(kpool + head_off + id0 * blk_stride, rk0 * kRowBytes);
      ts.k[1] = rsrc(kpool + head_off + id1 * blk_stride, rk1 * kRowBytes);
    } else {
      const bool k1 = (wl >> 1) != 0;
      ts.k[0] = rsrc(kpool + head_off + (k1 ? id1 : id0) * blk_stride, (k1 ? rk1 : rk0) * kRowBytes);
    }
    const bool v1 = vblk != 0;
    ts.v = rsrc(vpool + head_off + (v1 ? id1 : id0) * blk_stride, has_v ? (v1 ? rk1 : rk0) * kRowBytes : 0);
    if constexpr (kScaled) {
      // scale of token 32 th + (tl % 32): K for tl % 64 < 32, V otherwise
      const int t = tl & 31;
      const bool hi = t >= kBlock;
      ts.sc_ok = (t & 15) < (hi ? rk1 : rk0);
      ts.sc = sc_pool + (static_cast<size_t>(hi ? id1 : id0) * p.num_kv_heads + kh) * kBlock + (t & 15);
    }
  };
  // The loads themselves: the same 4 (+1 scale) loads for every tile, no branch.
  const int koff = (tg & 15) * kRowBytes + un * kUnit;             // K chunk i: row tg % 16 of its block
  const int voff = ((2 * tg) & 15) * kRowBytes + un * kUnit;       // V: rows 2 tp % 16, + 1
  auto gissue = [&](const TileSrc& ts, Staged& st) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (kScaled) {
        if (i < kKC) {
          const u32x2v_t c = __builtin_bit_cast(u32x2v_t, __builtin_amdgcn_raw_buffer_load_b64(ts.k[i], koff, 0, 0));
          st.k[i] = make_uint4(c.x, c.y, 0, 0);
        }
        const u32x2v_t d = __builtin_bit_cast(
            u32x2v_t, __builtin_amdgcn_raw_buffer_load_b64(ts.v, voff + i * kRowBytes, 0, 0));
        st.v[i] = make_uint4(d.x, d.y, 0, 0);
      } else {
        if (i < kKC) {
          const u32x4v_t c = __builtin_bit_cast(u32x4v_t, __builtin_amdgcn_raw_buffer_load_b128(ts.k[i], koff, 0, 0));
          st.k[i] = make_uint4(c.x, c.y, c.z, c.w);
        }
        const u32x4v_t d = __builtin_bit_cast(
            u32x4v_t, __builtin_amdgcn_raw_buffer_load_b128(ts.v, voff + i * kRowBytes, 0, 0));
        st.v[i] = make_uint4(d.x, d.y, d.z, d.w);
      }
    }
    if constexpr (kScaled) {
      st.sc = *ts.sc;
      st.sc_ok = ts.sc_ok;
    }
  };
  auto gload = [&](int tile, Staged& st) {
    TileSrc ts;
    tile_src(tile, ts);
    gissue(ts, st);
  };

  // LDS byte offsets of this thread's stores, the same for every stage
  const uint32_t k_lds = lds_address(&s_kv[0][0]), v_lds = lds_address(&s_kv[kStages][0]);
  // K chunk i: token 32 th + tg + 16 i, at + 32 D i bytes
  const uint32_t kw_a = lane_address(k_lds + k_off<kD>(32 * th + tg, un));
  // V^T: dims 8 u + e, tokens 32 th + 2 tp, + 1 (4 bytes in unit 4 th + tp / 4)
  uint32_t vw_a[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    vw_a[e] = lane_address(v_lds + vt_off(has_v ? 8 * un + e : 0, 4 * th + ((tg & 15) >> 2)) + ((tg & 3) << 2));

  // K chunk i of st -> bf16 (8-bit codes converted)
  auto k_bf16 = [&](const Staged& st, int i) -> uint4 {
    if constexpr (kScaled) {
      return make_uint4(code_pair_to_bf16x2<KV, 0>(st.k[i].x), code_pair_to_bf16x2<KV, 2>(st.k[i].x),
                        code_pair_to_bf16x2<KV, 0>(st.k[i].y), code_pair_to_bf16x2<KV, 2>(st.k[i].y));
    } else {
      return st.k[i];
    }
  };
  // the two V tokens of st as 16-bit words (bf16 for a bf16 cache, fp16 for
  // fp8 codes): vw[i][k] = dims 8 u + 2k, +1 of token 2 tg + i. int8 codes
  // need no step here: v_word converts them straight from st.
  auto v_prep = [&](const Staged& st, uint32_t (&vw)[2][4]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (KV == PKV_FP8) {
        // exact: E4M3 values are fp16 values
        const f32x2_t f0 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(st.v[i].x), false);
        const f32x2_t f1 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(st.v[i].x), true);
        const f32x2_t f2 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(st.v[i].y), false);
        const f32x2_t f3 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(st.v[i].y), true);
        vw[i][0] = pack_f16(f0.x, f0.y);
        vw[i][1] = pack_f16(f1.x, f1.y);
        vw[i][2] = pack_f16(f2.x, f2.y);
        vw[i][3] = pack_f16(f3.x, f3.y);
      } else if constexpr (KV == PKV_BF16) {
        vw[i][0] = st.v[i].x;
        vw[i][1] = st.v[i].y;
        vw[i][2] = st.v[i].z;
        vw[i][3] = st.v[i].w;
      }
    }
  };
  // dim 8 u + e of the two tokens as one word of the V^T stage (token 2 tg low)
  auto v_word = [&](const Staged& st, const uint32_t (&vw)[2][4], int e) -> uint32_t {
    if constexpr (KV == PKV_I8) {
      const uint32_t w0 = (e < 4) ? st.v[0].x : st.v[0].y;
      const uint32_t w1 = (e < 4) ? st.v[1].x : st.v[1].y;
      switch (e & 3) {
        case 0: return i8pair_to_f16x2<0>(w0, w1);
        case 1: return i8pair_to_f16x2<1>(w0, w1);
        case 2: return i8pair_to_f16x2<2>(w0, w1);
        default: return i8pair_to_f16x2<3>(w0, w1);
      }
    } else {
      return __builtin_amdgcn_perm(vw[1][e >> 1], vw[0][e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
    }
  };
  auto sc_store = [&](const Staged& st, int stage) {
    if constexpr (kScaled) {
      // the 4 wavefronts of a group store the same values to the same places
      const float sc = st.sc_ok ? st.sc : 0.f;
      s_sc[stage][((tl & 32) ? kTile : 0) + 32 * th + (tl & 31)] = (tl & 32) ? sc : sc * p.scale_log2;
    }
  };
  auto lstore = [&](const Staged& st, int stage) {
    const int so = stage * kKBytes;
#pragma unroll
    for (int i = 0; i < kKC; ++i) lds_write16(kw_a, so + 32 * kD * i, k_bf16(st, i));
    if (has_v) {
      uint32_t vw[2][4];
      v_prep(st, vw);
#pragma unroll
      for (int e = 0; e < 8; ++e) lds_write4(vw_a[e], so, v_word(st, vw, e));
    }
    sc_store(st, stage);
  };

  // LDS byte offsets of this lane's MFMA operand reads, the same for every stage
  const int ar = lane & 31;
  uint32_t kr_a[kKS];                               // K row 32 th + sigma(ar), unit 2 ks + h
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) kr_a[ks] = lane_address(k_lds + k_off<kD>(32 * th + sigma(ar), 2 * ks + h));
  uint32_t vr_a[kDB][2];                            // V^T row 32 db + ar, unit 2 (2 th + k2) + h
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) vr_a[db][k2] = lane_address(v_lds + vt_off(32 * db + ar, 2 * (2 * th + k2) + h));
  }

  // S^T of this wavefront's half of the tile in `stage`
  auto qk = [&](int stage, f32x16_t& s) {
    const int so = stage * kKBytes;
    s = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const uint4 a = lds_read16(kr_a[ks], so);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), qb[ks], s, 0, 0, 0);
    }
  };

  // ---- online softmax state of this lane's row, over this wavefront's tokens ----
  float m = neg_inf(), l = 0.f;
  float mu_off = 0.f;   // 8-bit caches: kP16Shift + lvs, set before the loop
  f32x16_t o[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) o[db] = f32x16_t{};
  f32x16_t sacc;   // S^T of the tile being softmaxed
  bf16x8_t phi[2], plo[2];   // P^T of that tile: bf16 high parts and residuals (8-bit caches: fp16 in phi)

  // scores: register v of the wavefront's half holds token
  // 32 th + 8 h + 16 (v / 8) + (v % 8) of the tile; chunk c = v / 4
  auto tok_of = [&](int v) { return 32 * th + 8 * h + 16 * (v >> 3) + (v & 7); };

  // Phase 1 of tile j: the softmax of its scores (sacc, scales in stage ss)
  // || S^T of tile j + 1 (K in stage sk), in 8 slots of one MFMA; then O is
  // rescaled if the reference max moved and sacc becomes tile j + 1's S^T.
  auto phase1 = [&](auto diag_tag, int j, int sk, int ss) {
    constexpr bool kDiag = decltype(diag_tag)::value;
    const int so = sk * kKBytes;
    const float* scs = s_sc[ss];
    const int tlim = pos - j * kTile;     // tile tokens past this one are masked
    uint4 ka[3];
    ka[0] = lds_read16(kr_a[0], so);
    ka[1] = lds_read16(kr_a[1], so);
    ka[2] = lds_read16(kr_a[2], so);
    float4 sc4;
    auto read_sc = [&](int t0) { sc4 = *reinterpret_cast<const float4*>(scs + t0); };
    if constexpr (kScaled) read_sc(tok_of(0));
    float sv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) sv[v] = sacc[v];
    f32x16_t sn = f32x16_t{};
    auto mfma1 = [&](int ks) {
      sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ka[ks % 3]), qb[ks], sn, 0, 0, 0);
      if (ks + 3 < kKS) ka[ks % 3] = lds_read16(kr_a[ks + 3], so);
    };
    // slots 0-3: scale, mask and max of scores 4 c .. 4 c + 3
    float cmax = neg_inf();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      mfma1(c);
      float kv[4];
      if constexpr (kScaled) {
        kv[0] = sc4.x; kv[1] = sc4.y; kv[2] = sc4.z; kv[3] = sc4.w;
        read_sc(c < 3 ? tok_of(4 * (c + 1)) : kTile + tok_of(0));   // next: K scales, then V scales of scores 0..3
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = 4 * c + e;
        float x = sv[v];
        if constexpr (kScaled) {
          // K scale x softmax scale, rounded here: the max below and the
          // exponent's argument must use the same value. (Contracted into the
          // later subtraction, the product would enter the exponent
          // unrounded, and the largest weight would miss its exact power of
          // two by a few ulps.)
#pragma clang fp contract(off)
          x *= kv[e];
        }
        if constexpr (kDiag) {
          if (tok_of(v) > tlim) x = neg_inf();
        }
        sv[v] = x;
        cmax = fmaxf(cmax, x);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // slots 4-7: exponentials of scores 4 c .. 4 c + 3 (the reference max first)
    float corr = 1.f, mu = 0.f, rsum = 0.f;
    uint32_t pw_hi[8], pw_lo[8];   // P^T words: registers 2 k, 2 k + 1
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (4 + c < kKS) mfma1(4 + c);
      if (c == 0) {
        float tmax = xor32_max(cmax);
        if constexpr (!kScaled) tmax *= p.scale_log2;   // the max commutes with a positive scale
        // move the reference max only when the tile exceeds it by more than
        // the slack: weights stay below 2^kSlack and O is rarely rescaled
        const bool need = tmax > m + kSlack;
        corr = need ? __builtin_amdgcn_exp2f(m - tmax) : 1.f;   // m = -inf -> 0
        l *= corr;
        m = need ? tmax : m;
        mu = (m == neg_inf()) ? 0.f : (kScaled ? m + mu_off : m);
      }
      float vv[4];
      if constexpr (kScaled) {
        vv[0] = sc4.x; vv[1] = sc4.y; vv[2] = sc4.z; vv[3] = sc4.w;
        if (c < 3) read_sc(kTile + tok_of(4 * (c + 1)));
      }
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const int v = 4 * c + e;
        float pw[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          if constexpr (kScaled) pw[k] = __builtin_amdgcn_exp2f(sv[v + k] - mu);
          else pw[k] = __builtin_amdgcn_exp2f(fmaf(sv[v + k], p.scale_log2, -mu));
          rsum += pw[k];
          if constexpr (kScaled) pw[k] *= vv[e + k];
        }
        if constexpr (kScaled) {
          pw_hi[v >> 1] = pack_f16(pw[0], pw[1]);
        } else {
          // high parts rounded to bf16, residuals exact in float32 then rounded
          const uint32_t hp = pack_bf16(pw[0], pw[1]);
          const uint32_t lp = pack_bf16(pw[0] - __uint_as_float(hp << 16), pw[1] - __uint_as_float(hp & 0xffff0000u));
          pw_hi[v >> 1] = hp;
          pw_lo[v >> 1] = lp;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    rsum = xor32_sum(rsum);
    l += rsum;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      phi[k2] = __builtin_bit_cast(bf16x8_t, make_uint4(pw_hi[4 * k2], pw_hi[4 * k2 + 1], pw_hi[4 * k2 + 2], pw_hi[4 * k2 + 3]));
      if constexpr (!kScaled) {
        plo[k2] = __builtin_bit_cast(bf16x8_t, make_uint4(pw_lo[4 * k2], pw_lo[4 * k2 + 1], pw_lo[4 * k2 + 2], pw_lo[4 * k2 + 3]));
      }
    }
    if (wave_any(corr != 1.f)) {
#pragma unroll
      for (int db = 0; db < kDB; ++db) o[db] *= corr;
    }
    sacc = sn;   // S^T of tile j + 1 (garbage past the last tile, unused)
  };

  // Phase 2 of tile j: O^T += V_j^T P_j^T over this wavefront's 32 tokens
  // (V in stage sv_stage) || this group's half of tile j + 2 from st to
  // stage st_stage, then tile j + 3's loads (from ns) into st; 8 slots of two
  // bf16 MFMAs (8-bit caches: one fp16 MFMA) on different accumulators.
  auto phase2 = [&](int sv_stage, int st_stage, Staged& st, const TileSrc& ns) {
    const int vo = sv_stage * kKBytes;   // V^T stage read
    const int wo = st_stage * kKBytes;   // stage written
    uint4 va[2][kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db) va[0][db] = lds_read16(vr_a[db][0], vo);
    uint32_t vw[2][4];
    // slot s: k-step k2 = s / 4. A bf16 cache: (s % 4) = high part of the
    // first / second half of the dims blocks, then the residual of the first /
    // second half. 8-bit caches: one fp16 MFMA on dims block s % 4 (head_dim
    // 64: on block (s % 4) / 2, in the even slots).
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const int k2 = sl >> 2, q = sl & 3;
      if (sl == 0) {
#pragma unroll
        for (int db = 0; db < kDB; ++db) va[1][db] = lds_read16(vr_a[db][1], vo);
      }
      if constexpr (kScaled) {
        constexpr int kEvery = 4 / kDB;
        if (sl % kEvery == 0) {
          const int db = q / kEvery;
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, va[k2][db]),
                                                         __builtin_bit_cast(f16x8_t, phi[k2]), o[db], 0, 0, 0);
        }
      } else {
        const bf16x8_t b = (q < 2) ? phi[k2] : plo[k2];
#pragma unroll
        for (int d2 = 0; d2 < kDB / 2; ++d2) {
          const int db = (kDB / 2) * (q & 1) + d2;
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va[k2][db]), b, o[db], 0, 0, 0);
        }
      }
      // staging of tile j + 2 (st -> LDS stage st_stage), then tile j + 3's loads
      if (sl < 2) {
        if (sl < kKC) lds_write16(kw_a, wo + 32 * kD * sl, k_bf16(st, sl));
      } else if (sl == 2) {
        if (has_v) v_prep(st, vw);
      } else if (sl < 7) {
        if (has_v) {
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            const int e = 2 * (sl - 3) + e2;
            lds_write4(vw_a[e], wo, v_word(st, vw, e));
          }
        }
      } else {
        sc_store(st, st_stage);
        gissue(ns, st);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- prologue: this group's halves of tiles 0 and 1 in LDS, tile 2 in
  // flight, S^T of tile 0; 8-bit caches: the largest V scale of keys
  // [0, kv_end), each thread scanning every 512th key ----
  Staged sa{};
  float vmax = 0.f;
  {
    Staged sb{};
    gload(0, sa);
    gload(1, sb);
    if constexpr (kScaled) {
      // in batches of 8 keys per thread whose loads are all issued before
      // any is used
      constexpr int kScan = 8;
      for (int t0 = tid; t0 < kv_end; t0 += kScan * kThreads) {
        int id[kScan];
#pragma unroll
        for (int u = 0; u < kScan; ++u) {
          // ids from LDS when they all fit there, else straight from the
          // (cache-hot) table, unconditionally: the block of
          // min(t, kv_end - 1) is always one the range needs
          const int t = t0 + u * kThreads;
          const int bi = min(t, kv_end - 1) / kBlock;
          const int raw = kIdsInLds ? s_ids[bi] : trow[bi];
          id[u] = t < kv_end ? raw : -1;
        }
        float sv[kScan];
#pragma unroll
        for (int u = 0; u < kScan; ++u) {
          const int t = t0 + u * kThreads;
          sv[u] = static_cast<unsigned>(id[u]) < static_cast<unsigned>(p.num_blocks)
                      ? p.v_scale[(static_cast<size_t>(id[u]) * p.num_kv_heads + kh) * kBlock + t % kBlock]
                      : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kScan; ++u) vmax = fmaxf(vmax, sv[u]);
      }
    }
    lstore(sa, 0);
    lstore(sb, 1);
  }
  gload(2, sa);
  if constexpr (kScaled) {
    vmax = coset_reduce<1>(vmax, OpMax{});   // over the wavefront, by VALU lane exchanges; NaN ignored
    if (lane == 0) s_vmax[w] = vmax;
  }
  __syncthreads();
  // 8-bit caches: 2^lvs >= twice every V scale read (lvs = 0 if all are 0)
  if constexpr (kScaled) {
    float vm = s_vmax[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) vm = fmaxf(vm, s_vmax[i]);
    mu_off = kP16Shift + (vm > 0.f ? static_cast<float>(__builtin_amdgcn_frexp_expf(vm) + 1) : 0.f);
  }
  qk(0, sacc);

  // ---- main loop. Every wavefront runs phase 1 and phase 2 of each tile
  // with a barrier after each; group 1 passes one extra barrier before the
  // loop and group 0 one after it, so group 1 runs exactly one phase behind:
  // on each SIMD one group's softmax issues beside the other group's PV
  // MFMAs. The groups share no staged data; within a group the barriers
  // order the staging of a tile before its use and the reuse of a stage
  // after its last read. ----
  // Tile j lives in stage j % 3. The loop over the tiles before the diagonal
  // is unrolled by three so that its stages are compile-time constants: the
  // stage offsets of its LDS accesses then sit in the instructions'
  // immediate fields instead of being added per lane. The last (at most two)
  // of those tiles and the (at most three) masked ones at the diagonal take
  // their stage at run time.
  auto iter = [&](auto diag_tag, auto stage, int j) {
    const int S = stage;
    const int S1 = (S + 1) % kStages, S2 = (S + 2) % kStages;
    TileSrc ns;
    tile_src(j + 3, ns);
    __builtin_amdgcn_sched_barrier(0);
    phase1(diag_tag, j, S1, S);
    __syncthreads();
    phase2(S, S2, sa, ns);
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  // Group 1 issues at a higher wavefront priority for the loop: on each SIMD
  // the older wavefront (group 0's) otherwise wins the issue slots whenever
  // both are ready, so group 1's phases ran longer and group 0 waited for it
  // at every barrier. Measured on MI355X, the mixed int8 step's chunked pass:
  // 53.8-54.0 against 54.3-54.5 us (group 0 raised instead: 54.2-54.5).
  if (th == 1) __builtin_amdgcn_s_setprio(1);
  if (th == 1) __syncthreads();
  const int fdc = min(first_diag, ntiles);
  int j = 0;
  // tiles before the diagonal: stages 0, 1, 2 in turn from tile 0
  for (; j + 3 <= fdc; j += 3) {
    iter(std::false_type{}, I0{}, j);
    iter(std::false_type{}, I1{}, j + 1);
    iter(std::false_type{}, I2{}, j + 2);
  }
  for (; j < fdc; ++j) iter(std::false_type{}, j % kStages, j);
  for (; j < ntiles; ++j) iter(std::true_type{}, j % kStages, j);
  if (th == 0) __syncthreads();
  __builtin_amdgcn_s_setprio(0);

  // ---- merge the two token halves: wavefront w + 4 hands (o, m, l) to w ----
  bad = __syncthreads_or(bad);   // also: every wavefront is done with the stages
  // the exponent o and l are taken relative to (8-bit caches: with the V scale reference)
  const float mref = (kScaled && m != neg_inf()) ? m + mu_off : m;
  constexpr int kMO = 16 * kDB;   // o values per lane
  float* mb = reinterpret_cast<float*>(&s_kv[0][0]) + (rb * kMergeFloats) * 64 + lane;   // [rb][o, m, l][64 lanes]
  if (th == 1) {
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
#pragma unroll
      for (int v = 0; v < 16; ++v) mb[(16 * db + v) * 64] = o[db][v];
    }
    mb[kMO * 64] = mref;
    mb[(kMO + 1) * 64] = l;
  }
  __syncthreads();
  if (th == 1 || !row_live) return;
  const float m2 = mb[kMO * 64], l2 = mb[(kMO + 1) * 64];
  const float mm = fmaxf(mref, m2);
  const float a1 = (mref == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f(mref - mm);
  const float a2 = (m2 == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f(m2 - mm);
  const float lt = l * a1 + l2 * a2;
  const float inv = norm_inv(lt);

  // ---- write: lane holds dims 32 db + 8 (v / 4) + 4 h + v % 4 of its row ----
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      float y[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int v = 4 * v4 + k;
        y[k] = (o[db][v] * a1 + mb[(16 * db + v) * 64] * a2) * inv;
      }
      float4 x = make_float4(y[0], y[1], y[2], y[3]);
      if (bad) x = make_float4(qnan(), qnan(), qnan(), qnan());
      *reinterpret_cast<float4*>(out_row + 32 * db + 8 * v4 + 4 * h) = x;
    }
  }
  if (h == 0 && p.lse != nullptr) {
    const float lse = bad ? qnan() : norm_lse2(mm, lt);
    p.lse[static_cast<size_t>(q0 + pi) * p.num_q_heads + hq] = lse;
  }
}

template <int KV, int G, int D>
hipError_t launch_t(const ChunkedParams& p, hipStream_t st) {
  constexpr int P = kRows / G;
  const int QT = (p.max_q_len + P - 1) / P;
  const int64_t items = static_cast<int64_t>(p.num_seqs) * p.num_kv_heads * QT;
  if (items > (int64_t(1) << 30)) return hipErrorInvalidValue;
  const int grid = static_cast<int>((items + kXcdsC - 1) / kXcdsC * kXcdsC);
  if (p.max_blocks <= kIdsCached) {
    hipLaunchKernelGGL((chunked_kernel<KV, G, true, D>), dim3(grid), dim3(kThreads), 0, st, p);
  } else {
    hipLaunchKernelGGL((chunked_kernel<KV, G, false, D>), dim3(grid), dim3(kThreads), 0, st, p);
  }
  return hipGetLastError();
}

template <int KV, int D>
hipError_t launch_g(const ChunkedParams& p, int group, hipStream_t st) {
  switch (group) {
    case 1: return launch_t<KV, 1, D>(p, st);
    case 2: return launch_t<KV, 2, D>(p, st);
    case 4: return launch_t<KV, 4, D>(p, st);
    case 8: return launch_t<KV, 8, D>(p, st);
    default: return hipErrorNotSupported;
  }
}

template <int KV>
hipError_t launch_d(const ChunkedParams& p, int head_dim, int group, hipStream_t st) {
  if (head_dim == 128) return launch_g<KV, 128>(p, group, st);
  if (head_dim == 64) return launch_g<KV, 64>(p, group, st);
  return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_chunked(const ChunkedParams& p, int kv_dtype, int head_dim, int group, hipStream_t st) {
  if (kv_dtype == PKV_BF16) return launch_d<PKV_BF16>(p, head_dim, group, st);
  if (kv_dtype == PKV_I8) return launch_d<PKV_I8>(p, head_dim, group, st);
  if (kv_dtype == PKV_FP8) return launch_d<PKV_FP8>(p, head_dim, group, st);
  return hipErrorNotSupported;
}

}  // namespace pkv
