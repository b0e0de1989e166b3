// Device-side helpers shared by the gfx950 kernels of the paged-KV attention
// library: element decoding, wavefront reductions and small vector types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kWave = 64;
constexpr int kBlock = 16;                 // tokens per KV block (the only size built)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Buffer descriptor over `bytes` bytes at `base` (raw dwords, no stride):
// loads at offsets past `bytes` return 0 and access no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes, 0x00020000);
}

constexpr int kBufNt = 2;   // buffer-load cache policy: non-temporal

// 16-byte non-temporal load at byte offset `off` of a buffer (0 past its end).
__device__ __forceinline__ uint4 buffer_load_nt16(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufNt));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The same with the default cache policy.
__device__ __forceinline__ uint4 buffer_load_plain16(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 4-byte float load at byte offset `off` of a buffer (0 past its end).
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// ---- element decoding ------------------------------------------------------

// bfloat16 pair packed in one dword -> two floats (low half first). A bf16 is
// the upper 16 bits of the binary32 with the same value.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float i8_at(uint32_t w, int byte) {
  return static_cast<float>(static_cast<int8_t>((w >> (8 * byte)) & 0xffu));
}

// 16 bytes of a row -> EPL floats.
template <int KV>
__device__ __forceinline__ void unpack16(const uint4& x, float* f) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  if constexpr (KV == PKV_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  } else if constexpr (KV == PKV_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    }
  } else if constexpr (KV == PKV_I8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int b = 0; b < 4; ++b) f[4 * i + b] = i8_at(w[i], b);
    }
  } else {
    // FP8: gfx950's conversion decodes the OCP E4M3 format exactly (two codes
    // per instruction)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), false);
      const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), true);
      f[4 * i + 0] = lo.x;
      f[4 * i + 1] = lo.y;
      f[4 * i + 2] = hi.x;
      f[4 * i + 3] = hi.y;
    }
  }
}

// Caches that store an 8-bit code and a float32 scale per (token, kv head).
constexpr bool is_scaled_kv(int kv) { return kv == PKV_I8 || kv == PKV_FP8; }

// OCP FP8 E4M3 code of y: the nearest E4M3 value, ties to the even code,
// saturating at 448 (sign, 4 exponent bits with bias 7, 3 mantissa bits;
// exponent field 0 holds the subnormals m * 2^-9). |y| is written as
// q * 2^(e - 3) with e its binade exponent (at least -6, where the subnormals
// share the 2^-9 step); q = rint(|y| * 2^(3 - e)), an exact power-of-two
// scaling and one round-half-to-even, lands in [0, 16]; 16 carries into the
// next binade.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.0f);
  int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xffu) - 127;
  e = e < -6 ? -6 : e;
  float q = __builtin_rintf(__builtin_ldexpf(a, 3 - e));
  if (q >= 16.0f) {
    q = 8.0f;
    ++e;
  }
  const uint32_t qi = static_cast<uint32_t>(q);
  return sign | (qi < 8u ? qi : ((static_cast<uint32_t>(e + 7) << 3) | (qi - 8u)));
}

template <int KV>
struct KvGeom {
  static constexpr int kEsize = KV == PKV_F32 ? 4 : (KV == PKV_BF16 ? 2 : 1);
  static constexpr int kEpl = 16 / kEsize;   // elements a lane holds per 16-byte load
};

// ---- cross-lane reductions -------------------------------------------------
// DPP controls (GCN/CDNA encoding): quad permutes and in-row mirrors.
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Max / sum of x over the lanes l, l + S, l + 2 S, ... of the wavefront (S a
// power of two, 1 <= S <= 32): every lane receives the result for its coset
// l mod S. Within a 16-lane row the steps are DPP row rotations (by S, 2 S,
// ... 8, which cover the row's lanes of the coset); across rows, gfx950's
// v_permlane16_swap and v_permlane32_swap, which exchange rows between two
// registers, so that with x in both each lane sees its own value and the one
// 16 (32) lanes away: VALU steps, no LDS crossbar round trip.
constexpr int kDppRowRor1 = 0x121;   // row_ror:1; row_ror:r is kDppRowRor1 + r - 1
template <int S, typename Op>
__device__ __forceinline__ float coset_reduce(float x, Op op) {
  static_assert(S >= 1 && S <= 32 && (S & (S - 1)) == 0, "stride");
  if constexpr (S <= 1) x = op(x, dpp<kDppRowRor1>(x));
  if constexpr (S <= 2) x = op(x, dpp<kDppRowRor1 + 1>(x));
  if constexpr (S <= 4) x = op(x, dpp<kDppRowRor1 + 3>(x));
  if constexpr (S <= 8) x = op(x, dpp<kDppRowRor1 + 7>(x));
  if constexpr (S <= 16) {
    const auto h = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(h[0]), __uint_as_float(h[1]));
  }
  const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(w[0]), __uint_as_float(w[1]));
}
struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpAdd {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};

// Sum / max over aligned groups of W lanes (W in 1,2,4,8,16,32,64); every
// lane of the group receives the result. Within a 16-lane row the steps are
// DPP moves (quad permutes, then the half-row and row mirrors, each of which
// pairs a lane with one in the other half of its group); across rows,
// v_permlane16_swap and v_permlane32_swap. Every step combines two values
// with a commutative operation, so each lane of a group computes the same
// bits.
template <int W, typename Op>
__device__ __forceinline__ float group_reduce(float x, Op op) {
  if constexpr (W >= 2) x = op(x, dpp<kDppQuadXor1>(x));
  if constexpr (W >= 4) x = op(x, dpp<kDppQuadXor2>(x));
  if constexpr (W >= 8) x = op(x, dpp<kDppRowHalfMirror>(x));
  if constexpr (W >= 16) x = op(x, dpp<kDppRowMirror>(x));
  if constexpr (W >= 32) {
    const auto h = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(h[0]), __uint_as_float(h[1]));
  }
  if constexpr (W >= 64) {
    const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(w[0]), __uint_as_float(w[1]));
  }
  return x;
}

template <int W>
__device__ __forceinline__ float group_sum(float x) {
  return group_reduce<W>(x, OpAdd{});
}

template <int W>
__device__ __forceinline__ float group_max(float x) {
  return group_reduce<W>(x, OpMax{});
}

__device__ __forceinline__ float wave_max(float x) { return group_reduce<kWave>(x, OpMax{}); }

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_read_exec() & __ballot(p); }

__device__ __forceinline__ int readlane(int x, int lane) { return __builtin_amdgcn_readlane(x, lane); }

// A value known to be equal on every lane, moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(x) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }
__device__ __forceinline__ float qnan() { return __builtin_nanf(""); }

// Normalising an online-softmax state (numerator O, denominator L, base-2
// reference max M): L > 0 gives O / L and lse = (M + log2 L) ln 2; L == 0 (no
// key) gives 0 and -inf; a NaN L (a NaN was read) gives NaN.
__device__ __forceinline__ float norm_inv(float L) { return L > 0.f ? 1.f / L : (L == 0.f ? 0.f : qnan()); }
__device__ __forceinline__ float norm_lse2(float M, float L) {
  return L > 0.f ? (M + log2f(L)) * kLn2 : (L == 0.f ? neg_inf() : qnan());
}

}  // namespace pkv
