// Scaled 8-bit quantization of one (token, head) row, shared by the
// reshape_and_cache kernel and the decode pass that appends the step's new
// rows, so both write the same codes and scales bit for bit.
//
// Int8 (course README "Build an LLM Inference Engine From Scratch",
// curriculum S08, symmetric reading of its q = round(w / scale) + zero with
// zero = 0): a group of R = D / EPL aligned lanes holds one row; the group
// takes amax = max |x|, scale = amax / 127 (IEEE float32 division; amax == 0
// gives 1) and code = clamp(rint(x / scale), -127, 127), again with an IEEE
// division and round-half-to-even, so codes are exactly those of a float32
// reference.
//
// FP8 (same README, curriculum S00 bf16/fp8, read as OCP E4M3 scaled like
// the int8 cache): scale = amax / 448 and code = the E4M3 code of the float32
// quotient x / scale (nearest value, ties to the even code, saturating).
#pragma once

#include "pkv_device.h"

namespace pkv {

// Lane r (0 .. R-1) of an aligned group of R lanes, holding the 16 bytes
// `raw` of elements [r EPL, (r + 1) EPL) of one row in SRC: the row's codes
// -> codes_out[dst_row][D] and its scale -> scales_out[dst_row].
template <int SRC, int D, int KV = PKV_I8>
__device__ __forceinline__ void quantize_piece(uint4 raw, void* codes_out, float* scales_out, int64_t dst_row,
                                               int r) {
  static_assert(is_scaled_kv(KV), "a scaled 8-bit cache");
  constexpr float kMaxCode = KV == PKV_I8 ? 127.0f : 448.0f;
  constexpr int EPL = KvGeom<SRC>::kEpl;  // source elements per lane (4 or 8)
  constexpr int R = D / EPL;              // lanes per row
  float x[EPL];
  unpack16<SRC>(raw, x);
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = group_max<R>(amax);
  const float scale = amax > 0.f ? amax / kMaxCode : 1.0f;
  uint32_t packed[EPL / 4];
#pragma unroll
  for (int e = 0; e < EPL / 4; ++e) packed[e] = 0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    uint32_t byte;
    if constexpr (KV == PKV_I8) {
      float qv = __builtin_rintf(x[e] / scale);
      qv = fminf(fmaxf(qv, -127.0f), 127.0f);
      byte = static_cast<uint32_t>(static_cast<int32_t>(qv)) & 0xffu;
    } else {
      byte = e4m3_code(x[e] / scale);
    }
    packed[e / 4] |= byte << (8 * (e % 4));
  }
  char* dst = static_cast<char*>(codes_out) + dst_row * D + r * EPL;
  if constexpr (EPL == 8) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
  } else {
    *reinterpret_cast<uint32_t*>(dst) = packed[0];
  }
  if (r == 0) scales_out[dst_row] = scale;
}

// The same, reading the piece from row `row` of src_rows ([rows][D] in SRC).
template <int SRC, int D, int KV = PKV_I8>
__device__ __forceinline__ void quantize_row_piece(const void* src_rows, void* codes_out, float* scales_out,
                                                   int64_t row, int64_t dst_row, int r) {
  constexpr int EPL = KvGeom<SRC>::kEpl;
  const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const char*>(src_rows) +
                                                    (row * D + r * EPL) * KvGeom<SRC>::kEsize);
  quantize_piece<SRC, D, KV>(raw, codes_out, scales_out, dst_row, r);
}

}  // namespace pkv
