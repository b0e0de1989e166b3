// reshape_and_cache for gfx950: scatter the step's new K/V rows into their
// pool slots (the "append" of a decode step: page "llm-inference" on
// shehab-ashraf.github.io, section "KV Cache", subsection "The Idea").
//
// Float caches: one thread moves one 16-byte piece of one (token, head) row of
// K and the same piece of V; consecutive threads cover a row, so both the read
// of the new rows and the write of each destination row are coalesced.
//
// Int8 and FP8 caches: a group of D / EPL lanes quantizes one (token, head)
// row (the shared row quantizer of quant_row.h).
#include "pkv_device.h"
#include "pkv_launch.h"
#include "quant_row.h"

namespace pkv {

namespace {

template <int KV, int D>
__global__ __launch_bounds__(256) void reshape_copy_kernel(ReshapeParams p) {
  constexpr int kRowBytes = D * KvGeom<KV>::kEsize;
  constexpr int kPieces = kRowBytes / 16;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = static_cast<int64_t>(p.num_tokens) * p.num_kv_heads * kPieces;
  if (gid >= total) return;
  const int piece = static_cast<int>(gid % kPieces);
  const int64_t row = gid / kPieces;  // token * Hkv + head
  const int64_t tok = row / p.num_kv_heads;
  const int h = static_cast<int>(row % p.num_kv_heads);
  const int64_t slot = p.slots[tok];
  if (slot < 0 || slot >= p.num_slots) return;
  const int64_t blk = slot / kBlock;
  const int64_t off = slot % kBlock;
  const int64_t dst = ((blk * p.num_kv_heads + h) * kBlock + off) * kRowBytes + piece * 16;
  const int64_t src = row * kRowBytes + piece * 16;
  *reinterpret_cast<uint4*>(static_cast<char*>(p.k) + dst) =
      *reinterpret_cast<const uint4*>(static_cast<const char*>(p.k_new) + src);
  *reinterpret_cast<uint4*>(static_cast<char*>(p.v) + dst) =
      *reinterpret_cast<const uint4*>(static_cast<const char*>(p.v_new) + src);
}

template <int SRC, int D, int KV>
__global__ __launch_bounds__(256) void reshape_quant_kernel(ReshapeParams p) {
  constexpr int R = D / KvGeom<SRC>::kEpl;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = static_cast<int64_t>(p.num_tokens) * p.num_kv_heads * R;
  // groups of R lanes are aligned and total is a multiple of R, so a group
  // leaves together and the shuffles below only see live lanes
  if (gid >= total) return;
  const int r = static_cast<int>(gid % R);
  const int64_t row = gid / R;
  const int64_t tok = row / p.num_kv_heads;
  const int h = static_cast<int>(row % p.num_kv_heads);
  const int64_t slot = p.slots[tok];
  if (slot < 0 || slot >= p.num_slots) return;
  const int64_t blk = slot / kBlock;
  const int64_t off = slot % kBlock;
  const int64_t dst_row = (blk * p.num_kv_heads + h) * kBlock + off;
  quantize_row_piece<SRC, D, KV>(p.k_new, p.k, p.k_scale, row, dst_row, r);
  quantize_row_piece<SRC, D, KV>(p.v_new, p.v, p.v_scale, row, dst_row, r);
}

template <int KV, int D>
hipError_t launch_copy(const ReshapeParams& p, hipStream_t st) {
  constexpr int kPieces = D * KvGeom<KV>::kEsize / 16;
  const int64_t total = static_cast<int64_t>(p.num_tokens) * p.num_kv_heads * kPieces;
  hipLaunchKernelGGL((reshape_copy_kernel<KV, D>), dim3(static_cast<uint32_t>((total + 255) / 256)), dim3(256),
                     0, st, p);
  return hipGetLastError();
}

template <int SRC, int D, int KV>
hipError_t launch_quant(const ReshapeParams& p, hipStream_t st) {
  constexpr int R = D / KvGeom<SRC>::kEpl;
  const int64_t total = static_cast<int64_t>(p.num_tokens) * p.num_kv_heads * R;
  hipLaunchKernelGGL((reshape_quant_kernel<SRC, D, KV>), dim3(static_cast<uint32_t>((total + 255) / 256)), dim3(256),
                     0, st, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_reshape_d(const ReshapeParams& p, int src, int kv, hipStream_t st) {
  if (kv == PKV_F32 && src == PKV_F32) return launch_copy<PKV_F32, D>(p, st);
  if (kv == PKV_BF16 && src == PKV_BF16) return launch_copy<PKV_BF16, D>(p, st);
  if (kv == PKV_I8 && src == PKV_F32) return launch_quant<PKV_F32, D, PKV_I8>(p, st);
  if (kv == PKV_I8 && src == PKV_BF16) return launch_quant<PKV_BF16, D, PKV_I8>(p, st);
  if (kv == PKV_FP8 && src == PKV_F32) return launch_quant<PKV_F32, D, PKV_FP8>(p, st);
  if (kv == PKV_FP8 && src == PKV_BF16) return launch_quant<PKV_BF16, D, PKV_FP8>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_reshape(const ReshapeParams& p, int src_dtype, int kv_dtype, int head_dim, hipStream_t st) {
  if (p.num_tokens == 0) return hipSuccess;
  switch (head_dim) {
    case 64: return launch_reshape_d<64>(p, src_dtype, kv_dtype, st);
    case 128: return launch_reshape_d<128>(p, src_dtype, kv_dtype, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
