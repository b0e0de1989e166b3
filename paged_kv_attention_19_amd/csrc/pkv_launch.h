// Internal interface between the C-ABI layer (api.hip) and the kernel files.
// Kernel parameter blocks are plain structs passed by value to the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

struct ReshapeParams {
  const void* k_new;
  const void* v_new;
  const int64_t* slots;
  void* k;
  void* v;
  float* k_scale;
  float* v_scale;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int64_t num_slots;
};

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  const int32_t* tables;
  const int32_t* ctx;
  const int32_t* nsplits;  // unused when direct
  float* o;                // out (direct) or o_part
  float* lse;              // out_lse (direct, may be null) or lse_part
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t max_ns;
  int32_t direct;          // 1: one split per sequence, normalised output to o/lse
  float scale_log2;        // softmax scale * log2(e)
  float* part;             // balanced mode: partials of cut segments
  int32_t* counters;       // balanced mode: one arrival counter per (sequence, kv head), zero between calls
  // split mode with append: the step's new rows, written to their slots
  // before the sequence's last block is read (k_new == nullptr: no append)
  const void* k_new;       // [batch][num_kv_heads][head_dim] in new_dtype
  const void* v_new;
  const int64_t* slots;    // [batch]
  void* k_w;               // the cache, writable
  void* v_w;
  float* k_scale_w;
  float* v_scale_w;
  int64_t num_slots;
  int32_t new_dtype;
};

struct CombineParams {
  const float* o_part;
  const float* lse_part;
  const int32_t* nsplits;
  float* out;
  float* out_lse;
  int32_t batch;
  int32_t num_q_heads;
  int32_t max_ns;
};

struct ChunkedParams {
  const void* q;
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  const int32_t* tables;
  const int32_t* ctx;
  const int32_t* cu_q;
  float* out;
  float* lse;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t max_q_len;
  float scale_log2;
};

// Each launcher returns hipSuccess or the launch error; it assumes the host
// checks of api.hip have passed (supported dtypes, sizes, group size).
hipError_t launch_reshape(const ReshapeParams& p, int src_dtype, int kv_dtype, int head_dim,
                          hipStream_t stream);
// Decode partial pass, one entry per KV element type; `waves` (2, 4, 8)
// is the number of wavefronts per workgroup. A negative `waves` launches the
// balanced single-pass decode on -waves workgroups instead.
hipError_t launch_decode_partial_f32(const DecodeParams& p, int q_dtype, int head_dim, int group, int waves,
                                     hipStream_t stream);
hipError_t launch_decode_partial_bf16(const DecodeParams& p, int q_dtype, int head_dim, int group, int waves,
                                     hipStream_t stream);
hipError_t launch_decode_partial_i8(const DecodeParams& p, int q_dtype, int head_dim, int group, int waves,
                                     hipStream_t stream);
hipError_t launch_decode_partial_fp8(const DecodeParams& p, int q_dtype, int head_dim, int group, int waves,
                                     hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t stream);
hipError_t launch_chunked(const ChunkedParams& p, int kv_dtype, int head_dim, int group,
                          hipStream_t stream);

}  // namespace pkv
