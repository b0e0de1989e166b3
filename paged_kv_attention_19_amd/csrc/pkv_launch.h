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
  // several new rows per sequence (decode_rows_kernel): row r of sequence b
  // is q row cu_q[b] + r at position n_b - L_b + r, L_b = cu_q[b+1] - cu_q[b]
  const int32_t* cu_q;
  int32_t max_q_len;
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

// ---- PKV_DEBUG=1: validation of device-resident metadata (validate.hip) ----
enum DebugCode {
  kBadContextLen = 1,
  kBadNumSplits,
  kBadBlockId,
  kBadCuQ0,
  kBadCuQOrder,
  kChunkPastMaxQ,
  kChunkPastContext,
  kSlotPastPool,
  kAppendSlotMismatch,
};

// What to validate; null pointers (or zero counts) skip a check.
struct DebugRequest {
  const int32_t* tables = nullptr;   // with ctx: ids of blocks < ceil(n / 16) within the pool
  int32_t max_blocks = 0;
  const int32_t* ctx = nullptr;      // lengths within [0, max_blocks * 16]
  const int32_t* nsplits = nullptr;  // split counts within [1, max_ns]
  int32_t max_ns = 0;
  int32_t batch = 0;                 // sequences
  int32_t num_blocks = 0;
  const int32_t* cu_q = nullptr;     // with ctx: cu_q[0] == 0, chunks of 0 .. min(max_q_len, n) rows
  int32_t max_q_len = 0;
  const int64_t* slots = nullptr;    // slots below num_slots (negative ones are skips)
  int32_t num_tokens = 0;
  int64_t num_slots = 0;
  const int64_t* append_slots = nullptr;   // with tables, ctx: slot of token n - 1
};

struct DebugFinding {
  int code;          // 0: nothing found
  long long index;   // entry of the offending array
};

bool debug_enabled();
// Launches the checks on `stream`, waits for them, and fills *f.
hipError_t debug_check(const DebugRequest& r, hipStream_t stream, DebugFinding* f);
// printf-style text for a code, with one %lld for the index.
const char* debug_code_text(int code);

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
// Several new rows per sequence (chunks of at most max_q_len rows with
// max_q_len * group <= 8), one workgroup per (sequence, kv head): the chunked
// entry point's path for short chunks (p.cu_q, p.max_q_len set; bf16 q).
hipError_t launch_decode_rows_bf16(const DecodeParams& p, int head_dim, int group, hipStream_t stream);
hipError_t launch_decode_rows_i8(const DecodeParams& p, int head_dim, int group, hipStream_t stream);
hipError_t launch_decode_rows_fp8(const DecodeParams& p, int head_dim, int group, hipStream_t stream);
// The same rows on MFMA (rows_mfma.hip): max_q_len * group <= 16, bf16 q, head_dim 128.
hipError_t launch_rows_mfma(const DecodeParams& p, int kv_dtype, int head_dim, int group, hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t stream);
hipError_t launch_chunked(const ChunkedParams& p, int kv_dtype, int head_dim, int group,
                          hipStream_t stream);

}  // namespace pkv
