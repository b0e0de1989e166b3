// Decode partial-pass instantiations for the fp8 (OCP E4M3) KV cache.
#include "decode_kernel.h"

namespace pkv {

hipError_t launch_decode_partial_fp8(const DecodeParams& p, int q_dtype, int head_dim, int group, int waves,
                                    hipStream_t st) {
  return launch_partial_kv<PKV_FP8>(p, q_dtype, head_dim, group, waves, st);
}

hipError_t launch_decode_rows_fp8(const DecodeParams& p, int head_dim, int group, hipStream_t st) {
  return launch_rows_kv<PKV_FP8>(p, head_dim, group, st);
}

}  // namespace pkv
