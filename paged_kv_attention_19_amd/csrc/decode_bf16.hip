// Decode partial-pass instantiations for the bf16 KV cache.
#include "decode_kernel.h"

namespace pkv {

hipError_t launch_decode_partial_bf16(const DecodeParams& p, int q_dtype, int head_dim, int group, int waves,
                                   hipStream_t st) {
  return launch_partial_kv<PKV_BF16>(p, q_dtype, head_dim, group, waves, st);
}

hipError_t launch_decode_rows_bf16(const DecodeParams& p, int head_dim, int group, hipStream_t st) {
  return launch_rows_kv<PKV_BF16>(p, head_dim, group, st);
}

}  // namespace pkv
