// Chunked prefill (causal query chunks over a paged prefix) -- MFMA kernel.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

hipError_t launch_chunked(const ChunkedParams&, int, int, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pkv
