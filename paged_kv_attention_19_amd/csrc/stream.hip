// Read-only HBM stream (pkv_measure.h): the bandwidth a kernel that only
// reads a buffer once reaches, launch and drain included. Each workgroup
// reads one contiguous slab with 16-byte non-temporal buffer loads, kUnroll
// loads per lane in flight before any is used.
#include <hip/hip_runtime.h>

#include "pkv_device.h"
#include "pkv_measure.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int64_t kChunksPerGroupStep = int64_t(kThreads) * kUnroll;   // 16-byte chunks per slab pass
constexpr int kMaxGroups = 4096;

int groups_for(int64_t chunks) {
  const int64_t g = (chunks + kChunksPerGroupStep - 1) / kChunksPerGroupStep;
  return static_cast<int>(g < kMaxGroups ? g : kMaxGroups);
}

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const char* src, int64_t chunks, uint32_t* sink) {
  const int64_t per = (chunks + gridDim.x - 1) / gridDim.x;
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t hi = lo + per < chunks ? lo + per : chunks;
  uint32_t acc = 0;
  if (lo < hi) {
    // one descriptor over the slab: loads past its end return 0 with no branch
    const __amdgpu_buffer_rsrc_t r = pkv::buffer_rsrc(src + lo * 16, static_cast<int>((hi - lo) * 16));
    for (int64_t c = threadIdx.x; c < hi - lo; c += kChunksPerGroupStep) {
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = pkv::buffer_load_nt16(r, static_cast<int>((c + u * kThreads) * 16));
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  for (int m = 1; m < 64; m <<= 1) acc ^= __shfl_xor(acc, m);
  if (threadIdx.x == 0 && acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

int32_t pkv_stream_read_workgroups(size_t bytes) { return bytes == 0 ? 0 : groups_for(static_cast<int64_t>(bytes / 16)); }

pkv_status pkv_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  // errors are reported as status codes only (pkv_last_error belongs to the attention calls)
  if (src == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15u) != 0 || bytes > (size_t(1) << 40))
    return PKV_ERR_INVALID_ARG;
  const int64_t chunks = static_cast<int64_t>(bytes / 16);
  const int groups = groups_for(chunks);
  // a slab is addressed by a 32-bit buffer descriptor
  if ((chunks + groups - 1) / groups * 16 >= (int64_t(1) << 31)) return PKV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(stream_read_kernel, dim3(groups), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const char*>(src), chunks, sink);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
