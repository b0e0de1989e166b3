// Validation of device-resident metadata (block tables, context lengths,
// split counts, cu_q_lens, slots) for the PKV_DEBUG=1 mode of the entry
// points. The normal path never reads these values on the host: the kernels
// bound-check them and turn a bad sequence into NaN. In debug mode a pass
// over them runs first, the host waits for it, and the call fails with the
// first offending entry named.
//
// The finding is one 64-bit key in a fixed device word per GPU: (code << 56) |
// index, lowered with atomicMin, so the report is the lowest code and, within
// it, the lowest index, whichever thread saw it first.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>

#include "pkv_launch.h"

namespace {

static __device__ unsigned long long first_bad;

constexpr int kThreads = 256;
constexpr int kMaxGroups = 2048;
constexpr unsigned long long kNone = ~0ull;

__device__ __forceinline__ void report(int code, long long index) {
  atomicMin(&first_bad, (static_cast<unsigned long long>(code) << 56) | static_cast<unsigned long long>(index));
}

__global__ void reset_kernel() { first_bad = kNone; }

// (sequence, block) pairs of a decode or chunked batch.
__global__ void check_tables_kernel(const int32_t* tables, int32_t max_blocks, const int32_t* ctx, int32_t batch,
                                    int32_t num_blocks) {
  const long long total = static_cast<long long>(batch) * max_blocks;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<long long>(gridDim.x) * blockDim.x) {
    const int b = static_cast<int>(i / max_blocks);
    const int j = static_cast<int>(i % max_blocks);
    const int n = ctx[b];
    const bool n_ok = n >= 0 && static_cast<long long>(n) <= static_cast<long long>(max_blocks) * 16;
    if (j == 0 && !n_ok) report(pkv::kBadContextLen, b);
    if (n_ok && j < (n + 15) / 16) {
      const int id = tables[i];
      if (id < 0 || id >= num_blocks) report(pkv::kBadBlockId, i);
    }
  }
}

__global__ void check_splits_kernel(const int32_t* nsplits, int32_t max_ns, int32_t batch) {
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < batch; b += gridDim.x * blockDim.x) {
    const int ns = nsplits[b];
    if (ns < 1 || ns > max_ns) report(pkv::kBadNumSplits, b);
  }
}

__global__ void check_cu_kernel(const int32_t* cu_q, int32_t max_q_len, const int32_t* ctx, int32_t num_seqs) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < num_seqs; i += gridDim.x * blockDim.x) {
    if (i == 0 && cu_q[0] != 0) report(pkv::kBadCuQ0, 0);
    const int L = cu_q[i + 1] - cu_q[i];
    if (L < 0) report(pkv::kBadCuQOrder, i);
    else if (L > max_q_len) report(pkv::kChunkPastMaxQ, i);
    else if (L > ctx[i]) report(pkv::kChunkPastContext, i);
  }
}

__global__ void check_slots_kernel(const int64_t* slots, int32_t n, int64_t num_slots) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    if (slots[i] >= num_slots) report(pkv::kSlotPastPool, i);
}

// slot_mapping[b] of the decode-with-append call is the slot of token n_b - 1
__global__ void check_append_slots_kernel(const int64_t* slots, const int32_t* tables, int32_t max_blocks,
                                          const int32_t* ctx, int32_t batch) {
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < batch; b += gridDim.x * blockDim.x) {
    const int n = ctx[b];
    if (n < 1 || static_cast<long long>(n) > static_cast<long long>(max_blocks) * 16) continue;   // reported above
    const long long want = static_cast<long long>(tables[static_cast<long long>(b) * max_blocks + (n - 1) / 16]) * 16 +
                           (n - 1) % 16;
    if (slots[b] != want) report(pkv::kAppendSlotMismatch, b);
  }
}

int groups_for(long long items) {
  const long long g = (items + kThreads - 1) / kThreads;
  return static_cast<int>(g < 1 ? 1 : (g > kMaxGroups ? kMaxGroups : g));
}

hipError_t finish(hipStream_t st, pkv::DebugFinding* f) {
  unsigned long long key = kNone;
  hipError_t e = hipMemcpyFromSymbolAsync(&key, HIP_SYMBOL(first_bad), sizeof(key), 0, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  f->code = key == kNone ? 0 : static_cast<int>(key >> 56);
  f->index = key == kNone ? -1 : static_cast<long long>(key & ((1ull << 56) - 1));
  return hipSuccess;
}

}  // namespace

namespace pkv {

bool debug_enabled() {
  const char* e = std::getenv("PKV_DEBUG");
  return e != nullptr && std::strcmp(e, "1") == 0;
}

hipError_t debug_check(const DebugRequest& r, hipStream_t st, DebugFinding* f) {
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(1), 0, st);
  if (r.tables != nullptr && r.batch > 0)
    hipLaunchKernelGGL(check_tables_kernel, dim3(groups_for(static_cast<long long>(r.batch) * r.max_blocks)),
                       dim3(kThreads), 0, st, r.tables, r.max_blocks, r.ctx, r.batch, r.num_blocks);
  if (r.nsplits != nullptr && r.batch > 0)
    hipLaunchKernelGGL(check_splits_kernel, dim3(groups_for(r.batch)), dim3(kThreads), 0, st, r.nsplits, r.max_ns,
                       r.batch);
  if (r.cu_q != nullptr && r.batch > 0)
    hipLaunchKernelGGL(check_cu_kernel, dim3(groups_for(r.batch)), dim3(kThreads), 0, st, r.cu_q, r.max_q_len,
                       r.ctx, r.batch);
  if (r.slots != nullptr && r.num_tokens > 0)
    hipLaunchKernelGGL(check_slots_kernel, dim3(groups_for(r.num_tokens)), dim3(kThreads), 0, st, r.slots,
                       r.num_tokens, r.num_slots);
  if (r.append_slots != nullptr && r.batch > 0)
    hipLaunchKernelGGL(check_append_slots_kernel, dim3(groups_for(r.batch)), dim3(kThreads), 0, st, r.append_slots,
                       r.tables, r.max_blocks, r.ctx, r.batch);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  return finish(st, f);
}

const char* debug_code_text(int code) {
  switch (code) {
    case kBadContextLen: return "context_lens[%lld] is negative or longer than the table holds";
    case kBadNumSplits: return "num_splits[%lld] is outside [1, max_num_splits]";
    case kBadBlockId: return "block_tables entry %lld (row-major) is outside [0, num_blocks)";
    case kBadCuQ0: return "cu_q_lens[%lld] (the first entry) is not 0";
    case kBadCuQOrder: return "cu_q_lens decreases after entry %lld";
    case kChunkPastMaxQ: return "chunk %lld is longer than max_q_len";
    case kChunkPastContext: return "chunk %lld is longer than its context";
    case kSlotPastPool: return "slot_mapping[%lld] is past the pool";
    case kAppendSlotMismatch: return "slot_mapping[%lld] is not the slot of the sequence's token n - 1";
    default: return "metadata entry %lld is invalid";
  }
}

}  // namespace pkv
