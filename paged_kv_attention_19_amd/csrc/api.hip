// C-ABI entry points of the paged-KV attention library (declared in pkv.h):
// host-side argument checks, then kernel launches on the caller's stream.
// Nothing here allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "pkv.h"
#include "pkv_launch.h"

namespace {

thread_local std::string g_error;

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

pkv_status ok() {
  g_error.clear();
  return PKV_OK;
}

pkv_status hip_fail(hipError_t e, const char* what) {
  return fail(PKV_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
}

// PKV_DEBUG=1: validate the device-resident metadata of a call before its
// launches (a synchronising pass; see validate.hip). Returns PKV_OK when the
// mode is off or nothing is wrong.
pkv_status debug_validate(const char* fn, const pkv::DebugRequest& r, void* stream) {
  if (!pkv::debug_enabled()) return PKV_OK;
  pkv::DebugFinding f{};
  const hipError_t e = pkv::debug_check(r, static_cast<hipStream_t>(stream), &f);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s: PKV_DEBUG validation did not run: %s", fn, hipGetErrorString(e));
  if (f.code == 0) return PKV_OK;
  char what[256];
  snprintf(what, sizeof(what), pkv::debug_code_text(f.code), f.index);
  return fail(PKV_ERR_INVALID_ARG, "%s: PKV_DEBUG: %s", fn, what);
}

// The decode calls' metadata, for debug_validate.
pkv::DebugRequest decode_request(int32_t batch, const pkv_cache* cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens, const int32_t* num_splits,
                                 int32_t max_num_splits) {
  pkv::DebugRequest r;
  r.tables = block_tables;
  r.max_blocks = max_blocks_per_seq;
  r.ctx = context_lens;
  r.batch = batch;
  r.num_blocks = cache->num_blocks;
  if (max_num_splits > 1) {   // one split per sequence and the balanced mode read no split counts
    r.nsplits = num_splits;
    r.max_ns = max_num_splits;
  }
  return r;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

const char* dtype_name(int d) {
  switch (d) {
    case PKV_F32: return "F32";
    case PKV_BF16: return "BF16";
    case PKV_I8: return "I8";
    case PKV_FP8: return "FP8";
    default: return "?";
  }
}

// Checks shared by every call that reads or writes the pool.
pkv_status check_cache(const pkv_cache* c, const char* fn) {
  if (c == nullptr) return fail(PKV_ERR_INVALID_ARG, "%s: cache descriptor is NULL", fn);
  if (c->k == nullptr || c->v == nullptr) return fail(PKV_ERR_INVALID_ARG, "%s: cache k/v is NULL", fn);
  if (c->num_blocks < 1 || c->num_kv_heads < 1)
    return fail(PKV_ERR_INVALID_ARG, "%s: num_blocks=%d num_kv_heads=%d must be >= 1", fn, c->num_blocks,
                c->num_kv_heads);
  if (c->block_size != 16) return fail(PKV_ERR_UNSUPPORTED, "%s: block_size=%d (built: 16)", fn, c->block_size);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "%s: head_dim=%d (built: 64, 128)", fn, c->head_dim);
  if (c->kv_dtype != PKV_F32 && c->kv_dtype != PKV_BF16 && c->kv_dtype != PKV_I8 && c->kv_dtype != PKV_FP8)
    return fail(PKV_ERR_INVALID_ARG, "%s: kv_dtype=%d is not F32/BF16/I8/FP8", fn, c->kv_dtype);
  const bool scaled = c->kv_dtype == PKV_I8 || c->kv_dtype == PKV_FP8;
  if (scaled && (c->k_scale == nullptr || c->v_scale == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "%s: %s cache needs k_scale and v_scale", fn, dtype_name(c->kv_dtype));
  if (!aligned16(c->k) || !aligned16(c->v)) return fail(PKV_ERR_INVALID_ARG, "%s: cache k/v not 16-byte aligned", fn);
  if (scaled && ((reinterpret_cast<uintptr_t>(c->k_scale) | reinterpret_cast<uintptr_t>(c->v_scale)) & 3u))
    return fail(PKV_ERR_INVALID_ARG, "%s: scales not 4-byte aligned", fn);
  const int64_t tile_elems = static_cast<int64_t>(c->num_kv_heads) * c->block_size * c->head_dim;
  if (tile_elems * c->num_blocks > (int64_t(1) << 46))
    return fail(PKV_ERR_INVALID_ARG, "%s: pool of %d blocks is implausibly large", fn, c->num_blocks);
  return PKV_OK;
}

pkv_status check_group(int num_q_heads, int num_kv_heads, const char* fn) {
  if (num_q_heads < 1) return fail(PKV_ERR_INVALID_ARG, "%s: num_q_heads=%d", fn, num_q_heads);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: num_q_heads=%d not a multiple of num_kv_heads=%d", fn, num_q_heads,
                num_kv_heads);
  const int g = num_q_heads / num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(PKV_ERR_UNSUPPORTED, "%s: GQA group size %d (built: 1, 2, 4, 8)", fn, g);
  return PKV_OK;
}

// Wavefronts per decode workgroup. A workgroup reduces one split; its blocks
// are dealt to the wavefronts round-robin. Four wavefronts (one per SIMD)
// measured best on MI355X for every decode shape tried, from 8-block splits
// to 32-block ones: more add per-wave setup and merge work, fewer leave
// SIMDs idle. PKV_DECODE_WAVES (2, 4 or 8) overrides the choice, for tuning.
int decode_waves(int /*max_blocks_per_seq*/, int /*max_num_splits*/) {
  static const int forced = [] {
    const char* e = std::getenv("PKV_DECODE_WAVES");
    const int v = e ? std::atoi(e) : 0;
    return (v == 2 || v == 4 || v == 8) ? v : 0;
  }();
  return forced ? forced : 4;
}

// Balanced decode: 4 wavefronts per workgroup, 256 workgroups (one per CU)
// or 512 for large batches; each wavefront owns two partial slots of
// G (D + 1) floats (G <= Hq).
// (pkv_decode_workspace_bytes knows only num_q_heads and sizes the slots for
// a group of num_q_heads; the kernel uses group * (head_dim + 1) floats per
// slot.)
// Chunks of at most this many query rows per kv head (max_q_len times the GQA
// group) go to the decode kernels rather than an MFMA kernel: with so few
// rows an MFMA tile is mostly empty, while the decode kernels stream the K/V
// tiles once with every row in registers. Their VALU work grows with the
// rows. Measured on MI355X, 32 sequences of 128..384 tokens (8 kv heads), L
// new rows each with G query heads per kv head. Against the 128-row MFMA
// kernel, the decode kernels take 9.6-10.1 us at L x G = 1 or 2 (18.0-18.8),
// 13.0-13.2 at 4 (18.1-18.8) and 23.8-25.0 at 8 (18.3-19.9). Against the
// few-row MFMA kernel below, with head dims of 128: 8.4-9.8 against
// 10.0-11.6 at 2 rows (L 1, G 2 or L 2, G 1; bf16, int8 and fp8 caches);
// then the MFMA kernel leads, 12.9 against 11.8 at 3 rows (L 3, G 1), at 4
// 12.3-13.1 against 12.0 over bf16, 13.4-14.0 against 10.8-10.9 over int8
// and 12.7-13.3 against 10.4 over fp8.
constexpr int kRowsDecodeMax = 4;
constexpr int kRowsDecodeMax128 = 2;
constexpr int kRowsMfmaMax = 16;

// The chunked entry point's kernel for R = max_q_len * group rows per kv head.
int chunked_kernel_of(int64_t rows, int head_dim) {
  const bool mfma_rows = head_dim == 128;   // the few-row MFMA kernel is built for 128
  if (rows <= (mfma_rows ? kRowsDecodeMax128 : kRowsDecodeMax)) return PKV_CHUNKED_DECODE_ROWS;
  if (mfma_rows && rows <= kRowsMfmaMax) return PKV_CHUNKED_ROWS_MFMA;
  return PKV_CHUNKED_TILES;
}

constexpr int kBalancedMaxWorkgroups = 512;
size_t balanced_part_bytes(int heads_per_slot, int head_dim) {
  return static_cast<size_t>(kBalancedMaxWorkgroups) * 4 * 2 * heads_per_slot * (head_dim + 1) * sizeof(float);
}
size_t balanced_counter_bytes(int batch, int num_q_heads) {
  return (static_cast<size_t>(batch) * num_q_heads * sizeof(int32_t) + 255) & ~static_cast<size_t>(255);
}
int balanced_workgroups(int batch, int num_kv_heads, int max_blocks) {
  const int64_t tiles_bound = static_cast<int64_t>(batch) * num_kv_heads * max_blocks;
  return tiles_bound <= 65536 ? 256 : kBalancedMaxWorkgroups;
}

}  // namespace

// ---- scratch memory of the allocation-free decode entry point ----
// One fixed device array per GPU the library runs on, held until the process
// ends. Host code never uses the array's name as an address (on the host it
// is only a stand-in for the symbol): it asks the runtime for the device
// address once per device and passes that to the kernels.
constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Zero n int32 words (the balanced mode's arrival counters). A kernel rather
// than a memset node, so that a captured graph replays it correctly.
__global__ void zero_words_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, looked up on the first
// call there (with that device current) and kept.
pkv_status scratch_address(const char* fn, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_UNSUPPORTED, "%s: device %d (built: < %d)", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(PKV_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed: %s", fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

// Scratch bytes the no-alloc decode needs: as pkv_decode_workspace_bytes,
// but with the balanced mode's partial slots sized for the actual GQA group.
size_t noalloc_bytes(int batch, int num_q_heads, int group, int head_dim, int max_num_splits) {
  if (max_num_splits == 0) return balanced_counter_bytes(batch, num_q_heads) + balanced_part_bytes(group, head_dim);
  return pkv_decode_workspace_bytes(batch, num_q_heads, head_dim, max_num_splits);
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_error.c_str(); }

const char* pkv_version(void) { return "pkv 0.1 gfx950"; }

pkv_status pkv_reshape_and_cache(const void* k_new, const void* v_new, int32_t src_dtype,
                                 const int64_t* slot_mapping, int32_t num_tokens, const pkv_cache* cache,
                                 void* stream) {
  const char* fn = "pkv_reshape_and_cache";
  if (pkv_status st = check_cache(cache, fn); st != PKV_OK) return st;
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "%s: num_tokens=%d", fn, num_tokens);
  if (num_tokens == 0) return ok();
  if (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "%s: k_new/v_new/slot_mapping is NULL", fn);
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(PKV_ERR_INVALID_ARG, "%s: k_new/v_new not 16-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(slot_mapping) & 7u) != 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: slot_mapping not 8-byte aligned", fn);
  const int kv = cache->kv_dtype;
  if (kv == PKV_I8 || kv == PKV_FP8) {
    if (src_dtype != PKV_F32 && src_dtype != PKV_BF16)
      return fail(PKV_ERR_INVALID_ARG, "%s: %s cache takes F32 or BF16 rows, got %s", fn, dtype_name(kv),
                  dtype_name(src_dtype));
  } else if (src_dtype != kv) {
    return fail(PKV_ERR_INVALID_ARG, "%s: %s cache needs %s rows, got %s", fn, dtype_name(kv), dtype_name(kv),
                dtype_name(src_dtype));
  }
  pkv::ReshapeParams p{};
  p.k_new = k_new;
  p.v_new = v_new;
  p.slots = slot_mapping;
  p.k = cache->k;
  p.v = cache->v;
  p.k_scale = cache->k_scale;
  p.v_scale = cache->v_scale;
  p.num_tokens = num_tokens;
  p.num_kv_heads = cache->num_kv_heads;
  p.num_slots = static_cast<int64_t>(cache->num_blocks) * cache->block_size;
  pkv::DebugRequest dr;
  dr.slots = slot_mapping;
  dr.num_tokens = num_tokens;
  dr.num_slots = p.num_slots;
  if (pkv_status st = debug_validate(fn, dr, stream); st != PKV_OK) return st;
  const hipError_t e = pkv::launch_reshape(p, src_dtype, kv, cache->head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim, int32_t max_num_splits) {
  if (batch <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_num_splits < 0) return 0;
  if (max_num_splits == 0) return balanced_counter_bytes(batch, num_q_heads) + balanced_part_bytes(num_q_heads, head_dim);
  if (max_num_splits == 1) return 0;
  const size_t rows = static_cast<size_t>(batch) * max_num_splits * num_q_heads;
  const size_t bytes = rows * (static_cast<size_t>(head_dim) + 1) * sizeof(float);
  return (bytes + 255) & ~static_cast<size_t>(255);
}

// Argument checks shared by the decode entry points; *empty is set when there
// is nothing to launch (batch == 0).
static pkv_status check_decode(const char* fn, const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                               const pkv_cache* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, const int32_t* num_splits, int32_t max_num_splits,
                               float scale, const float* out, const void* workspace, size_t workspace_bytes,
                               bool* empty, bool library_scratch = false) {
  if (pkv_status st = check_cache(cache, fn); st != PKV_OK) return st;
  if (batch < 0) return fail(PKV_ERR_INVALID_ARG, "%s: batch=%d", fn, batch);
  if (pkv_status st = check_group(num_q_heads, cache->num_kv_heads, fn); st != PKV_OK) return st;
  if (batch == 0) {
    *empty = true;
    return ok();
  }
  if (batch > 65535) return fail(PKV_ERR_UNSUPPORTED, "%s: batch=%d (built: <= 65535)", fn, batch);
  if (q_dtype != PKV_F32 && q_dtype != PKV_BF16)
    return fail(PKV_ERR_INVALID_ARG, "%s: q_dtype=%s (F32 or BF16)", fn, dtype_name(q_dtype));
  if (q == nullptr || block_tables == nullptr || context_lens == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "%s: q/block_tables/context_lens is NULL", fn);
  if (out == nullptr && max_num_splits == 1)
    return fail(PKV_ERR_INVALID_ARG, "%s: out is NULL (partials-only mode needs max_num_splits > 1)", fn);
  if (!aligned16(q) || !aligned16(out)) return fail(PKV_ERR_INVALID_ARG, "%s: q/out not 16-byte aligned", fn);
  if (max_blocks_per_seq < 1) return fail(PKV_ERR_INVALID_ARG, "%s: max_blocks_per_seq=%d", fn, max_blocks_per_seq);
  const bool balanced = max_num_splits == 0;
  if (max_num_splits < 0 || max_num_splits > 65535)
    return fail(PKV_ERR_INVALID_ARG, "%s: max_num_splits=%d (0..65535)", fn, max_num_splits);
  if (max_num_splits > 1 && num_splits == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "%s: num_splits is NULL with max_num_splits=%d", fn, max_num_splits);
  if (balanced && num_splits != nullptr)
    return fail(PKV_ERR_INVALID_ARG, "%s: max_num_splits=0 (balanced) takes no num_splits", fn);
  if (balanced && out == nullptr) return fail(PKV_ERR_INVALID_ARG, "%s: out is NULL in balanced mode", fn);
  if (balanced && static_cast<int64_t>(batch) * cache->num_kv_heads * max_blocks_per_seq > (int64_t(1) << 40))
    return fail(PKV_ERR_UNSUPPORTED, "%s: batch too large for the balanced mode", fn);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  const int D = cache->head_dim;
  const size_t need = library_scratch ? 0 : pkv_decode_workspace_bytes(batch, num_q_heads, D, max_num_splits);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(PKV_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace == nullptr ? size_t(0) : workspace_bytes);
  if (need > 0 && !aligned16(workspace)) return fail(PKV_ERR_INVALID_ARG, "%s: workspace not 16-byte aligned", fn);
  return ok();

}

// Split mode (max_num_splits >= 1): the partial pass, then the merge when
// there are several splits and an output. `append` (may be null) adds the
// step's new rows to the pass. The arguments have been checked.
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  int32_t src_dtype;
  const int64_t* slots;
};

static pkv_status run_split_decode(const char* fn, const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                                   const pkv_cache* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, const int32_t* num_splits, int32_t max_num_splits,
                                   float scale, float* out, float* out_lse, void* workspace,
                                   const AppendArgs* append, void* stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int D = cache->head_dim;
  const int group = num_q_heads / cache->num_kv_heads;
  const bool direct = max_num_splits == 1;
  float* o_part = static_cast<float*>(workspace);
  float* lse_part = direct ? nullptr : o_part + static_cast<size_t>(batch) * max_num_splits * num_q_heads * D;

  pkv::DecodeParams p{};
  p.q = q;
  p.k = cache->k;
  p.v = cache->v;
  p.k_scale = cache->k_scale;
  p.v_scale = cache->v_scale;
  p.tables = block_tables;
  p.ctx = context_lens;
  p.nsplits = num_splits;
  p.o = direct ? out : o_part;
  p.lse = direct ? out_lse : lse_part;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = cache->num_kv_heads;
  p.max_blocks = max_blocks_per_seq;
  p.num_blocks = cache->num_blocks;
  p.max_ns = max_num_splits;
  p.direct = direct ? 1 : 0;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.batch = batch;
  if (append != nullptr) {
    p.k_new = append->k_new;
    p.v_new = append->v_new;
    p.slots = append->slots;
    p.new_dtype = append->src_dtype;
    p.k_w = cache->k;
    p.v_w = cache->v;
    p.k_scale_w = cache->k_scale;
    p.v_scale_w = cache->v_scale;
    p.num_slots = static_cast<int64_t>(cache->num_blocks) * cache->block_size;
  }
  const int waves = decode_waves(max_blocks_per_seq, max_num_splits);
  hipError_t e;
  switch (cache->kv_dtype) {
    case PKV_F32: e = pkv::launch_decode_partial_f32(p, q_dtype, D, group, waves, st); break;
    case PKV_BF16: e = pkv::launch_decode_partial_bf16(p, q_dtype, D, group, waves, st); break;
    case PKV_I8: e = pkv::launch_decode_partial_i8(p, q_dtype, D, group, waves, st); break;
    default: e = pkv::launch_decode_partial_fp8(p, q_dtype, D, group, waves, st); break;
  }
  if (e != hipSuccess) return hip_fail(e, fn);
  if (!direct && out != nullptr) {
    pkv::CombineParams cp{};
    cp.o_part = o_part;
    cp.lse_part = lse_part;
    cp.nsplits = num_splits;
    cp.out = out;
    cp.out_lse = out_lse;
    cp.batch = batch;
    cp.num_q_heads = num_q_heads;
    cp.max_ns = max_num_splits;
    e = pkv::launch_combine(cp, D, st);
    if (e != hipSuccess) return hip_fail(e, fn);
  }
  return ok();
}

// Balanced mode (max_num_splits == 0): one launch; the workspace holds the
// arrival counters (zero on entry), then the partial slots. The arguments have
// been checked.
static pkv_status run_balanced_decode(const char* fn, const void* q, int32_t q_dtype, int32_t batch,
                                      int32_t num_q_heads, const pkv_cache* cache, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* context_lens, float scale,
                                      float* out, float* out_lse, void* workspace, void* stream) {
  const int D = cache->head_dim;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int group = num_q_heads / cache->num_kv_heads;
  pkv::DecodeParams p{};
  p.q = q;
  p.k = cache->k;
  p.v = cache->v;
  p.k_scale = cache->k_scale;
  p.v_scale = cache->v_scale;
  p.tables = block_tables;
  p.ctx = context_lens;
  p.o = out;
  p.lse = out_lse;
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = cache->num_kv_heads;
  p.max_blocks = max_blocks_per_seq;
  p.num_blocks = cache->num_blocks;
  p.max_ns = 0;
  p.direct = 1;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.counters = static_cast<int32_t*>(workspace);
  p.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + balanced_counter_bytes(batch, num_q_heads));
  const int wgs = balanced_workgroups(batch, cache->num_kv_heads, max_blocks_per_seq);
  hipError_t e;
  switch (cache->kv_dtype) {
    case PKV_F32: e = pkv::launch_decode_partial_f32(p, q_dtype, D, group, -wgs, st); break;
    case PKV_BF16: e = pkv::launch_decode_partial_bf16(p, q_dtype, D, group, -wgs, st); break;
    case PKV_I8: e = pkv::launch_decode_partial_i8(p, q_dtype, D, group, -wgs, st); break;
    default: e = pkv::launch_decode_partial_fp8(p, q_dtype, D, group, -wgs, st); break;
  }
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

// One split per sequence while every table is at most 64 blocks (1024
// tokens) wide: a workgroup then streams at most 16 blocks per wavefront and
// the launch has no merge. Wider tables go to the balanced mode, which evens
// out long and short sequences at the price of a cross-workgroup merge.
// Measured on MI355X, decode launch alone (bf16, 16 q / 8 kv heads, D 128):
// n in [128, 384] (24-block tables), B = 8 .. 128: 7.9 / 8.0 / 9.8 / 15.5 /
// 26.6 us with one split against 22.1 / 20.8 / 22.6 / 28.2 / 41.9 us
// balanced; 256 log-uniform n in [64, 8192] (512-block tables): 295 us
// balanced against 333 us with one split.
constexpr int kOneSplitMaxBlocks = 64;

int32_t pkv_decode_default_max_num_splits(int32_t max_blocks_per_seq) {
  if (max_blocks_per_seq < 1) {
    fail(PKV_ERR_INVALID_ARG, "pkv_decode_default_max_num_splits: max_blocks_per_seq=%d", max_blocks_per_seq);
    return -1;
  }
  return max_blocks_per_seq <= kOneSplitMaxBlocks ? 1 : 0;
}

pkv_status pkv_paged_attention_decode(const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                                      const pkv_cache* cache, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                                      const int32_t* num_splits, int32_t max_num_splits, float scale, float* out,
                                      float* out_lse, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "pkv_paged_attention_decode";
  bool empty = false;
  if (pkv_status st = check_decode(fn, q, q_dtype, batch, num_q_heads, cache, block_tables, max_blocks_per_seq,
                                   context_lens, num_splits, max_num_splits, scale, out, workspace, workspace_bytes,
                                   &empty);
      st != PKV_OK || empty)
    return st;
  if (pkv_status st = debug_validate(fn, decode_request(batch, cache, block_tables, max_blocks_per_seq, context_lens,
                                                        num_splits, max_num_splits),
                                     stream);
      st != PKV_OK)
    return st;
  if (max_num_splits == 0)
    return run_balanced_decode(fn, q, q_dtype, batch, num_q_heads, cache, block_tables, max_blocks_per_seq,
                               context_lens, scale, out, out_lse, workspace, stream);
  return run_split_decode(fn, q, q_dtype, batch, num_q_heads, cache, block_tables, max_blocks_per_seq, context_lens,
                          num_splits, max_num_splits, scale, out, out_lse, workspace, nullptr, stream);
}

pkv_status pkv_paged_attention_decode_append(const void* k_new, const void* v_new, int32_t src_dtype,
                                             const int64_t* slot_mapping, const void* q, int32_t q_dtype,
                                             int32_t batch, int32_t num_q_heads, const pkv_cache* cache,
                                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                                             const int32_t* context_lens, const int32_t* num_splits,
                                             int32_t max_num_splits, float scale, float* out, float* out_lse,
                                             void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "pkv_paged_attention_decode_append";
  if (max_num_splits == 0)
    return fail(PKV_ERR_UNSUPPORTED, "%s: the balanced mode (max_num_splits = 0) has no append", fn);
  bool empty = false;
  if (pkv_status st = check_decode(fn, q, q_dtype, batch, num_q_heads, cache, block_tables, max_blocks_per_seq,
                                   context_lens, num_splits, max_num_splits, scale, out, workspace, workspace_bytes,
                                   &empty);
      st != PKV_OK || empty)
    return st;
  if (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "%s: k_new/v_new/slot_mapping is NULL", fn);
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(PKV_ERR_INVALID_ARG, "%s: k_new/v_new not 16-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(slot_mapping) & 7u) != 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: slot_mapping not 8-byte aligned", fn);
  const int kv = cache->kv_dtype;
  if (kv == PKV_I8 || kv == PKV_FP8) {
    if (src_dtype != PKV_F32 && src_dtype != PKV_BF16)
      return fail(PKV_ERR_INVALID_ARG, "%s: %s cache takes F32 or BF16 rows, got %s", fn, dtype_name(kv),
                  dtype_name(src_dtype));
  } else if (src_dtype != kv) {
    return fail(PKV_ERR_INVALID_ARG, "%s: %s cache needs %s rows, got %s", fn, dtype_name(kv), dtype_name(kv),
                dtype_name(src_dtype));
  }
  pkv::DebugRequest dr =
      decode_request(batch, cache, block_tables, max_blocks_per_seq, context_lens, num_splits, max_num_splits);
  dr.append_slots = slot_mapping;
  if (pkv_status st = debug_validate(fn, dr, stream); st != PKV_OK) return st;
  const AppendArgs append{k_new, v_new, src_dtype, slot_mapping};
  return run_split_decode(fn, q, q_dtype, batch, num_q_heads, cache, block_tables, max_blocks_per_seq, context_lens,
                          num_splits, max_num_splits, scale, out, out_lse, workspace, &append, stream);
}

pkv_status pkv_lse_combine(const float* o_part, const float* lse_part, int32_t batch, int32_t num_q_heads,
                           int32_t head_dim, int32_t max_num_splits, const int32_t* num_splits, float* out,
                           float* out_lse, void* stream) {
  const char* fn = "pkv_lse_combine";
  if (batch < 0 || num_q_heads < 1 || max_num_splits < 1)
    return fail(PKV_ERR_INVALID_ARG, "%s: batch=%d num_q_heads=%d max_num_splits=%d", fn, batch, num_q_heads,
                max_num_splits);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "%s: head_dim=%d (built: 64, 128)", fn, head_dim);
  if (batch == 0) return ok();
  if (static_cast<int64_t>(batch) * num_q_heads > (int64_t(1) << 30))
    return fail(PKV_ERR_INVALID_ARG, "%s: batch * num_q_heads too large", fn);
  if (o_part == nullptr || lse_part == nullptr || num_splits == nullptr || out == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "%s: o_part/lse_part/num_splits/out is NULL", fn);
  pkv::CombineParams cp{};
  cp.o_part = o_part;
  cp.lse_part = lse_part;
  cp.nsplits = num_splits;
  cp.out = out;
  cp.out_lse = out_lse;
  cp.batch = batch;
  cp.num_q_heads = num_q_heads;
  cp.max_ns = max_num_splits;
  pkv::DebugRequest dr;
  dr.nsplits = num_splits;
  dr.max_ns = max_num_splits;
  dr.batch = batch;
  if (pkv_status st = debug_validate(fn, dr, stream); st != PKV_OK) return st;
  const hipError_t e = pkv::launch_combine(cp, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

int32_t pkv_chunked_kernel_for(int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim) {
  const char* fn = "pkv_chunked_kernel_for";
  if (max_q_len < 1 || num_kv_heads < 1) {
    fail(PKV_ERR_INVALID_ARG, "%s: max_q_len=%d, num_kv_heads=%d", fn, max_q_len, num_kv_heads);
    return -1;
  }
  if (check_group(num_q_heads, num_kv_heads, fn) != PKV_OK) return -1;
  if (head_dim != 64 && head_dim != 128) {
    fail(PKV_ERR_UNSUPPORTED, "%s: head_dim=%d (built: 64, 128)", fn, head_dim);
    return -1;
  }
  return chunked_kernel_of(static_cast<int64_t>(max_q_len) * (num_q_heads / num_kv_heads), head_dim);
}

pkv_status pkv_paged_attention_chunked(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                                       const int32_t* cu_q_lens, int32_t max_q_len, const pkv_cache* cache,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, float scale, float* out, float* out_lse,
                                       void* stream) {
  const char* fn = "pkv_paged_attention_chunked";
  if (pkv_status st = check_cache(cache, fn); st != PKV_OK) return st;
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "%s: num_seqs=%d", fn, num_seqs);
  if (pkv_status st = check_group(num_q_heads, cache->num_kv_heads, fn); st != PKV_OK) return st;
  if (num_seqs == 0) return ok();
  if (q_dtype != PKV_BF16) return fail(PKV_ERR_UNSUPPORTED, "%s: q_dtype=%s (built: BF16)", fn, dtype_name(q_dtype));
  if (cache->kv_dtype == PKV_F32)
    return fail(PKV_ERR_UNSUPPORTED, "%s: F32 cache (built: BF16, I8, FP8)", fn);
  if (q == nullptr || cu_q_lens == nullptr || block_tables == nullptr || context_lens == nullptr || out == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "%s: q/cu_q_lens/block_tables/context_lens/out is NULL", fn);
  if (!aligned16(q) || !aligned16(out)) return fail(PKV_ERR_INVALID_ARG, "%s: q/out not 16-byte aligned", fn);
  if (max_q_len < 1) return fail(PKV_ERR_INVALID_ARG, "%s: max_q_len=%d", fn, max_q_len);
  if (max_blocks_per_seq < 1) return fail(PKV_ERR_INVALID_ARG, "%s: max_blocks_per_seq=%d", fn, max_blocks_per_seq);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  pkv::ChunkedParams p{};
  p.q = q;
  p.k = cache->k;
  p.v = cache->v;
  p.k_scale = cache->k_scale;
  p.v_scale = cache->v_scale;
  p.tables = block_tables;
  p.ctx = context_lens;
  p.cu_q = cu_q_lens;
  p.out = out;
  p.lse = out_lse;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = cache->num_kv_heads;
  p.max_blocks = max_blocks_per_seq;
  p.num_blocks = cache->num_blocks;
  p.max_q_len = max_q_len;
  p.scale_log2 = scale * 1.4426950408889634f;
  pkv::DebugRequest dr;
  dr.tables = block_tables;
  dr.max_blocks = max_blocks_per_seq;
  dr.ctx = context_lens;
  dr.batch = num_seqs;
  dr.num_blocks = cache->num_blocks;
  dr.cu_q = cu_q_lens;
  dr.max_q_len = max_q_len;
  if (pkv_status st = debug_validate(fn, dr, stream); st != PKV_OK) return st;
  const int group = num_q_heads / cache->num_kv_heads;
  const int64_t rows = static_cast<int64_t>(max_q_len) * group;
  const int path = chunked_kernel_of(rows, cache->head_dim);
  if (path != PKV_CHUNKED_TILES) {
    // chunks of a few rows (speculative verification): the decode kernels or
    // the few-row MFMA kernel, with every chunk row of a kv head's query
    // heads on each K/V tile (the MFMA one is built for head dims of 128; with
    // 64, chunks of 5 to 16 rows per kv head take the chunk kernel below)
    pkv::DecodeParams dp{};
    dp.q = q;
    dp.k = cache->k;
    dp.v = cache->v;
    dp.k_scale = cache->k_scale;
    dp.v_scale = cache->v_scale;
    dp.tables = block_tables;
    dp.ctx = context_lens;
    dp.o = out;
    dp.lse = out_lse;
    dp.batch = num_seqs;
    dp.num_q_heads = num_q_heads;
    dp.num_kv_heads = cache->num_kv_heads;
    dp.max_blocks = max_blocks_per_seq;
    dp.num_blocks = cache->num_blocks;
    dp.direct = 1;
    dp.scale_log2 = p.scale_log2;
    dp.cu_q = cu_q_lens;
    dp.max_q_len = max_q_len;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (path == PKV_CHUNKED_ROWS_MFMA) {
      e = pkv::launch_rows_mfma(dp, cache->kv_dtype, cache->head_dim, group, st);
    } else {
      switch (cache->kv_dtype) {
        case PKV_BF16: e = pkv::launch_decode_rows_bf16(dp, cache->head_dim, group, st); break;
        case PKV_I8: e = pkv::launch_decode_rows_i8(dp, cache->head_dim, group, st); break;
        default: e = pkv::launch_decode_rows_fp8(dp, cache->head_dim, group, st); break;
      }
    }
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
  }
  const hipError_t e = pkv::launch_chunked(p, cache->kv_dtype, cache->head_dim, num_q_heads / cache->num_kv_heads,
                                           static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return fail(PKV_ERR_UNSUPPORTED, "%s: this configuration is not built", fn);
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

pkv_status pkv_paged_attention_decode_noalloc(const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                                              const pkv_cache* cache, const int32_t* block_tables,
                                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                                              const int32_t* num_splits, int32_t max_num_splits, float scale,
                                              float* out, float* out_lse, void* stream) {
  const char* fn = "pkv_paged_attention_decode_noalloc";
  if (out == nullptr) return fail(PKV_ERR_INVALID_ARG, "%s: out is NULL (no partials-only mode here)", fn);
  // every argument is checked as for pkv_paged_attention_decode; the
  // library's scratch stands in for the workspace
  bool empty = false;
  if (pkv_status st = check_decode(fn, q, q_dtype, batch, num_q_heads, cache, block_tables, max_blocks_per_seq,
                                   context_lens, num_splits, max_num_splits, scale, out, nullptr, 0, &empty,
                                   /*library_scratch=*/true);
      st != PKV_OK || empty)
    return st;
  const int group = num_q_heads / cache->num_kv_heads;
  const size_t need = noalloc_bytes(batch, num_q_heads, group, cache->head_dim, max_num_splits);
  if (need > kScratchBytes)
    return fail(PKV_ERR_WORKSPACE, "%s: needs %zu bytes of scratch, the library holds %zu per device "
                "(fewer splits or a smaller batch per call, or pkv_paged_attention_decode with a workspace)",
                fn, need, kScratchBytes);
  if (pkv_status st = debug_validate(fn, decode_request(batch, cache, block_tables, max_blocks_per_seq, context_lens,
                                                        num_splits, max_num_splits),
                                     stream);
      st != PKV_OK)
    return st;
  void* ws = nullptr;
  if (need > 0) {
    if (pkv_status st = scratch_address(fn, &ws); st != PKV_OK) return st;
  }
  if (max_num_splits == 0) {
    // the array keeps the last call's contents (another mode's partials may
    // sit where the counters go): clear the counters first
    const int words = static_cast<int>(balanced_counter_bytes(batch, num_q_heads) / sizeof(int32_t));
    hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<int32_t*>(ws), words);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return hip_fail(e, fn);
    return run_balanced_decode(fn, q, q_dtype, batch, num_q_heads, cache, block_tables, max_blocks_per_seq,
                               context_lens, scale, out, out_lse, ws, stream);
  }
  return run_split_decode(fn, q, q_dtype, batch, num_q_heads, cache, block_tables, max_blocks_per_seq, context_lens,
                          num_splits, max_num_splits, scale, out, out_lse, ws, nullptr, stream);
}

}  // extern "C"
