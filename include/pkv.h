/*
 * pkv.h -- C ABI of the paged-KV attention library for AMD MI355X (gfx950).
 *
 * The library computes attention of each request's new query rows over its
 * KV history, with the history held in fixed-size blocks of a shared pool and
 * addressed through a per-request block table (page "S20 · The Complete
 * Engine", section "Core idea": step 2 gives each request a block_table of
 * physical block ids). A decode step appends the new token's K and V to the
 * cache and then attends its single query over the whole history (page
 * "llm-inference" on shehab-ashraf.github.io, section "KV Cache", subsection
 * "The Idea"). Query heads share KV heads in contiguous groups (GQA, course
 * README "Build an LLM Inference Engine From Scratch", section "The
 * curriculum", S03). Softmax is computed online and long contexts are split
 * into ranges merged by log-sum-exp (same README, S12, and its claim s12 in
 * section "The code asserts its own claims").
 *
 * Conventions for every entry point:
 *  - Every pointer argument is a DEVICE pointer owned by the caller, except the
 *    pkv_cache descriptor itself, which is read on the host during the call.
 *    The library never allocates, frees or synchronises; it only launches
 *    kernels on `stream` (a hipStream_t; NULL = the null stream) and returns.
 *  - Host-visible arguments (sizes, dtypes, pointers' null-ness, alignment) are
 *    checked before any launch. On failure the call returns a negative
 *    pkv_status, launches nothing, and pkv_last_error() describes the problem
 *    (text is per calling thread, valid until that thread's next call).
 *  - Values that live in device memory (context_lens, block_tables,
 *    slot_mapping, num_splits, cu_q_lens) are NOT read on the host. Kernels
 *    never read or write outside the buffers described here, whatever those
 *    values are: a block id outside [0, num_blocks), a context length beyond
 *    max_blocks_per_seq * block_size, or a split count outside
 *    [1, max_num_splits] turns that sequence's outputs into NaN; a slot outside
 *    [0, num_blocks * block_size) is skipped like a negative slot.
 *  - Debug mode: with the environment variable PKV_DEBUG=1 (read at every
 *    call), the calls that read such values first run a validation pass over
 *    them on `stream`, WAIT for it (a host synchronisation, so not usable under
 *    graph capture), and return PKV_ERR_INVALID_ARG without launching the
 *    computation if an entry is bad: a context length outside
 *    [0, max_blocks_per_seq * block_size], a block id outside [0, num_blocks)
 *    among a sequence's first ceil(n / block_size) entries, a split count
 *    outside [1, max_num_splits], cu_q_lens[0] != 0, a decreasing cu_q_lens, a
 *    chunk longer than max_q_len or than its context, a slot past the pool, or
 *    (decode with append) a slot that is not the slot of token n - 1.
 *    pkv_last_error() names the first offending entry. The validation's
 *    finding lives in a fixed device word per GPU, so debug-mode calls that
 *    overlap on one GPU may report each other's findings.
 *  - Launch failures reported by the HIP runtime return PKV_ERR_HIP.
 *  - Calls on one stream run in order; calls on different streams that write
 *    the same buffers race.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pkv_status;
#define PKV_OK 0
#define PKV_ERR_INVALID_ARG (-1)  /* null pointer, bad size, bad layout */
#define PKV_ERR_UNSUPPORTED (-2)  /* valid but not built: head_dim, block_size, dtype combination */
#define PKV_ERR_WORKSPACE (-3)    /* workspace missing or smaller than pkv_decode_workspace_bytes() */
#define PKV_ERR_HIP (-4)          /* the HIP runtime refused a launch */

/* element types */
#define PKV_F32 0   /* IEEE binary32 */
#define PKV_BF16 1  /* bfloat16 (upper half of a binary32) */
#define PKV_I8 2    /* int8 code with a float32 scale per (token, kv head) */
#define PKV_FP8 3   /* OCP FP8 E4M3 code with a float32 scale per (token, kv head) */

/*
 * The KV block pool.
 *   k, v       : [num_blocks][num_kv_heads][block_size][head_dim] row-major,
 *                elements of kv_dtype. One (block, head) tile is contiguous.
 *   k_scale,
 *   v_scale    : [num_blocks][num_kv_heads][block_size] float32 for PKV_I8
 *                and PKV_FP8, NULL otherwise. Stored value = value(code) * scale,
 *                value(code) the integer for I8, the E4M3 value for FP8.
 * Token t of a sequence lives in block block_table[t / block_size] at offset
 * t % block_size; slot s of the pool is block s / block_size, offset
 * s % block_size.
 * Built: block_size == 16; head_dim in {64, 128}; k and v 16-byte aligned.
 */
typedef struct pkv_cache {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t kv_dtype;
  void* k;
  void* v;
  float* k_scale;
  float* v_scale;
} pkv_cache;

/* Text of the last error on this thread ("" if none). */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

/*
 * reshape_and_cache: write new K/V rows into their pool slots (the "append"
 * of the decode step; page "llm-inference", section "KV Cache").
 *   k_new, v_new : [num_tokens][num_kv_heads][head_dim] of src_dtype, 16-byte aligned.
 *   slot_mapping : int64 [num_tokens]; slot < 0 skips the row.
 *   Float caches (F32, BF16) copy the bytes unchanged and need
 *   src_dtype == kv_dtype. The I8 cache takes F32 or BF16 rows and quantizes
 *   each (token, head) row symmetrically: amax = max |x| (float32),
 *   scale = amax / 127 (IEEE float32 division; amax == 0 gives scale 1),
 *   code = clamp(rint(x / scale), -127, 127) with an IEEE division and
 *   round-half-to-even (course README, curriculum S08 quantization).
 *   The FP8 cache (course README, curriculum S00 bf16/fp8) takes F32 or BF16
 *   rows and scales them the same way with scale = amax / 448; code = the OCP
 *   E4M3 value nearest to the float32 quotient x / scale, ties to the even
 *   code, saturating at 448 (E4M3: sign, 4 exponent bits with bias 7, 3
 *   mantissa bits, subnormals m * 2^-9, S.1111.111 NaN, no infinities).
 *   Two rows with the same slot in one call: undefined which one lands.
 *   Writing a chunk in pieces gives the same bytes as writing it at once
 *   (course README, claim s11).
 */
pkv_status pkv_reshape_and_cache(const void* k_new, const void* v_new, int32_t src_dtype,
                                 const int64_t* slot_mapping, int32_t num_tokens,
                                 const pkv_cache* cache, void* stream);

/*
 * Bytes of device workspace pkv_paged_attention_decode needs:
 *   max_num_splits == 0 : the balanced mode's arrival counters (batch *
 *                         num_q_heads int32, rounded up to 256) followed by
 *                         its partial slots (2048 x 2 x num_q_heads x
 *                         (head_dim + 1) float32). The counters must be zero
 *                         before the first call on a workspace; every call
 *                         leaves them zero.
 *   max_num_splits == 1 : 0 (the partial pass writes `out` directly);
 *   otherwise           : batch * max_num_splits * num_q_heads * (head_dim + 1) * 4,
 *                         rounded up to 256. Layout: o_part float32
 *                         [batch][max_num_splits][num_q_heads][head_dim], then
 *                         lse_part float32 [batch][max_num_splits][num_q_heads].
 * Returns 0 for non-positive arguments.
 */
size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_num_splits);

/*
 * The decode mode to use when the caller has no split plan of its own: the
 * max_num_splits value to pass to pkv_paged_attention_decode with
 * num_splits == NULL. Host-only; touches no device.
 *   max_blocks_per_seq <= 64 : 1, one split per sequence. Each workgroup
 *                              streams one (sequence, kv head), at most 16
 *                              blocks per wavefront, with no merge.
 *   otherwise                : 0, the balanced mode (its workspace from
 *                              pkv_decode_workspace_bytes(..., 0)), which
 *                              evens out long and short sequences.
 * Every choice gives the same result up to rounding; this one only picks the
 * faster launch on MI355X for the table width (block sizes of 16 tokens).
 * Returns -1 (and sets pkv_last_error) for max_blocks_per_seq < 1.
 */
int32_t pkv_decode_default_max_num_splits(int32_t max_blocks_per_seq);

/*
 * paged_attention_decode: one query row per sequence over its paged history,
 * split-K (flash-decoding) with a log-sum-exp merge.
 *   q            : [batch][num_q_heads][head_dim] of q_dtype (F32 or BF16), 16-byte aligned.
 *   cache        : the pool (see pkv_cache); num_q_heads % num_kv_heads == 0,
 *                  num_q_heads / num_kv_heads in {1, 2, 4, 8}.
 *   block_tables : int32 [batch][max_blocks_per_seq].
 *   context_lens : int32 [batch]; n_b >= 0 tokens, counting the new one.
 *   num_splits   : int32 [batch]; ns_b in [1, max_num_splits]. Split s of
 *                  sequence b covers tokens [s*tps, min(n_b, (s+1)*tps)) with
 *                  tps = block_size * ceil(ceil(n_b / ns_b) / block_size);
 *                  every choice gives the same result up to rounding.
 *                  max_num_splits == 0 (num_splits NULL) selects the balanced
 *                  mode: the library deals the batch's (sequence, kv head,
 *                  block) tiles to the GPU's wavefronts in equal contiguous
 *                  ranges and merges cut sequences within the same launch, so
 *                  the split is chosen by the data, not the caller. Calls that
 *                  share a workspace must not overlap (one stream is fine).
 *   scale        : multiplies q . k before the softmax.
 *   out          : float32 [batch][num_q_heads][head_dim]:
 *                  sum_t softmax_t(scale * q . k_t) v_t over t < n_b.
 *                  With max_num_splits > 1, out == NULL runs the partial
 *                  pass only: the workspace then holds every split's
 *                  (o_part, lse_part) in the layout pkv_lse_combine reads,
 *                  e.g. to merge partials computed elsewhere.
 *   out_lse      : float32 [batch][num_q_heads] natural-log softmax
 *                  denominator, log sum_t exp(scale * q . k_t); may be NULL.
 *   n_b == 0 gives out = 0 and lse = -inf.
 *   workspace    : device buffer of at least
 *                  pkv_decode_workspace_bytes(batch, num_q_heads, head_dim,
 *                  max_num_splits) bytes (may be NULL when that is 0).
 */
pkv_status pkv_paged_attention_decode(const void* q, int32_t q_dtype, int32_t batch,
                                      int32_t num_q_heads, const pkv_cache* cache,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, const int32_t* num_splits,
                                      int32_t max_num_splits, float scale, float* out,
                                      float* out_lse, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * paged_attention_decode_noalloc: pkv_paged_attention_decode for callers that
 * cannot allocate device memory -- code under HIP graph capture, serving loops
 * that must not allocate, harnesses that forbid hipMalloc. The call allocates
 * nothing and takes no workspace: the split partials, or the balanced mode's
 * counters and partial slots, live in a fixed device array of
 * PKV_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.
 *   Arguments : as pkv_paged_attention_decode without the workspace; `out`
 *               must not be NULL (no partials-only mode).
 *   Limit     : the scratch a call needs must fit the array:
 *                 max_num_splits == 1 : none;
 *                 max_num_splits  > 1 : batch * max_num_splits * num_q_heads *
 *                                       (head_dim + 1) * 4 bytes (rounded up to 256);
 *                 max_num_splits == 0 : batch * num_q_heads * 4 (rounded up to
 *                                       256) + 2048 * 2 * (num_q_heads /
 *                                       num_kv_heads) * (head_dim + 1) * 4 bytes.
 *               A larger call returns PKV_ERR_WORKSPACE and launches nothing.
 *   Sharing   : every call on one GPU uses that GPU's one array. Calls that
 *               overlap on one GPU (different streams, or different threads
 *               without ordering) race and give undefined results; calls on
 *               one stream are fine. The balanced mode clears its counters
 *               at the start of each call (a small extra launch).
 *   Set-up    : the first call on a device looks up the array's device
 *               address there (that device must be current); a failure
 *               returns PKV_ERR_HIP.
 * Results equal pkv_paged_attention_decode's bit for bit (the same kernels).
 */
#define PKV_NOALLOC_SCRATCH_BYTES (((size_t)48) << 20)
pkv_status pkv_paged_attention_decode_noalloc(const void* q, int32_t q_dtype, int32_t batch,
                                              int32_t num_q_heads, const pkv_cache* cache,
                                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                                              const int32_t* context_lens, const int32_t* num_splits,
                                              int32_t max_num_splits, float scale, float* out,
                                              float* out_lse, void* stream);

/*
 * paged_attention_decode_append: pkv_reshape_and_cache of the step's new
 * rows followed by pkv_paged_attention_decode, in one pass (page
 * "llm-inference" on shehab-ashraf.github.io, section "KV Cache", subsection
 * "The Idea": the step's k, v are appended, then its q attends over the whole
 * history). The wavefront that reads a sequence's last block first writes
 * that sequence's new K/V rows to their slot, with the same arithmetic as
 * pkv_reshape_and_cache (int8 codes and scales bit for bit), and waits for the
 * stores before it reads the block.
 *   k_new, v_new : [batch][num_kv_heads][head_dim] of src_dtype, 16-byte
 *                  aligned; one new token per sequence. src_dtype as for
 *                  pkv_reshape_and_cache.
 *   slot_mapping : int64 [batch]; slot of sequence b's new token, which must
 *                  be the slot of its position n_b - 1 in its block table
 *                  (otherwise the result is unspecified). Slots outside the
 *                  pool are skipped.
 *   the rest     : as pkv_paged_attention_decode, split mode only:
 *                  max_num_splits == 0 returns PKV_ERR_UNSUPPORTED.
 * Sequences whose split count is invalid (their outputs are NaN) may be
 * left without their new rows written.
 */
pkv_status pkv_paged_attention_decode_append(const void* k_new, const void* v_new, int32_t src_dtype,
                                             const int64_t* slot_mapping, const void* q, int32_t q_dtype,
                                             int32_t batch, int32_t num_q_heads, const pkv_cache* cache,
                                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                                             const int32_t* context_lens, const int32_t* num_splits,
                                             int32_t max_num_splits, float scale, float* out, float* out_lse,
                                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attention_chunked: causal query chunks against their cached prefix
 * (chunked prefill, course README curriculum S11; the chunk's own K/V must
 * already be in the cache, written by pkv_reshape_and_cache).
 *   q            : BF16 [total_q][num_q_heads][head_dim], total_q = cu_q_lens[num_seqs].
 *   cu_q_lens    : int32 [num_seqs + 1], non-decreasing, cu_q_lens[0] == 0;
 *                  sequence i owns rows [cu_q_lens[i], cu_q_lens[i+1]).
 *   max_q_len    : an upper bound of every chunk length (sizes the grid).
 *   context_lens : int32 [num_seqs]; n_i counts the prefix and the chunk.
 *   Row r of chunk i (length L_i) sits at position n_i - L_i + r and attends
 *   the cached tokens t <= n_i - L_i + r (bottom-right aligned causal mask).
 *   out          : float32 [total_q][num_q_heads][head_dim]; out_lse float32
 *                  [total_q][num_q_heads] or NULL (natural log).
 *   Cache dtypes: BF16, I8 or FP8; head_dim 64 or 128; GQA group size in
 *   {1, 2, 4, 8}.
 *   A chunk longer than max_q_len or than its context yields NaN rows.
 * Chunks of a few rows per kv head (max_q_len * (num_q_heads /
 * num_kv_heads) = R) run on decode-shaped kernels, one workgroup per
 * (sequence, kv head)
 * streaming the sequence once with every chunk row of the group's query heads
 * against each K/V tile:
 *   R <= 2 (head_dim 128), R <= 4 (head_dim 64):
 *                 fp32 FMAs and dot products (the decode's arithmetic);
 *   2 < R <= 16 : (head_dim 128) 16x16 bf16 MFMAs for QK^T and PV, the weights split into a
 *                 bf16 high part and residual (~2^-17), 8-bit codes converted
 *                 to bf16 exactly;
 * e.g. speculative verification of up to 8 draft rows with 2 query heads per
 * kv head. Longer chunks (with head_dim 64: from 5 rows per kv head) run on
 * the 128-row MFMA kernel.
 * Arithmetic: QK^T with bf16 MFMA (exact products, fp32 sums); softmax in
 * fp32. The PV product's weights are bf16 pairs (a high part and its
 * residual, ~2^-17) over a BF16 cache, and fp16 (rounded once, 2^-12, with
 * the V scale folded in) over an I8 or FP8 cache, whose codes are exact in
 * fp16. The output therefore agrees with exact attention over the cached
 * values to about 2^-12 of |V| on rows that see few keys (less as more keys
 * average), for V scales of any magnitude.
 */
pkv_status pkv_paged_attention_chunked(const void* q, int32_t q_dtype, int32_t num_seqs,
                                       int32_t num_q_heads, const int32_t* cu_q_lens,
                                       int32_t max_q_len, const pkv_cache* cache,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, float scale, float* out,
                                       float* out_lse, void* stream);

/*
 * chunked_kernel_for: which kernel pkv_paged_attention_chunked runs for a call
 * of this shape, by the rule above (host only: no GPU, no allocation):
 *   PKV_CHUNKED_DECODE_ROWS : the decode core, R <= 2 (head_dim 128) or
 *                             R <= 4 (head_dim 64);
 *   PKV_CHUNKED_ROWS_MFMA   : the 16x16 MFMA few-row kernel, 2 < R <= 16
 *                             (head_dim 128);
 *   PKV_CHUNKED_TILES       : the 128-row MFMA kernel, every longer chunk.
 * R = max_q_len * (num_q_heads / num_kv_heads). Returns -1 (and sets
 * pkv_last_error) for a shape the entry point rejects: max_q_len < 1,
 * num_kv_heads < 1, a GQA group outside {1, 2, 4, 8}, head_dim not 64 or 128.
 */
#define PKV_CHUNKED_DECODE_ROWS 1
#define PKV_CHUNKED_ROWS_MFMA 2
#define PKV_CHUNKED_TILES 3
int32_t pkv_chunked_kernel_for(int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim);

/*
 * lse_combine: merge split partials (each normalised by its own denominator)
 * by log-sum-exp: M = max_s lse_s over splits with lse_s > -inf,
 * w_s = exp(lse_s - M), out = sum_s w_s o_s / sum_s w_s, lse = M + log sum_s w_s.
 * No live split gives out = 0, lse = -inf.
 *   o_part   : float32 [batch][max_num_splits][num_q_heads][head_dim]
 *   lse_part : float32 [batch][max_num_splits][num_q_heads]
 *   num_splits : int32 [batch]; splits s >= num_splits[b] are not read.
 *   out, out_lse : as in pkv_paged_attention_decode (out_lse may be NULL).
 * This is the second pass of pkv_paged_attention_decode, exported so that
 * partials from several sources can be merged.
 */
pkv_status pkv_lse_combine(const float* o_part, const float* lse_part, int32_t batch,
                           int32_t num_q_heads, int32_t head_dim, int32_t max_num_splits,
                           const int32_t* num_splits, float* out, float* out_lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
