/*
 * pkv_measure.h -- measurement aids of the paged-KV attention library (not
 * part of the attention path).
 *
 * Decode attention is bound by HBM reads: its time goes to streaming the KV
 * cache once (page "llm-inference" on shehab-ashraf.github.io, section "KV
 * Cache": decode is memory-bound; course README "Build an LLM Inference
 * Engine From Scratch", curriculum S06/S12). Its speed is best compared with
 * what a kernel that only reads the same number of bytes reaches on the same
 * machine in the same run, launch and drain included.
 */
#ifndef PKV_MEASURE_H
#define PKV_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * stream_read: read every byte of src once (16-byte non-temporal loads, the
 * decode kernels' load width and cache policy) and nothing else, in one launch
 * on `stream`.
 *   src   : device buffer, 16-byte aligned; bytes a multiple of 16, > 0.
 *   sink  : device buffer of at least 4 * pkv_stream_read_workgroups(bytes)
 *           bytes; written only in the (practically impossible) case that a
 *           workgroup's XOR of the words it read equals 0x9E3779B9, which
 *           keeps the loads from being optimised away. Its contents carry no
 *           meaning.
 * Returns PKV_ERR_INVALID_ARG for a NULL or misaligned pointer or a bad size,
 * PKV_ERR_HIP if the launch fails. Asynchronous; allocates nothing.
 */
pkv_status pkv_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Workgroups pkv_stream_read launches for `bytes` (0 for bytes == 0). */
int32_t pkv_stream_read_workgroups(size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* PKV_MEASURE_H */
