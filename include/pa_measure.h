/*
 * pa_measure.h -- ceiling kernels of libpa, used to measure the HBM bandwidth
 * a streaming kernel reaches on this device, next to the attention step.
 *
 * The method's decode step reads every cached K/V byte of each request once
 * per new token and is bound by memory bandwidth (Inside vLLM summary,
 * techfeed.io, section "エンジンの中核：スケジューラとKVキャッシュ管理"), so
 * the decode kernel is judged against what a plain streaming kernel achieves
 * on the same device: a copy (bytes read + bytes written) and a read-only
 * reduction.
 *
 * Same conventions as pa.h: device pointers, `stream` is a hipStream_t (NULL =
 * null stream), calls only enqueue work, errors are negative pa_status codes
 * with pa_last_error() set.
 */
#ifndef PA_MEASURE_H
#define PA_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[i] = src[i] for bytes bytes with 16-byte nontemporal loads and stores.
 * bytes must be a positive multiple of 16 and both pointers 16-byte aligned;
 * the buffers must not overlap. */
int pa_measure_copy(void* dst, const void* src, size_t bytes, void* stream);

/* Reads bytes bytes of src (16-byte loads) and writes one 32-bit XOR of all of
 * them per workgroup into out (device, at least 65536 uint32 entries), so the
 * reads cannot be elided.  Same size and alignment rules as pa_measure_copy. */
int pa_measure_read(const void* src, size_t bytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PA_MEASURE_H */
