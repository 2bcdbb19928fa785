/*
 * pa_measure.h -- ceiling kernels of libpa, used to measure the HBM bandwidth
 * a streaming kernel reaches on this device, next to the attention step.
 *
 * The method's decode step reads every cached K/V byte of each request once
 * per new token and is bound by memory bandwidth (Inside vLLM summary,
 * techfeed.io, section "エンジンの中核：スケジューラとKVキャッシュ管理"), so
 * the decode kernel is judged against what a plain streaming kernel achieves
 * on the same device: a copy (bytes read + bytes written), a read-only
 * reduction, and a gather of whole pages in random order.  The chunk kernel
 * is compute-bound and is judged against a matrix-core loop.
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

/* Reads npages whole pages of page_bytes bytes each, page pages[i] (device
 * int32 array) at src + pages[i] * page_bytes, in the given order, and writes
 * one 32-bit XOR per workgroup into out (at least 65536 uint32 entries).
 * Page numbers are clamped into [0, src_pages), so nothing outside the
 * src_pages * page_bytes buffer is read.  With a random permutation of 4 KB
 * pages this is the access pattern of the decode step (every (block, kv head)
 * page of K or V is a 4 KB run at a random place in the pool), without its
 * arithmetic.  page_bytes must be a positive multiple of 1024; src 16-byte
 * aligned. */
int pa_measure_gather(const void* src, int64_t src_pages, const int32_t* pages, int64_t npages,
                      int32_t page_bytes, uint32_t* out, void* stream);

/* bf16 matrix-core ceiling: two workgroups of four wavefronts per CU, each
 * wavefront running `iters` rounds of four independent 32x32x16 bf16 products
 * (v_mfma_f32_32x32x16_bf16) on register operands with no memory traffic; the
 * chunk kernel's products are these.  Writes one float per wavefront into out
 * (device, at least 65536 entries) and the launch's flop count (2 per
 * multiply-add) into *flops (host).  iters must be positive. */
int pa_measure_mfma(int32_t iters, float* out, int64_t* flops, void* stream);

/* The same matrix-core loop on operands spread like N(0,1) data (random sign,
 * exponent 2^-3 .. 2^0 and mantissa per bf16 element, four operand sets per
 * lane taken in turn so every product sees new inputs).  The products' power,
 * and with it the clock the chip holds, depends on how much their inputs
 * toggle; the chunk kernel multiplies such data.  Same outputs as
 * pa_measure_mfma; iters must be a positive multiple of 4. */
int pa_measure_mfma_random(int32_t iters, float* out, int64_t* flops, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PA_MEASURE_H */
