/*
 * fq_bench.h -- measurement helpers exported by libfq.so for the benchmark.
 *
 * These are not steps of the method: they set up and bound the timing of the
 * entry points in fq.h.  Same conventions as fq.h (device pointers owned by the
 * caller, work enqueued on `stream`, status returned synchronously, nothing
 * allocated, nothing synchronised).
 */
#ifndef FQ_BENCH_H
#define FQ_BENCH_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Cache flush before a cold timing: reads `bytes` (rounded down to a multiple
 * of 16, at least 16) of the 16-byte aligned device buffer `scratch`, so that
 * L2 and the Infinity Cache hold none of a later kernel's inputs.  A read, not a
 * write, so that it leaves no dirty lines whose write-back a later kernel would
 * be billed for.  `sink` (one device uint32_t) is written only for a bit pattern
 * no buffer of the benchmark holds; it keeps the loads alive.
 * FQ_E_INVALID: null or misaligned pointer, bytes < 16. */
int fqb_flush(const void* scratch, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Achievable-bandwidth reference: y[i] = x[i] for i < n, one 16-byte chunk per
 * thread over a grid covering the buffer (the fastest copy shape measured on
 * MI355X).  n % 4 == 0 and 16-byte aligned buffers that do not overlap.
 * FQ_E_INVALID otherwise. */
int fqb_copy_f32(const float* x, float* y, int64_t n, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FQ_BENCH_H */
