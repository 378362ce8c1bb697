/*
 * hist_bench.h -- measurement-only kernels of libpca_hist.so.
 *
 * These are not part of the histogram path. They exist so that a benchmark
 * can put the histogram's numbers next to the machine's own ceilings and
 * next to the one alternative the page names.
 *
 * Device pointers, caller-owned, no allocation; every call is asynchronous on
 * stream and returns a status synchronously (codes from hist.h).
 */
#ifndef PCA_HIST_BENCH_H
#define PCA_HIST_BENCH_H

#include "hist.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The fallback the page "Distributed Shared Memory" names in section "When
 * it beats global atomics": no on-chip privatisation, every element is an
 * atomic add straight into global memory, contended across the whole grid.
 * counts is zeroed first, then counts[b] = #{i : input[i] == b}; values
 * outside [0, num_bins) are skipped. n < 2^32. */
hist_status_t hist_bench_global_atomic(uint32_t *counts, const int32_t *input, uint64_t n,
                                       uint32_t num_bins, hipStream_t stream);

/* Stream-read ceiling: reads src[0..bytes) once with 16-byte loads and
 * writes one word per workgroup to sink (so the loads cannot be dropped).
 * src 16-byte aligned, bytes a multiple of 16; sink holds >= 4096 words. */
hist_status_t hist_bench_read(const void *src, uint64_t bytes, uint32_t *sink,
                              hipStream_t stream);

/* Plain copy dst[0..bytes) = src[0..bytes) with 16-byte loads and stores
 * (a kernel of known traffic, for scaling hardware byte counters).
 * Both 16-byte aligned, bytes a multiple of 16, no overlap. */
hist_status_t hist_bench_copy(void *dst, const void *src, uint64_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PCA_HIST_BENCH_H */
