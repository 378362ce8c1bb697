/*
 * hist_bench.h -- measurement-only kernels of libpca_hist.so.
 *
 * These are not part of the histogram path. They exist so that a benchmark
 * can put the histogram's numbers next to the machine's own ceilings (HBM
 * stream read, copy, LDS atomic rates) and next to the one alternative the
 * page names.
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

/* LDS atomic rate (calibration of the on-chip ceiling the histogram kernels
 * meet). Launches one 1024-thread workgroup per CU (128 KiB of LDS each);
 * every wave issues iters * 16 LDS atomic adds of 1 into a 32,768-word array,
 * with the addresses of one instruction laid out by pattern:
 *   0  64 consecutive words (no bank conflict)
 *   1  random words (a fixed pseudo-random pattern per instruction)
 *   2  all 64 lanes on one word
 *   3  eight groups of eight lanes, one word per group
 * with_return != 0 uses the returning form (ds_add_rtn_u32), as the 16-bit
 * counters do. The caller times the call on its stream; the rate per CU is
 * (CUs * 16 waves * iters * 16) instructions over that time. sink receives
 * one word per workgroup (so the work cannot be dropped) and must hold at
 * least the device's CU count (sink_words). */
hist_status_t hist_bench_lds_atomic(uint32_t pattern, uint32_t with_return, uint32_t iters,
                                   uint32_t *sink, uint32_t sink_words, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PCA_HIST_BENCH_H */
