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

/* LDS latency (the dependent-access probe of the CREDIT page, "CREDIT:
 * Cost-guided Reduction-reuse with Efficient DSMEM Inter-CTA Tiling", its
 * microbenchmark section: each access waits for the one before). One wave
 * on one CU runs a chain of iters LDS operations, each address depending on
 * the previous operation's returned value:
 *   0  ds_add_rtn_u32 from lane 0 alone
 *   1  ds_add_rtn_u32 from 64 lanes on 64 consecutive words
 *   2  ds_add_rtn_u32 from 64 lanes on one word
 *   3  ds_read_b32 from 64 lanes on consecutive words (load latency)
 * out (device, >= 3 uint64) receives the shader-clock cycles (s_memtime)
 * over the chain, the ticks of the 100 MHz real-time counter over it, and a
 * word that keeps the chain live. iters 1 .. 2^24. */
hist_status_t hist_bench_lds_latency(uint32_t pattern, uint32_t iters, uint64_t *out,
                                     hipStream_t stream);

/* Handoff latency between two workgroups through global memory: the gfx950
 * counterpart of the ping-pong of the page "Hopper DSMEM vs HBM" (its
 * latency test passes a token between two blocks of a cluster and, for
 * comparison, through global memory). Sixteen one-wave workgroups are
 * launched cooperatively (all resident at once); workgroup 0 and workgroup
 * `partner` (1..15) pass a token back and forth iters times, one round trip
 * per iteration, and every workgroup records the XCD it ran on (workgroups
 * are dealt to the XCDs in turn, so partner 8 normally shares workgroup 0's
 * XCD and its L2, and partner 1 does not; the recorded ids say where they
 * ran).
 *   mode 0  the token alone: relaxed device-scope atomic store and load
 *   mode 1  a 256-byte payload stored with plain stores before each token,
 *           the token a release store read with acquire loads; the receiver
 *           checks the payload
 * Every wait gives up after 2^22 polls, so the kernel always ends.
 * flags: device, >= 80 uint32 (zeroed by the call). out: device, >= 20
 * uint64: [0] shader-clock cycles over the iterations, [1] 100 MHz ticks,
 * [2] 1 if a wait gave up, [3] payload words that arrived wrong, [4 + b] the
 * XCD of workgroup b. iters 1 .. 2^20. UNSUPPORTED if the device cannot
 * launch cooperatively. */
hist_status_t hist_bench_handoff(uint32_t partner, uint32_t mode, uint32_t iters, uint32_t *flags,
                                 uint64_t *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PCA_HIST_BENCH_H */
