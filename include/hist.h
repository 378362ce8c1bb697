/*
 * hist.h -- partitioned on-chip (LDS) integer histogram for AMD Instinct
 * MI355X (gfx950). C ABI.
 *
 * The operation
 * -------------
 * The page "Distributed Shared Memory", section "The cluster histogram",
 * poses the problem: a histogram with more bins than one block's on-chip
 * memory holds. Its answer partitions the bins so that each cooperating block
 * owns a private slice, accumulates into the owner's slice with on-chip
 * atomics, and after a barrier adds every slice into the global bins. The
 * value that every such schedule reaches is
 *
 *     counts[b] = #{ i in [0, n) : input[i] == b },   0 <= b < num_bins,
 *
 * and that is what hist_run() writes. gfx950 has no cross-CU shared memory,
 * so the partitioning is done by ownership instead of remote atomics: a
 * workgroup owns a range of bins in its LDS (up to 160 KiB of uint32
 * counters) and counts only the elements that fall in it (bin-range
 * ownership); for bin counts far beyond LDS the input is first coarse-
 * scattered by owning range and then counted per owner (two-phase path).
 * Per-range results are merged by exclusive owners: each output bin is
 * written once by one thread, with no global atomics.
 *
 * Readings of the page where it is silent:
 *   - Values outside [0, num_bins) (including negatives) name no bin and are
 *     skipped. The page's kernel requires the bin count to equal the
 *     cluster's capacity exactly (same section); here any num_bins >= 1 works.
 *   - hist_run OVERWRITES counts (the page adds into global bins with
 *     atomics); a repeated call gives the same result. hist_run_accumulate
 *     adds instead.
 *   - Counters are uint32; n must be < 2^32 so no counter can wrap.
 *
 * Memory and ownership
 * --------------------
 * All device buffers belong to the caller. The library never calls
 * hipMalloc or hipFree. A plan borrows a caller-allocated device workspace
 * (size from hist_workspace_size) for its whole lifetime. input is read-only
 * and needs 4-byte alignment only; counts needs 4-byte alignment. counts,
 * input and the workspace must not overlap. One plan runs one hist_run at a
 * time: calls that share a plan must be ordered (e.g. on one stream).
 * hist_run and hist_run_accumulate queue kernel launches only (no memset, no
 * allocation, no synchronisation), so they can be captured into a HIP graph
 * (with timing disabled) and replayed; each replay reads the captured input
 * buffer as it is then.
 *
 * Errors
 * ------
 * Every entry point returns a status synchronously, before any work is
 * queued when arguments are bad; nothing exits, throws or logs. HIST_ERR_HIP
 * reports a launch error seen right after queuing (hipGetLastError); faults
 * during execution surface at the caller's next synchronisation, as in HIP.
 */
#ifndef PCA_HIST_H
#define PCA_HIST_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HIST_OK = 0,
    HIST_ERR_INVALID_ARG = 1, /* null pointer, bad size, overlap, misalignment, wrong device */
    HIST_ERR_UNSUPPORTED = 2, /* no gfx950 device current, or a size beyond what is supported */
    HIST_ERR_WORKSPACE = 3,   /* workspace null or smaller than hist_workspace_size reports */
    HIST_ERR_HIP = 4          /* a HIP call or kernel launch failed */
} hist_status_t;

/* Which schedule hist_run uses. AUTO picks from num_bins. */
typedef enum {
    HIST_PATH_AUTO = 0,
    HIST_PATH_FULL = 1,    /* every workgroup holds all bins in LDS (num_bins <= LDS capacity) */
    HIST_PATH_RANGE = 2,   /* bin-range ownership: R workgroups per input chunk, one range each */
    HIST_PATH_SCATTER = 3, /* two-phase: scatter by owning range, then per-owner LDS histograms */
    HIST_PATH_STREAM = 4   /* one persistent kernel: producers route tiles to the ranges that own
                              their bins and publish them; owners count each range in LDS as the
                              tiles arrive, moving to the ranges with the most work left
                              (num_bins <= 2^21; never chosen by AUTO) */
} hist_path_t;

/* Plan options. Zero-initialise and set only what you want to force;
 * 0 (or -1 for aggregation) means "choose automatically". */
typedef struct {
    int32_t path;       /* hist_path_t */
    int32_t groups;     /* FULL/RANGE: input chunks G; SCATTER: owner workgroups W; STREAM:
                           producer workgroups P (the rest start as owners) */
    int32_t range_bins; /* RANGE: bins per owned range (multiple of 256, <= LDS capacity:
                           40960 with 32-bit counters, 79616 with 16-bit, 155392 with
                           8-bit) */
    int32_t aggregation; /* wave-level duplicate aggregation ahead of the LDS adds, for
                            skewed inputs: -1 auto, 0 off, 1 hot slot (lanes holding the
                            wave's current hot value count in registers), 2 or 4 leader-peel
                            rounds (readfirstlane + ballot, one add per duplicate group) */
    int32_t wg_size;    /* sweep workgroup size: 256, 512 or 1024 (0 = auto) */
    int32_t xcd_map;    /* RANGE: 1 = place a chunk's R owners on one XCD (default),
                           2 = plain order (for measurement) */
    int32_t counter_bits; /* FULL/RANGE LDS counters: 32, 16 (two bins per word) or 8
                             (four bins per word); the packed widths stay exact through
                             carry events and hold 2x or 4x the bins per workgroup */
    int32_t lds_copies;   /* FULL/RANGE with 32-bit counters: interleaved LDS copies of the
                             slice (1, 2, 4, 8, 16; 0 = one); a lane adds to copy lane mod
                             copies, which spreads same-bin lanes of a wave over words and
                             banks at the cost of clearing and summing the copies */
    int32_t pacing;       /* RANGE with R > 1, 1024-thread workgroups and 16- or 8-bit
                             counters, how the R owners of a chunk read it: 0 auto, 1
                             plain loads, each owner at its own pace; 2 the same, with the
                             last wave idle (the paced kernel without its partner); 3..18
                             plain loads, each owner kept within (pacing - 2)
                             batches of the next range's owner by a pacer wave, so that the
                             lines one owner brings into the XCD's L2 serve the other
                             (bounded waits: an owner whose partner does not move stops
                             pacing); 2 and above count with 15 of the 16 waves */
    int32_t spin_log2;    /* STREAM: a wait for a block's tiles gives up after 2^spin_log2
                             polls (0 = 2^22, seconds), sets the plan's give-up flag
                             (hist_plan_check) and moves on; 1..30 */
    int32_t window;       /* SCATTER: a window of HIST_WINDOW_BINS consecutive bins counted in
                             place by the partition workgroups (their elements are never
                             staged), at the heaviest place a 1,024-element sample of each
                             run's input shows: 0 auto (from 2^22 elements, used when the
                             window holds at least a quarter of the sample), 1 never, 2 always.
                             Unless 1, the same sample also names a hot value outside the
                             window (a thirty-second of the sample or more), which the
                             partition counts in registers and never stages. */
} hist_plan_opts_t;

/* Bins of SCATTER's in-place window (hist_plan_opts_t.window). */
#define HIST_WINDOW_BINS 8192

/* Numeric description of a plan (for logs and benchmarks). */
typedef struct {
    int32_t path;          /* hist_path_t actually used */
    int32_t device;        /* HIP device ordinal the plan was made on */
    int32_t cu_count;
    int32_t xcd_count;
    uint32_t num_bins;
    uint32_t range_bins;   /* bins owned by one workgroup (S) */
    uint32_t ranges;       /* R = ceil(num_bins / S) */
    uint32_t groups;       /* FULL/RANGE: G chunks; SCATTER: W owner workgroups */
    uint32_t wg_size;
    int32_t aggregation;
    uint32_t tile_elems;   /* SCATTER: elements per scatter tile */
    uint32_t counter_bits; /* FULL/RANGE: 32, 16 or 8 */
    uint64_t max_n;
    uint64_t workspace_bytes;
    uint64_t max_group_elems; /* FULL/RANGE: the most elements one input chunk may hold;
                                 a call splits its input into at least
                                 ceil(n / max_group_elems) chunks (packed counters: this
                                 bounds each workgroup's carry events) */
    uint32_t event_cap;       /* FULL/RANGE with 8-bit counters: carry-event list entries
                                 per workgroup (the LDS its slice leaves, then 512 more in
                                 the workspace); otherwise 0 */
} hist_plan_info_t;

typedef struct hist_plan_impl hist_plan_t; /* opaque, host memory only */

/* Bytes of device workspace a plan for (num_bins, max_n, opts) needs on the
 * current device. opts may be NULL. Errors: INVALID_ARG for num_bins == 0,
 * max_n >= 2^32, bytes == NULL or bad opts; UNSUPPORTED when the current
 * device is not gfx950 or num_bins exceeds HIST_MAX_BINS. */
hist_status_t hist_workspace_size(uint32_t num_bins, uint64_t max_n,
                                  const hist_plan_opts_t *opts, uint64_t *bytes);

/* Largest num_bins any path supports (2^26 bins, 256 MiB of counts). */
#define HIST_MAX_BINS (1u << 26)

/* Make a plan on the current device for histograms of num_bins bins over
 * inputs of up to max_n elements (the page "Distributed Shared Memory",
 * section "The cluster histogram", sizes its cluster from the bin count; here
 * the plan picks the path, the bins each workgroup owns, the input chunks and
 * the workspace layout from num_bins, max_n and the device).
 *   plan            out: the new plan (host memory; free with hist_plan_destroy);
 *                   *plan is NULL on any error
 *   num_bins        1 .. HIST_MAX_BINS
 *   max_n           largest n a hist_run on this plan may take, < 2^32
 *   opts            NULL, or options to force (see hist_plan_opts_t)
 *   workspace       device memory of at least hist_workspace_size() bytes,
 *                   256-byte aligned, owned by the caller; may be NULL when
 *                   that size is 0. The plan keeps the pointer until
 *                   hist_plan_destroy and overwrites its contents on every run.
 *   workspace_bytes its size in bytes
 * Errors: INVALID_ARG for a null plan, num_bins == 0, max_n >= 2^32, bad
 * opts or a misaligned workspace; UNSUPPORTED when the current device is not
 * gfx950 or num_bins > HIST_MAX_BINS; WORKSPACE when workspace is NULL or
 * smaller than the plan needs. Host-only: queues no device work. */
hist_status_t hist_plan(hist_plan_t **plan, uint32_t num_bins, uint64_t max_n,
                        const hist_plan_opts_t *opts, void *workspace, uint64_t workspace_bytes);

/* The same call as hist_plan under an older name (identical arguments,
 * behaviour and errors). */
hist_status_t hist_plan_create(hist_plan_t **plan, uint32_t num_bins, uint64_t max_n,
                               const hist_plan_opts_t *opts, void *workspace,
                               uint64_t workspace_bytes);

/* Queue the histogram of input[0..n) into counts[0..num_bins) on stream
 * (0 = the null stream). num_bins must equal the plan's and n <= max_n.
 * n == 0 is valid and writes num_bins zeros. input may be NULL when n == 0.
 * The call is asynchronous; counts is complete when the stream reaches it. */
hist_status_t hist_run(hist_plan_t *plan, uint32_t *counts, const int32_t *input, uint64_t n,
                       uint32_t num_bins, hipStream_t stream);

/* Like hist_run, but adds the histogram into counts instead of overwriting it:
 * counts[b] += #{ i in [0, n) : input[i] == b }, modulo 2^32. This is the
 * page's own flush semantics (each block adds its slice into the global
 * bins, section "The cluster histogram"), and it lets an input be fed in
 * chunks: successive calls on the pieces of an input leave the histogram of
 * the whole. Each bin is still read and written by one exclusive owner, with
 * no atomics. n == 0 queues nothing. Arguments and errors as for hist_run. */
hist_status_t hist_run_accumulate(hist_plan_t *plan, uint32_t *counts, const int32_t *input,
                                  uint64_t n, uint32_t num_bins, hipStream_t stream);

/* The histogram with no device allocation at all, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * and harnesses that forbid hipMalloc. It computes what hist_run computes,
 * counts[b] = #{ i in [0, n) : input[i] == b }, with the same kernels: it
 * plans like hist_plan with default options for (num_bins, max_n = n) on the
 * current device, and takes the workspace from a device array the library
 * holds, HIST_STATIC_SCRATCH_BYTES on each device it runs on, kept until the
 * process ends. When the default plan's one-pass workspace (its partial rows)
 * does not fit, it counts the input in fewer, larger chunks.
 *   counts    device, num_bins uint32, overwritten; 4-byte aligned
 *   input     device, n int32, read-only; 4-byte aligned; NULL allowed when n == 0
 *   n         < 2^32
 *   num_bins  1 .. HIST_MAX_BINS
 *   stream    the stream to queue on (0 = the null stream)
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * call) and queues kernels only. Every call on a device shares that device's
 * array, which keeps the last call's contents: calls that overlap on one
 * device (on different streams, or from several threads without ordering)
 * race and give wrong counts. Calls ordered on one stream are safe.
 * Errors: INVALID_ARG as hist_run (null counts, NULL input with n > 0,
 * num_bins == 0, n >= 2^32, overlapping buffers, misalignment);
 * UNSUPPORTED when the current device is not gfx950 or num_bins >
 * HIST_MAX_BINS; WORKSPACE, before anything is queued, when the plan for
 * (num_bins, n) needs more than HIST_STATIC_SCRATCH_BYTES even in fewer
 * chunks. On an MI355X every n < 2^32 fits up to 79,616 bins; up to 318,464
 * bins at least 2^26 elements fit (8-bit counters need a minimum number of
 * chunks, each a partial row); on the two-phase path (more bins) the routed
 * slots take about 2n bytes, and at least 2^25 elements fit up to 2^20 bins,
 * 2^23 up to 2^24 bins. HIP when a launch fails. */
#define HIST_STATIC_SCRATCH_BYTES (128ull << 20)
hist_status_t hist_run_static(uint32_t *counts, const int32_t *input, uint64_t n,
                              uint32_t num_bins, hipStream_t stream);

/* Fill *info. */
hist_status_t hist_plan_info(const hist_plan_t *plan, hist_plan_info_t *info);

/* A device described by its numbers, for hist_plan_preview. */
typedef struct {
    int32_t cu_count;              /* compute units (MI355X: 256) */
    int32_t xcd_count;             /* L2 domains; cu_count is a multiple of it (MI355X: 8) */
    uint32_t lds_bytes;            /* LDS one workgroup may use, 65,536 .. 163,840 (MI355X:
                                      163,840) */
    uint32_t sweep_waves_per_simd; /* sweep waves one SIMD holds at once as far as registers
                                      allow (this library on gfx950: 6); 0 = no limit */
} hist_device_desc_t;

/* The plan hist_plan would make for (num_bins, max_n, opts) on the
 * described device, computed on the host with no device present: the same
 * path, counter width, ranges, chunks and workspace bytes, for capacity
 * planning and for tests of the planning rules. info->device is -1.
 * Errors: as hist_workspace_size, and HIST_ERR_INVALID_ARG for a null
 * argument or a device description outside the stated bounds. */
hist_status_t hist_plan_preview(const hist_device_desc_t *dev, uint32_t num_bins, uint64_t max_n,
                                const hist_plan_opts_t *opts, hist_plan_info_t *info);

/* Measured schedule choice.
 *
 * AUTO picks a schedule from num_bins alone, from sweeps over uniform and
 * Zipf inputs; the best schedule also depends on the data (a skewed input
 * can favour the two-phase path with the hot slot where a uniform one
 * favours bin-range ownership). hist_tune times the candidate schedules on
 * the caller's own input and reports the fastest, following the cost-guided
 * selection of "CREDIT: Cost-guided Reduction-reuse with Efficient DSMEM
 * Inter-CTA Tiling" (its cost model section, Eq. 7: a rate measured at the
 * same shape replaces a device peak). Its model predicts one schedule's
 * time from another's; here every candidate is cheap to run, so each is
 * measured directly.
 *
 * Candidates, in this order (those a bin count does not allow are skipped):
 * FULL with 32-, 16- and 8-bit counters; RANGE with 32-, 16- (plain and hot
 * slot) and 8-bit counters (plain and hot slot); SCATTER plain and with the
 * hot slot. Every other option is left to the plan. */
#define HIST_TUNE_MAX_ENTRIES 10

typedef struct {
    hist_plan_opts_t opts; /* the options naming the schedule (path, counter_bits,
                              aggregation; the rest 0) */
    double ms;             /* mean milliseconds per hist_run over reps runs; -1 if not run */
    int32_t status;        /* HIST_OK if measured; HIST_ERR_UNSUPPORTED when the bin count
                              does not allow it; HIST_ERR_WORKSPACE when its plan needs more
                              workspace than was given */
    int32_t reserved;
} hist_tune_entry_t;

/* Bytes of device workspace hist_tune needs to try every candidate for
 * (num_bins, max_n): the largest hist_workspace_size among them. Errors as
 * hist_workspace_size. */
hist_status_t hist_tune_workspace_size(uint32_t num_bins, uint64_t max_n, uint64_t *bytes);

/* Time every candidate schedule for (num_bins, max_n) on input[0..n): for
 * each, a plan on workspace, one untimed hist_run, then reps hist_runs
 * between two HIP events on stream. Writes the fastest candidate's options to
 * *best (pass them to hist_plan with the same num_bins and max_n), and
 * the candidates' entries, in the order above, to entries[0..*count) (at most
 * capacity of them; entries may be NULL when capacity is 0). counts (device,
 * num_bins uint32) receives each run's output; on success it holds the
 * histogram of input. Synchronous: returns after the last run completes. The
 * workspace's contents are overwritten. Errors: INVALID_ARG for a null input,
 * counts or best, n == 0, n > max_n, reps outside 1..1000, or a null count
 * with capacity > 0; UNSUPPORTED as hist_workspace_size; WORKSPACE when no
 * candidate's plan fits the workspace; HIP when a run or an event fails. */
hist_status_t hist_tune(uint32_t num_bins, uint64_t max_n, const int32_t *input, uint64_t n,
                        uint32_t *counts, void *workspace, uint64_t workspace_bytes,
                        uint32_t reps, hipStream_t stream, hist_plan_opts_t *best,
                        hist_tune_entry_t *entries, uint32_t capacity, uint32_t *count);

/* Predicted schedule choice: a cost model, not a measurement.
 *
 * The cost-guided selection of "CREDIT: Cost-guided Reduction-reuse with
 * Efficient DSMEM Inter-CTA Tiling" (its cost model section, Eq. 7-9)
 * predicts whether a schedule pays at a given shape from one baseline timing
 * at that shape, primitive rates measured once per device, and a static
 * account of each schedule's traffic, without timing the schedules. Here:
 *   - the baseline is a stream read of the caller's input: its achieved rate
 *     prices every pass over the input (Eq. 7 replaces a device peak with the
 *     rate achieved at the same shape);
 *   - the primitives (hist_model_calib_t) come from the library's probes:
 *     copy rate, LDS atomics per wave instruction on random words and the
 *     surcharge per same-word lane, one launch, a sweep's fixed cost, one
 *     8-bit carry event, the two-phase path's fixed cost;
 *   - the traffic: FULL and RANGE read the input once per owned range (each
 *     pass priced as a full read: cache hits between a chunk's owners are
 *     not credited) and merge G partial rows; SCATTER reads the input,
 *     writes and reads back 2-byte slots;
 *   - a sample of the input gives what the data decides: same-word lanes per
 *     LDS instruction, expected carry events of packed counters at the
 *     plan's chunk size, and the hot value the wave hot slot takes.
 * A schedule's time is its fixed costs + max(passes, LDS atomics) + carry
 * events + merge.
 *
 * Candidates, in their order of preference on equal predictions: FULL with
 * 16-, 8- and 32-bit counters; RANGE with 8-, 16- and 32-bit counters (2,048
 * bins and up); SCATTER with the hot slot, then without. */
#define HIST_MODEL_MAX_ENTRIES 8

typedef struct {
    double read_gbps;        /* HBM stream read, GB/s (hist_select replaces it with the rate
                                measured on the caller's input) */
    double copy_gbps;        /* copy, read + write bytes per second / 1e9 */
    double clock_ghz;        /* shader clock */
    double lds_cycles;       /* one wave instruction of LDS atomics on random words, cycles
                                of one CU */
    double lds_dup_cycles;   /* added per lane that shares its word with another lane */
    double launch_us;        /* one kernel launch */
    double sweep_fixed_us;   /* a sweep beyond its pass over the input: LDS clear, flush, ramp */
    double event_cycles;     /* one 8-bit carry event, logged and applied, cycles of one CU */
    double scatter_fixed_us; /* the two-phase path beyond its passes: scans, merge, launches */
} hist_model_calib_t;

typedef struct {
    hist_plan_opts_t opts; /* path, counter_bits, aggregation (the rest 0) */
    double predicted_us;   /* -1 when the bin count does not allow the schedule */
    double pass_us;        /* passes over the input and the staged slots */
    double lds_us;         /* LDS atomics */
    double events_us;      /* 8-bit carry events */
    double fixed_us;       /* fixed costs and the merge of partial rows */
    int32_t status;        /* HIST_OK, or HIST_ERR_UNSUPPORTED */
    int32_t reserved;
} hist_prediction_t;

/* The primitives as the library's probes measured them on an MI355X
 * (bench.py --calibrate). */
hist_status_t hist_model_calibration(hist_model_calib_t *cal);

/* Predict every candidate schedule's time for a histogram of num_bins bins
 * over n elements on the described device (host only, no device needed).
 * cal: the primitives (NULL: hist_model_calibration's). sample: host
 * int32[sample_n], elements of the input in no particular order (a few
 * thousand to 2^16; sample_n 0 treats the input as uniform and in range).
 * Writes the fastest predicted candidate's options to *best and the
 * candidates to entries[0..*count) (at most capacity; entries and count may
 * be NULL when capacity is 0). Errors: INVALID_ARG for null dev or best,
 * num_bins == 0, n == 0 or n >= 2^32, a null sample with sample_n > 0, bad
 * calibration figures; UNSUPPORTED for num_bins > HIST_MAX_BINS. */
hist_status_t hist_predict(const hist_device_desc_t *dev, const hist_model_calib_t *cal,
                           uint32_t num_bins, uint64_t n, const int32_t *sample, uint32_t sample_n,
                           hist_plan_opts_t *best, hist_prediction_t *entries, uint32_t capacity,
                           uint32_t *count);

/* hist_predict on the current device for the caller's device input: takes a
 * sample of up to 64 runs of 1,024 elements at evenly spaced places, times
 * one stream read of the input (the baseline), and predicts. workspace:
 * device memory of at least HIST_SELECT_WORKSPACE_BYTES, 256-byte aligned
 * (overwritten). Synchronous. No schedule is run. Errors: as hist_predict,
 * WORKSPACE for a missing or small workspace, UNSUPPORTED when the current
 * device is not gfx950, HIP when a launch or copy fails. */
#define HIST_SELECT_WORKSPACE_BYTES (64u * 1024u * 4u + 16384u)
hist_status_t hist_select(uint32_t num_bins, const int32_t *input, uint64_t n,
                          const hist_model_calib_t *cal, void *workspace, uint64_t workspace_bytes,
                          hipStream_t stream, hist_plan_opts_t *best, hist_prediction_t *entries,
                          uint32_t capacity, uint32_t *count);

/* Write a one-line description ("path=range R=2 S=32768 G=128 ...") into
 * buf (always NUL-terminated when len > 0). */
hist_status_t hist_plan_describe(const hist_plan_t *plan, char *buf, uint64_t len);

/* Per-kernel timing for measurement. When enabled, hist_run attaches a pair
 * of HIP events to the kernels of each phase it launches (hipExtLaunchKernel:
 * the start of the phase's first kernel and the end of its last), so a
 * phase's time is its kernels' own execution, as a profiler's kernel trace
 * reports it, with nothing queued between kernels.
 * hist_plan_timing_read waits for the recorded events and returns, for each
 * phase p < HIST_MAX_PHASES, the summed milliseconds and the launch count,
 * then clears the record. Phase names come from hist_plan_phase_name.
 * capacity bounds the number of hist_run calls recorded (older ones beyond
 * it are not recorded). Enabling allocates host-side HIP events only. */
#define HIST_MAX_PHASES 7
hist_status_t hist_plan_timing_enable(hist_plan_t *plan, uint32_t capacity);
hist_status_t hist_plan_timing_read(hist_plan_t *plan, double *ms, uint32_t *launches);
const char *hist_plan_phase_name(const hist_plan_t *plan, uint32_t phase);

/* Whether a bounded wait of the plan's last run gave up (STREAM plans; 0
 * for every other path). Waits for the stream first. A give-up means the
 * counts of that run are incomplete; it cannot happen unless a wait outlasts
 * its bound (spin_log2). Errors: INVALID_ARG for a null argument, HIP when
 * the copy fails. */
hist_status_t hist_plan_check(hist_plan_t *plan, hipStream_t stream, uint32_t *gave_up);

/* The timeline of a STREAM plan's last run, one record of
 * HIST_STREAM_TRACE_WORDS 32-bit words per workgroup of its persistent
 * kernel, in the order the workgroups started (record i is the workgroup
 * that took ticket i; tickets below the plan's producer count are the
 * producers). Words: 0 ticket, 1 start, 2 end of its producer part (0 for an
 * owner from the start), 3 end, 4 tiles routed, 5 blocks counted, 6 stints
 * written to the pool, 7 ticks waiting for tiles' flags, 8 moves to another
 * range denied by the move budget (0 or 1), 9 ticks writing stints, 10 ticks
 * counting blocks, 11 range scans; 12..15 zero. Times are the low 32 bits of the
 * 100 MHz constant clock (s_memrealtime), so differences are taken modulo
 * 2^32. Waits for the stream, then copies into out (host memory of capacity
 * words) and sets *workgroups; 0 workgroups for other paths. Errors:
 * INVALID_ARG for a null plan or workgroups pointer, or a capacity below
 * workgroups x HIST_STREAM_TRACE_WORDS; HIP when the copy fails. */
#define HIST_STREAM_TRACE_WORDS 16
hist_status_t hist_plan_stream_trace(hist_plan_t *plan, hipStream_t stream, uint32_t *out,
                                     uint32_t capacity, uint32_t *workgroups);

void hist_plan_destroy(hist_plan_t *plan);

const char *hist_status_str(hist_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* PCA_HIST_H */
