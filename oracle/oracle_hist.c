/*
 * oracle_hist.c -- CPU oracle for the partitioned on-chip histogram.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes
 * ----------------
 * The page "Distributed Shared Memory", section "The cluster histogram",
 * defines the workload: every element of the input names one bin, the thread
 * that reads it adds exactly one to that bin in the slice of the block that
 * owns the bin, and at the end each block adds its slice into the global
 * array of bins. Integer addition is exact, associative and commutative, so
 * however the bins are partitioned and whichever block touches them first,
 * the final value of bin b is the number of input elements equal to b.
 * That plain definition is what this oracle writes out:
 *
 *     counts[b] = #{ i in [0, n) : input[i] == b },   0 <= b < num_bins.
 *
 * Readings where the page is silent (it requires the bin count to equal the
 * cluster's capacity exactly and says nothing of values outside it):
 *   - values that are negative or >= num_bins name no bin; they are skipped
 *     and reported in the return value ("dropped");
 *   - the output is overwritten, not accumulated into;
 *   - counters are 32-bit unsigned; n must stay below 2^32 so none can wrap.
 *
 * It is a single sequential loop on purpose: no blocking, no threads, no
 * vector tricks, so that it can be checked against the definition by eye.
 */
#include <stdint.h>
#include <string.h>

/* Returns the number of elements that named no bin, or UINT64_MAX when the
 * arguments are unusable (null pointers with n > 0, num_bins == 0, or n too
 * large for a 32-bit counter). */
uint64_t oracle_hist(const int32_t *input, uint64_t n, uint32_t num_bins,
                     uint32_t *counts)
{
    if (num_bins == 0 || counts == NULL) return UINT64_MAX;
    if (n > 0 && input == NULL) return UINT64_MAX;
    if (n > (uint64_t)UINT32_MAX) return UINT64_MAX;

    memset(counts, 0, (size_t)num_bins * sizeof(uint32_t));

    uint64_t dropped = 0;
    for (uint64_t i = 0; i < n; ++i) {
        int64_t x = input[i];
        if (x >= 0 && x < (int64_t)num_bins)
            counts[x] += 1;
        else
            dropped += 1;
    }
    return dropped;
}
