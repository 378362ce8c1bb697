// hist_tune.hip -- measured schedule choice (declared in hist.h).
//
// Host code only, on top of the public entry points: each candidate schedule
// gets a plan on the caller's workspace, one untimed run and `reps` runs
// between two HIP events on the caller's stream. The cost-guided selection
// of "CREDIT: Cost-guided Reduction-reuse with Efficient DSMEM Inter-CTA
// Tiling" (cost model section, Eq. 7) prices a schedule with a rate measured
// at the same shape rather than a device peak; every candidate here is cheap
// enough to be measured itself, on the caller's data.
#include "hist.h"

#include <hip/hip_runtime.h>

#include <cstring>

namespace {

struct Candidate {
    int32_t path, counter_bits, aggregation;
};

// The order hist.h documents.
constexpr Candidate kCandidates[HIST_TUNE_MAX_ENTRIES] = {
    {HIST_PATH_FULL, 32, 0},    {HIST_PATH_FULL, 16, 0},    {HIST_PATH_FULL, 8, 0},
    {HIST_PATH_RANGE, 32, 0},   {HIST_PATH_RANGE, 16, 0},   {HIST_PATH_RANGE, 16, 1},
    {HIST_PATH_RANGE, 8, 0},    {HIST_PATH_RANGE, 8, 1},    {HIST_PATH_SCATTER, 0, 0},
    {HIST_PATH_SCATTER, 0, 1},
};

hist_plan_opts_t opts_of(const Candidate &c)
{
    hist_plan_opts_t o;
    std::memset(&o, 0, sizeof(o));
    o.path = c.path;
    o.counter_bits = c.counter_bits;
    o.aggregation = c.aggregation;
    return o;
}

// Mean milliseconds per run of one plan: one untimed run, then reps runs
// between two events.
hist_status_t time_plan(hist_plan_t *plan, uint32_t *counts, const int32_t *input, uint64_t n,
                        uint32_t num_bins, uint32_t reps, hipStream_t stream, double *ms)
{
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess) return HIST_ERR_HIP;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return HIST_ERR_HIP;
    }
    hist_status_t st = hist_run(plan, counts, input, n, num_bins, stream);
    if (st == HIST_OK && hipEventRecord(e0, stream) != hipSuccess) st = HIST_ERR_HIP;
    for (uint32_t k = 0; st == HIST_OK && k < reps; ++k)
        st = hist_run(plan, counts, input, n, num_bins, stream);
    if (st == HIST_OK && hipEventRecord(e1, stream) != hipSuccess) st = HIST_ERR_HIP;
    float t = 0.f;
    if (st == HIST_OK && (hipEventSynchronize(e1) != hipSuccess ||
                          hipEventElapsedTime(&t, e0, e1) != hipSuccess))
        st = HIST_ERR_HIP;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (st == HIST_OK) *ms = (double)t / reps;
    return st;
}

}  // namespace

extern "C" {

hist_status_t hist_tune_workspace_size(uint32_t num_bins, uint64_t max_n, uint64_t *bytes)
{
    if (!bytes) return HIST_ERR_INVALID_ARG;
    uint64_t most = 0;
    bool any = false;
    for (const Candidate &c : kCandidates) {
        const hist_plan_opts_t o = opts_of(c);
        uint64_t b = 0;
        const hist_status_t st = hist_workspace_size(num_bins, max_n, &o, &b);
        if (st == HIST_ERR_UNSUPPORTED) continue;  // not for this bin count (or no device)
        if (st != HIST_OK) return st;
        any = true;
        if (b > most) most = b;
    }
    if (!any) return HIST_ERR_UNSUPPORTED;
    *bytes = most;
    return HIST_OK;
}

hist_status_t hist_tune(uint32_t num_bins, uint64_t max_n, const int32_t *input, uint64_t n,
                        uint32_t *counts, void *workspace, uint64_t workspace_bytes,
                        uint32_t reps, hipStream_t stream, hist_plan_opts_t *best,
                        hist_tune_entry_t *entries, uint32_t capacity, uint32_t *count)
{
    if (!input || !counts || !best || n == 0 || n > max_n || reps == 0 || reps > 1000)
        return HIST_ERR_INVALID_ARG;
    if (capacity > 0 && (!entries || !count)) return HIST_ERR_INVALID_ARG;
    if (((uintptr_t)workspace & 255u) != 0) return HIST_ERR_INVALID_ARG;
    // Arguments and device first: the same checks as a plain plan.
    uint64_t probe = 0;
    {
        const hist_status_t st = hist_workspace_size(num_bins, max_n, nullptr, &probe);
        if (st != HIST_OK) return st;
    }
    double best_ms = -1.0;
    uint32_t written = 0;
    bool fits_any = false;
    for (const Candidate &c : kCandidates) {
        hist_tune_entry_t e;
        std::memset(&e, 0, sizeof(e));
        e.opts = opts_of(c);
        e.ms = -1.0;
        uint64_t need = 0;
        hist_status_t st = hist_workspace_size(num_bins, max_n, &e.opts, &need);
        if (st == HIST_OK && need > 0 && (!workspace || need > workspace_bytes))
            st = HIST_ERR_WORKSPACE;
        if (st == HIST_OK) {
            fits_any = true;
            hist_plan_t *plan = nullptr;
            st = hist_plan(&plan, num_bins, max_n, &e.opts, need ? workspace : nullptr,
                           need ? workspace_bytes : 0);
            if (st == HIST_OK) {
                st = time_plan(plan, counts, input, n, num_bins, reps, stream, &e.ms);
                hist_plan_destroy(plan);
            }
            if (st != HIST_OK && st != HIST_ERR_UNSUPPORTED) return st;
        }
        e.status = st;
        if (st == HIST_OK && (best_ms < 0.0 || e.ms < best_ms)) {
            best_ms = e.ms;
            *best = e.opts;
        }
        if (written < capacity) entries[written++] = e;
    }
    if (count) *count = written;
    if (best_ms < 0.0) return fits_any ? HIST_ERR_UNSUPPORTED : HIST_ERR_WORKSPACE;
    return HIST_OK;
}

}  // extern "C"
