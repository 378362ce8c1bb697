/* Plain C99 client of the library's C ABI (include/hist.h, include/hist_bench.h).
 * Built and run by tests/test_abi_cpu.py with gcc, no GPU needed: every entry
 * point must link, and calls with bad arguments must return the documented
 * status without touching a device. Prints the public structs' layout, then
 * "ok", and exits 0 on success. */
#include "hist.h"
#include "hist_bench.h"

#include <stddef.h>
#include <stdio.h>
#include <string.h>

static int failures = 0;

static void expect(const char *what, int got, int want)
{
    if (got != want) {
        printf("%s: got %d, want %d\n", what, got, want);
        ++failures;
    }
}

int main(void)
{
    uint64_t bytes = 0;
    hist_plan_t *plan = NULL;
    hist_plan_info_t info;
    hist_plan_opts_t opts;
    double ms[HIST_MAX_PHASES];
    uint32_t launches[HIST_MAX_PHASES];
    char buf[64];

    memset(&opts, 0, sizeof(opts));
    opts.aggregation = -1;
    expect("workspace_size(num_bins=0)", hist_workspace_size(0, 10, &opts, &bytes),
           HIST_ERR_INVALID_ARG);
    expect("workspace_size(bytes=NULL)", hist_workspace_size(10, 10, NULL, NULL),
           HIST_ERR_INVALID_ARG);
    opts.path = 9;
    expect("workspace_size(bad path)", hist_workspace_size(10, 10, &opts, &bytes),
           HIST_ERR_INVALID_ARG);
    expect("plan(NULL)", hist_plan(NULL, 10, 10, NULL, NULL, 0), HIST_ERR_INVALID_ARG);
    expect("plan(num_bins=0)", hist_plan(&plan, 0, 10, NULL, NULL, 0), HIST_ERR_INVALID_ARG);
    expect("plan(max_n=2^32)", hist_plan(&plan, 10, 1ull << 32, NULL, NULL, 0),
           HIST_ERR_INVALID_ARG);
    expect("plan(misaligned workspace)", hist_plan(&plan, 10, 10, NULL, (void *)3, 0),
           HIST_ERR_INVALID_ARG);
    expect("plan left NULL", plan == NULL, 1);
    expect("plan_create(NULL)", hist_plan_create(NULL, 10, 10, NULL, NULL, 0),
           HIST_ERR_INVALID_ARG);
    expect("run(NULL)", hist_run(NULL, NULL, NULL, 0, 1, NULL), HIST_ERR_INVALID_ARG);
    expect("run_static(NULL)", hist_run_static(NULL, NULL, 0, 1, NULL), HIST_ERR_INVALID_ARG);
    expect("run_static(num_bins=0)", hist_run_static((uint32_t *)16, NULL, 0, 0, NULL),
           HIST_ERR_INVALID_ARG);
    expect("run_static(input=NULL, n=5)", hist_run_static((uint32_t *)16, NULL, 5, 8, NULL),
           HIST_ERR_INVALID_ARG);
    expect("run_accumulate(NULL)", hist_run_accumulate(NULL, NULL, NULL, 0, 1, NULL),
           HIST_ERR_INVALID_ARG);
    expect("plan_info(NULL)", hist_plan_info(NULL, &info), HIST_ERR_INVALID_ARG);
    expect("plan_describe(NULL)", hist_plan_describe(NULL, buf, sizeof(buf)), HIST_ERR_INVALID_ARG);
    {
        /* planning needs no device: an MI355X as the kernels see it */
        hist_device_desc_t dev = {256, 8, 163840, 6};
        expect("plan_preview(NULL dev)", hist_plan_preview(NULL, 8, 8, NULL, &info),
               HIST_ERR_INVALID_ARG);
        expect("plan_preview(65536 bins)", hist_plan_preview(&dev, 65536, 1u << 26, NULL, &info),
               HIST_OK);
        expect("plan_preview path", info.path, HIST_PATH_FULL);
        expect("plan_preview groups", (int)info.groups, 256);
    }
    {
        hist_plan_opts_t best;
        hist_tune_entry_t entries[HIST_TUNE_MAX_ENTRIES];
        uint32_t count = 0;
        expect("tune_workspace_size(bytes=NULL)", hist_tune_workspace_size(10, 10, NULL),
               HIST_ERR_INVALID_ARG);
        expect("tune(input=NULL)", hist_tune(10, 10, NULL, 1, NULL, NULL, 0, 1, NULL, &best,
                                             entries, HIST_TUNE_MAX_ENTRIES, &count),
               HIST_ERR_INVALID_ARG);
    }
    {
        /* the cost model needs no device: a prediction on an MI355X description */
        hist_device_desc_t dev = {256, 8, 163840, 6};
        hist_model_calib_t cal;
        hist_plan_opts_t best;
        hist_prediction_t pred[HIST_MODEL_MAX_ENTRIES];
        uint32_t count = 0;
        int32_t sample[4096];
        int i;
        for (i = 0; i < 4096; ++i) sample[i] = (int32_t)((i * 2654435761u) % 65536u);
        expect("model_calibration", hist_model_calibration(&cal), HIST_OK);
        expect("predict(NULL dev)", hist_predict(NULL, &cal, 10, 10, NULL, 0, &best, NULL, 0, NULL),
               HIST_ERR_INVALID_ARG);
        expect("predict(65536 bins)", hist_predict(&dev, &cal, 65536, 1u << 26, sample, 4096, &best,
                                                   pred, HIST_MODEL_MAX_ENTRIES, &count), HIST_OK);
        expect("predict count", (int)count, HIST_MODEL_MAX_ENTRIES);
        expect("predict path", best.path, HIST_PATH_FULL);
        expect("select(input=NULL)", hist_select(10, NULL, 10, NULL, NULL, 0, NULL, &best, NULL, 0,
                                                 NULL), HIST_ERR_INVALID_ARG);
    }
    expect("timing_enable(NULL)", hist_plan_timing_enable(NULL, 1), HIST_ERR_INVALID_ARG);
    expect("timing_read(NULL)", hist_plan_timing_read(NULL, ms, launches), HIST_ERR_INVALID_ARG);
    expect("phase_name(0)", strcmp(hist_plan_phase_name(NULL, 0), "sweep"), 0);
    expect("bench_global_atomic(NULL)", hist_bench_global_atomic(NULL, NULL, 0, 1, NULL),
           HIST_ERR_INVALID_ARG);
    expect("bench_read(NULL)", hist_bench_read(NULL, 16, NULL, NULL), HIST_ERR_INVALID_ARG);
    expect("bench_copy(NULL)", hist_bench_copy(NULL, NULL, 16, NULL), HIST_ERR_INVALID_ARG);
    expect("bench_lds_atomic(bad pattern)", hist_bench_lds_atomic(4, 0, 1, NULL, 0, NULL),
           HIST_ERR_INVALID_ARG);
    expect("status_str(OK)", strcmp(hist_status_str(HIST_OK), "ok"), 0);
    hist_plan_destroy(NULL);
    /* struct layouts, for the Python binding's ctypes mirrors */
    printf("layout %zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(hist_plan_info_t),
           sizeof(hist_plan_opts_t), offsetof(hist_plan_info_t, max_group_elems),
           offsetof(hist_plan_info_t, event_cap), sizeof(hist_device_desc_t),
           sizeof(hist_tune_entry_t), offsetof(hist_tune_entry_t, ms),
           offsetof(hist_tune_entry_t, status));
    printf("layout2 %zu %zu %zu %zu\n", sizeof(hist_model_calib_t), sizeof(hist_prediction_t),
           offsetof(hist_prediction_t, predicted_us), offsetof(hist_prediction_t, status));
    if (failures == 0) printf("ok\n");
    return failures == 0 ? 0 : 1;
}
