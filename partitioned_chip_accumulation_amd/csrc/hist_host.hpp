// hist_host.hpp -- host-side hooks shared between the library's source files
// (internal to libpca_hist.so; not part of the C ABI).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "hist.h"

namespace pca_host {

// HIST_OK when device dev is one the kernels run on (gfx950), else
// HIST_ERR_UNSUPPORTED; the device's numbers are queried once per device.
hist_status_t device_supported(int dev);

// Plan a histogram of num_bins bins for exactly n elements on device dev (the
// current device) with default options, placing its workspace at ws
// (ws_bytes, 256-byte aligned), and queue it on stream: the kernels and the
// result of hist_run. When the default plan's one-pass workspace (its
// partial rows) exceeds ws_bytes, fewer input chunks are taken; when the plan
// still does not fit, HIST_ERR_WORKSPACE is returned before anything is
// queued. Argument errors as hist_run.
hist_status_t run_in_workspace(uint32_t *counts, const int32_t *input, uint64_t n,
                               uint32_t num_bins, hipStream_t stream, void *ws, uint64_t ws_bytes,
                               int dev);

}  // namespace pca_host
