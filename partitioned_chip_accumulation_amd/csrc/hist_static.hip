// hist_static.hip -- hist_run_static: the histogram with no allocation, its
// workspace in a device array the library holds (declared in hist.h).
//
// The array lives in this file only. Host code never passes its name to a
// kernel: on the host that name is a stand-in, not a device address. The
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that pointer reaches the kernels (as the
// workspace pointer hist_run passes).
#include "hist.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "hist_host.hpp"

namespace {

constexpr uint64_t kScratchBytes = HIST_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// One copy per device, at its own address on each; kept until the process
// ends. Nothing in it must start at zero: every run writes each region of
// the workspace before reading it.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceScratch {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

// The array's address on device dev, which must be current.
hist_status_t scratch_on(int dev, void **ptr)
{
    if (dev < 0 || dev >= kMaxDevices) return HIST_ERR_UNSUPPORTED;
    DeviceScratch &d = g_scratch[dev];
    std::call_once(d.once, [&d] {
        d.err = hipGetSymbolAddress(&d.ptr, HIP_SYMBOL(scratch));
        if (d.err != hipSuccess) {
            (void)hipGetLastError();
            d.ptr = nullptr;
        }
    });
    if (d.err != hipSuccess || !d.ptr) return HIST_ERR_HIP;
    *ptr = d.ptr;
    return HIST_OK;
}

}  // namespace

extern "C" hist_status_t hist_run_static(uint32_t *counts, const int32_t *input, uint64_t n,
                                         uint32_t num_bins, hipStream_t stream)
{
    if (!counts || (n > 0 && !input) || num_bins == 0 || n > (uint64_t)UINT32_MAX)
        return HIST_ERR_INVALID_ARG;
    if (num_bins > HIST_MAX_BINS) return HIST_ERR_UNSUPPORTED;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return HIST_ERR_UNSUPPORTED;
    }
    hist_status_t st = pca_host::device_supported(dev);
    if (st != HIST_OK) return st;
    void *ws = nullptr;
    st = scratch_on(dev, &ws);
    if (st != HIST_OK) return st;
    return pca_host::run_in_workspace(counts, input, n, num_bins, stream, ws, kScratchBytes, dev);
}
