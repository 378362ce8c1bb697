// hist_bench.hip -- measurement-only kernels (declared in hist_bench.h).
#include "hist_bench.h"

#include <hip/hip_runtime.h>

#include <algorithm>

namespace pca_bench {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void k_zero(uint32_t *__restrict__ d, uint64_t n)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x)
        d[i] = 0u;
}

// Every element is one device-scope atomic add into global memory.
__global__ __launch_bounds__(256) void k_global_atomic(uint32_t *__restrict__ counts,
                                                       const int32_t *__restrict__ in, uint64_t n,
                                                       uint32_t num_bins)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x) {
        const uint32_t x = (uint32_t)in[i];
        if (x < num_bins) atomicAdd(counts + x, 1u);
    }
}

__global__ __launch_bounds__(256) void k_read(const u32x4 *__restrict__ src, uint64_t nvec,
                                              uint32_t *__restrict__ sink)
{
    u32x4 acc = {0u, 0u, 0u, 0u};
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < nvec; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= (a ^ b) ^ (c ^ d);
    }
    for (; i < nvec; i += stride) acc ^= __builtin_nontemporal_load(src + i);
    uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
    // keep the loads live: the store depends on every loaded value but almost never runs
    if (v == 0x9E3779B9u) sink[blockIdx.x % 4096] = v;
}

__global__ __launch_bounds__(256) void k_copy(u32x4 *__restrict__ dst, const u32x4 *__restrict__ src,
                                              uint64_t nvec)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride)
        dst[i] = src[i];
}

int grid_for(uint64_t work, int per_block)
{
    int dev = 0, cu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev);
    const uint64_t want = (work + per_block - 1) / per_block;
    return (int)std::max<uint64_t>(1, std::min<uint64_t>(want, (uint64_t)cu * 16));
}

// LDS atomic rate for one address pattern (calibration). Each lane holds 16
// precomputed word addresses in registers and adds to them in turn, so the
// loop issues nothing but the atomics and its counter. PATTERN: 0 distinct
// consecutive words (no bank conflict), 1 random words of a 32,768-word
// array, 2 all 64 lanes of the wave on one word, 3 eight groups of eight
// lanes, one word per group.
constexpr uint32_t kCalWords = 32768;

template <int PATTERN, bool RTN>
__global__ __launch_bounds__(1024) void k_lds_atomic(uint32_t iters, uint32_t *__restrict__ sink)
{
    __shared__ uint32_t lds[kCalWords];
    for (uint32_t i = threadIdx.x; i < kCalWords; i += blockDim.x) lds[i] = 0u;
    __syncthreads();
    const uint32_t lane = threadIdx.x & 63u;
    uint32_t a[16];
#pragma unroll
    for (uint32_t j = 0; j < 16; ++j) {
        uint32_t w;
        if (PATTERN == 0) {
            w = j * 64u + lane;
        } else if (PATTERN == 1) {
            // splitmix-style mix of (block, thread, j): a fixed random pattern per j
            uint32_t h = (blockIdx.x * 1024u + threadIdx.x) * 16u + j;
            h = (h ^ (h >> 16)) * 0x7FEB352Du;
            h = (h ^ (h >> 15)) * 0x846CA68Bu;
            w = h ^ (h >> 16);
        } else if (PATTERN == 2) {
            w = j * 97u;
        } else {
            w = j * 97u + (lane >> 3) * 4099u;
        }
        a[j] = w & (kCalWords - 1u);
    }
    uint32_t acc = 0;
    for (uint32_t it = 0; it < iters; ++it) {
#pragma unroll
        for (uint32_t j = 0; j < 16; ++j) {
            if (RTN)
                acc += __hip_atomic_fetch_add(lds + a[j], 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_WORKGROUP);
            else
                __hip_atomic_fetch_add(lds + a[j], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = lds[0] + acc;
}

}  // namespace pca_bench

using namespace pca_bench;

extern "C" {

hist_status_t hist_bench_global_atomic(uint32_t *counts, const int32_t *input, uint64_t n,
                                       uint32_t num_bins, hipStream_t stream)
{
    if (!counts || (n && !input) || num_bins == 0 || n > (uint64_t)UINT32_MAX)
        return HIST_ERR_INVALID_ARG;
    hipLaunchKernelGGL(k_zero, dim3(grid_for(num_bins, 256)), dim3(256), 0, stream, counts,
                       (uint64_t)num_bins);
    if (n)
        hipLaunchKernelGGL(k_global_atomic, dim3(grid_for(n, 256 * 16)), dim3(256), 0, stream,
                           counts, input, n, num_bins);
    return hipGetLastError() == hipSuccess ? HIST_OK : HIST_ERR_HIP;
}

hist_status_t hist_bench_read(const void *src, uint64_t bytes, uint32_t *sink, hipStream_t stream)
{
    if (!src || !sink || (bytes & 15u) || ((uintptr_t)src & 15u)) return HIST_ERR_INVALID_ARG;
    const int grid = std::min(grid_for(bytes / 16, 256 * 8), 4096);
    hipLaunchKernelGGL(k_read, dim3(grid), dim3(256), 0, stream,
                       static_cast<const u32x4 *>(src), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? HIST_OK : HIST_ERR_HIP;
}

hist_status_t hist_bench_lds_atomic(uint32_t pattern, uint32_t with_return, uint32_t iters,
                                   uint32_t *sink, uint32_t sink_words, hipStream_t stream)
{
    if (pattern > 3 || iters == 0 || !sink) return HIST_ERR_INVALID_ARG;
    int dev = 0, cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return HIST_ERR_UNSUPPORTED;
    if (cu <= 0 || sink_words < (uint32_t)cu) return HIST_ERR_INVALID_ARG;
    void (*k)(uint32_t, uint32_t *) = nullptr;
    switch (pattern * 2 + (with_return ? 1 : 0)) {
    case 0: k = k_lds_atomic<0, false>; break;
    case 1: k = k_lds_atomic<0, true>; break;
    case 2: k = k_lds_atomic<1, false>; break;
    case 3: k = k_lds_atomic<1, true>; break;
    case 4: k = k_lds_atomic<2, false>; break;
    case 5: k = k_lds_atomic<2, true>; break;
    case 6: k = k_lds_atomic<3, false>; break;
    default: k = k_lds_atomic<3, true>; break;
    }
    hipLaunchKernelGGL(k, dim3(cu), dim3(1024), 0, stream, iters, sink);
    return hipGetLastError() == hipSuccess ? HIST_OK : HIST_ERR_HIP;
}

hist_status_t hist_bench_copy(void *dst, const void *src, uint64_t bytes, hipStream_t stream)
{
    if (!dst || !src || (bytes & 15u) || ((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u))
        return HIST_ERR_INVALID_ARG;
    const uintptr_t a = (uintptr_t)dst, b = (uintptr_t)src;
    if (a < b + bytes && b < a + bytes) return HIST_ERR_INVALID_ARG;
    hipLaunchKernelGGL(k_copy, dim3(grid_for(bytes / 16, 256 * 8)), dim3(256), 0, stream,
                       static_cast<u32x4 *>(dst), static_cast<const u32x4 *>(src), bytes / 16);
    return hipGetLastError() == hipSuccess ? HIST_OK : HIST_ERR_HIP;
}

}  // extern "C"
