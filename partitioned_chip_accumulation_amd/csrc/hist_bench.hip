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

// LDS latency: one wave, a chain of dependent operations on LDS, each one's
// address waiting for the previous one's returned value (the address is
// base ^ (old >> 31), which stays base since the counts stay below 2^31).
// PATTERN: 0 ds_add_rtn_u32 from lane 0 alone, 1 from 64 lanes on 64
// consecutive words, 2 from 64 lanes on one word, 3 ds_read_b32 from 64
// lanes on consecutive words (the load latency, for reference).
// out[0] = shader-clock cycles (s_memtime) over the chain, out[1] = ticks of
// the 100 MHz real-time counter (s_memrealtime), out[2] = the final address
// (keeps the chain live).
template <int PATTERN>
__global__ __launch_bounds__(64) void k_lds_latency(uint32_t iters, uint64_t *__restrict__ out)
{
    __shared__ uint32_t lds[4096];
    const uint32_t lane = threadIdx.x;
    for (uint32_t i = lane; i < 4096; i += 64) lds[i] = 0u;
    __syncthreads();
    const uint32_t base = PATTERN == 2 ? 1024u : lane;
    uint32_t a = base;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    if (PATTERN != 0 || lane == 0) {
        for (uint32_t k = 0; k < iters; ++k) {
            uint32_t old;
            if constexpr (PATTERN == 3)
                old = __hip_atomic_load(lds + a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            else
                old = __hip_atomic_fetch_add(lds + a, 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_WORKGROUP);
            a = base ^ (old >> 31);
        }
    }
    asm volatile("" ::"v"(a) : "memory");  // the chain's last value is in before the clocks
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
        out[0] = t1 - t0;
        out[1] = r1 - r0;
        out[2] = a;
    }
}

// Handoff latency between two workgroups through global memory. Workgroup 0
// and workgroup `partner` pass a token back and forth iters times (one round
// trip per iteration) in a word of flags[]; every other workgroup only
// records where it ran. The launch is cooperative, so all workgroups are
// resident at once, and every wait gives up after kSpin polls, so the kernel
// always ends (out[2] then reports the time-out).
//   mode 0: the token alone, relaxed device-scope atomic store and load;
//   mode 1: before each token, the sender's 64 lanes store a 256-byte
//           payload with plain stores, and the token is a release store read
//           with acquire loads; the receiver checks the payload.
// out[0] = shader-clock cycles over the iterations (workgroup 0), out[1] =
// 100 MHz real-time ticks, out[2] = 1 if a wait gave up, out[3] = payload
// words that arrived wrong, out[4 + b] = the XCD (HW_REG_XCC_ID) workgroup b
// ran on, for b < 16. flags holds the token (word 0) and the payload (words
// 16..79), zeroed by the host first.
constexpr uint32_t kSpin = 1u << 22;

__device__ __forceinline__ uint32_t xcc_id()
{
    uint32_t x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    return x & 0xFu;
}

__global__ __launch_bounds__(64) void k_handoff(uint32_t partner, uint32_t mode, uint32_t iters,
                                                uint32_t *__restrict__ flags,
                                                uint64_t *__restrict__ out)
{
    const uint32_t lane = threadIdx.x, b = blockIdx.x;
    if (lane == 0 && b < 16) out[4 + b] = xcc_id();
    if (b != 0 && b != partner) return;
    uint32_t *token = flags;
    uint32_t *payload = flags + 16;
    const bool ping = b == 0;
    uint32_t bad = 0, timeout = 0;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (uint32_t k = 0; k < iters && !timeout; ++k) {
        // the sender of round k's first half is workgroup 0, of its second half the partner
        for (uint32_t half = 0; half < 2; ++half) {
            const uint32_t want = 2u * k + half + 1u;
            const bool send = ping == (half == 0);
            if (send) {
                if (mode == 1) {
                    payload[lane] = want * 64u + lane;
                    if (lane == 0)
                        __hip_atomic_store(token, want, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                } else if (lane == 0) {
                    __hip_atomic_store(token, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            } else {
                uint32_t spins = 0, v;
                do {
                    v = mode == 1 ? __hip_atomic_load(token, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT)
                                  : __hip_atomic_load(token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } while (v != want && ++spins < kSpin);
                if (v != want) {
                    timeout = 1;
                    break;
                }
                if (mode == 1 && payload[lane] != want * 64u + lane) ++bad;
            }
        }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    // payload mismatches of the receiving lanes, summed over the wave
    for (int d = 32; d >= 1; d >>= 1) bad += __shfl_xor(bad, d, 64);
    if (lane == 0) {
        if (ping) {
            out[0] = t1 - t0;
            out[1] = r1 - r0;
        }
        if (timeout) __hip_atomic_fetch_or(out + 2, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (bad) __hip_atomic_fetch_add(out + 3, (uint64_t)bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__global__ void k_zero64(uint64_t *__restrict__ d, uint32_t n)
{
    for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) d[i] = 0ull;
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

hist_status_t hist_bench_lds_latency(uint32_t pattern, uint32_t iters, uint64_t *out,
                                     hipStream_t stream)
{
    if (pattern > 3 || iters == 0 || iters > (1u << 24) || !out) return HIST_ERR_INVALID_ARG;
    void (*k)(uint32_t, uint64_t *) = pattern == 0   ? k_lds_latency<0>
                                      : pattern == 1 ? k_lds_latency<1>
                                      : pattern == 2 ? k_lds_latency<2>
                                                     : k_lds_latency<3>;
    hipLaunchKernelGGL(k, dim3(1), dim3(64), 0, stream, iters, out);
    return hipGetLastError() == hipSuccess ? HIST_OK : HIST_ERR_HIP;
}

hist_status_t hist_bench_handoff(uint32_t partner, uint32_t mode, uint32_t iters, uint32_t *flags,
                                 uint64_t *out, hipStream_t stream)
{
    if (partner < 1 || partner >= 16 || mode > 1 || iters == 0 || iters > (1u << 20) || !flags ||
        !out)
        return HIST_ERR_INVALID_ARG;
    int dev = 0, coop = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess ||
        !coop)
        return HIST_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(k_zero, dim3(1), dim3(128), 0, stream, flags, (uint64_t)80);
    hipLaunchKernelGGL(k_zero64, dim3(1), dim3(64), 0, stream, out, 20u);
    if (hipGetLastError() != hipSuccess) return HIST_ERR_HIP;
    void *args[] = {&partner, &mode, &iters, &flags, &out};
    if (hipLaunchCooperativeKernel(reinterpret_cast<const void *>(k_handoff), dim3(16), dim3(64), args,
                                   0, stream) != hipSuccess) {
        (void)hipGetLastError();
        return HIST_ERR_HIP;
    }
    return HIST_OK;
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
