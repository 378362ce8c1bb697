// hist_common.hpp -- shared pieces of the gfx950 kernels of the partitioned LDS
// histogram: the input view, wave and LDS helpers, the wave hot slot, and the
// zero-fill kernel. Part of libpca_hist.so (see hist_kernels.hpp for the
// overview).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pca {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The input split into a 16-byte aligned body of int4 vectors and at most
// three scalars before (head) and after (tail) it. The host fills this from
// the caller's pointer, which only needs 4-byte alignment.
struct InputView {
    const int32_t *ptr;
    uint64_t nvec;  // vectors in the body, which starts at ptr + head
    uint32_t head;  // 0..3 elements before the body
    uint32_t tail;  // 0..3 elements after the body
};

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// Inclusive sums by DPP, one VALU add a step with no LDS round trip: row
// shifts by 1, 2, 4 and 8 within each row of 16 lanes (a lane shifted in
// from outside the row reads 0), then, across rows, lane 15 of rows 0 and 2
// into rows 1 and 3 (row_bcast:15) and lane 31 into rows 2 and 3
// (row_bcast:31). Every lane of the wave must be active: DPP reads the
// source lane's register whether or not that lane runs.
__device__ __forceinline__ uint32_t row_inclusive_scan(uint32_t v)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);  // row_shr:8
    return v;
}

__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v)
{
    v = row_inclusive_scan(v);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

__device__ __forceinline__ void lds_add(uint32_t *lds, uint32_t slot, uint32_t v)
{
    __hip_atomic_fetch_add(lds + slot, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ uint32_t lds_add_rtn(uint32_t *lds, uint32_t slot, uint32_t v)
{
    return __hip_atomic_fetch_add(lds + slot, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// v << (sh mod 32), the shift as the hardware does it: VOP shifts read only
// the low five bits of the amount, so a caller need not mask it (in C++ a
// shift by 32 or more is undefined, and a mask would cost an instruction).
__device__ __forceinline__ uint32_t shl_mod32(uint32_t v, uint32_t sh)
{
    uint32_t r;
    asm("v_lshlrev_b32_e64 %0, %1, %2" : "=v"(r) : "v"(sh), "v"(v));
    return r;
}

// A returning add to the dynamic LDS word at byte address a. A kernel that
// declares no static LDS has its dynamic block at LDS address 0, so an offset
// into the block is the address itself and needs no base added per access.
// Only kernels with no static LDS may use this; a compiler check keeps them so.
typedef __attribute__((address_space(3))) uint32_t lds_u32;
__device__ __forceinline__ uint32_t dyn_lds_add_rtn(uint32_t a, uint32_t v)
{
    return __hip_atomic_fetch_add((lds_u32 *)(uintptr_t)a, v, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Add one to lds[slot] for every lane with valid set.
//
// ROUNDS > 0 adds a bounded wave-level duplicate aggregation in front of the
// LDS atomics: the lowest pending lane's slot is broadcast (readlane), the
// lanes holding the same slot are found with one ballot, and a single lane
// adds their popcount. Matched lanes retire. After ROUNDS rounds, or as soon
// as a round finds no duplicate, the remaining lanes add one each. Skewed
// inputs (a hot bin taking many lanes of a wave) then cost one atomic per
// distinct hot slot instead of one per lane. Every ballot runs on all active
// lanes, so callers keep control flow wave-uniform around it.
template <int ROUNDS>
__device__ __forceinline__ void lds_count(uint32_t *lds, uint32_t slot, bool valid)
{
    if constexpr (ROUNDS == 0) {
        if (valid) lds_add(lds, slot, 1u);
    } else {
        bool pending = valid;
#pragma unroll
        for (int k = 0; k < ROUNDS; ++k) {
            const uint64_t act = __ballot(pending);
            if (act == 0) return;
            const int leader = __builtin_ctzll(act);
            const uint32_t lead = __builtin_amdgcn_readlane(slot, leader);
            const bool mine = pending && slot == lead;
            const uint64_t m = __ballot(mine);
            if (mine && lane_id() == (uint32_t)leader) lds_add(lds, lead, (uint32_t)__popcll(m));
            pending = pending && !mine;
            if (__popcll(m) == 1) break;
        }
        if (pending) lds_add(lds, slot, 1u);
    }
}

// Wave-level duplicate aggregation by a hot slot kept in registers.
//
// A wave holds one wave-uniform "hot" slot h and a per-lane count c. Lanes
// whose element is h add to c instead of issuing an LDS atomic; the wave
// flushes c (one wave reduction, one LDS add) when h changes and at the end.
// h is chosen from the data as it streams: once per vector the wave takes the
// first active lane's slot (readfirstlane) as a candidate and counts, with two
// ballots, how many lanes hold it and how many hold h; the candidate replaces
// h only when it holds at least 8 of the 64 lanes and clearly more than h.
// A hot bin (a tenth of the input on one value) is then counted almost
// entirely in registers, while uniform data never selects a slot and pays
// one compare per element.
constexpr uint32_t kNoSlot = 0xFFFFFFFFu;

struct HotSlot {
    uint32_t h = kNoSlot;  // wave-uniform
    uint32_t c = 0;        // per lane
    uint32_t tick = 0;     // wave-uniform: candidates are checked every 4th vector
};

// The sum over the wave's 64 lanes, in every lane (all lanes active).
__device__ __forceinline__ uint32_t wave_sum(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(v), 63);
}

// The wave's pending count for h, summed (whole wave, convergent).
__device__ __forceinline__ uint32_t hot_take(HotSlot &hs)
{
    const uint32_t total = hs.h == kNoSlot ? 0u : wave_sum(hs.c);
    hs.c = 0;
    return total;
}

// Returns true when the wave must flush its old hot slot (call hot_take and
// add the total to the old slot, then set hs.h = *next). Whole wave.
__device__ __forceinline__ bool hot_should_switch(HotSlot &hs, uint32_t s0, bool v0,
                                                  uint32_t *next)
{
    if ((hs.tick++ & 3u) != 0u) return false;
    const uint64_t act = __ballot(v0);
    if (act == 0) return false;
    const uint32_t cand = __builtin_amdgcn_readlane(s0, __builtin_ctzll(act));
    if (cand == hs.h) return false;
    const uint32_t mc = (uint32_t)__popcll(__ballot(v0 && s0 == cand));
    if (mc < 8) return false;
    const uint32_t mh = (uint32_t)__popcll(__ballot(v0 && s0 == hs.h));
    if (mc <= mh + 4) return false;
    *next = cand;
    return true;
}

template <bool NT>
__device__ __forceinline__ i32x4 load_vec(const i32x4 *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <int WG>
__device__ __forceinline__ void zero_lds(uint32_t *lds, uint32_t len)
{
    u32x4 *l4 = reinterpret_cast<u32x4 *>(lds);
    const uint32_t len4 = (len + 3) >> 2;
    for (uint32_t i = threadIdx.x; i < len4; i += WG) l4[i] = u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// Fill counts with zeros (n == 0).
__global__ void k_fill_zero(uint32_t *__restrict__ dst, uint64_t len)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < len;
         i += (uint64_t)gridDim.x * blockDim.x)
        dst[i] = 0u;
}

}  // namespace pca
