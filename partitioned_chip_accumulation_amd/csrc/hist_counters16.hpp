// hist_counters16.hpp -- 16-bit LDS counters kept exact by carry events
//
// Part of the gfx950 kernels of libpca_hist.so (see hist_kernels.hpp for the
// overview).
#pragma once

#include "hist_common.hpp"

namespace pca {

// ---------------------------------------------------------------------------
// 16-bit LDS counters.
//
// Two bins share one 32-bit LDS word (bin 2w in the low half, 2w+1 in the
// high half), which doubles the bins one workgroup can own. Increments are
// ds_add_rtn_u32 of 1 or 1 << 16 (or k, k << 16 after wave aggregation), and
// the returned old value exposes the two ways a half can overflow: the low
// half wrapping (its carry then lands in the high half) and a carry out of
// the whole word. Each such event is appended to a short LDS list. With A_lo
// and A_hi the true counts, W the final word, L the low-half wraps and C the
// carries out of the word:
//     A_lo = (W & 0xFFFF) + 65536 L,   A_hi = (W >> 16) + 65536 C - L.
// Each low wrap needs 65536 low increments and each carry out 2^32 of added
// weight, so a workgroup that counts E elements logs at most 2E / 65536
// events; the host keeps E <= 2^24, which bounds the list at 512 of its
// kEventCap entries.
constexpr uint32_t kEventCap = 1024;
constexpr uint32_t kEvLoWrap = 0x40000000u;
constexpr uint32_t kEvCarry = 0x80000000u;

__device__ __forceinline__ void add16(uint32_t *words, uint32_t *evlist, uint32_t *ev_count,
                                      uint32_t s, uint32_t k)
{
    const uint32_t w = s >> 1;
    const bool hi = (s & 1u) != 0;
    const uint32_t delta = hi ? (k << 16) : k;
    const uint32_t old = lds_add_rtn(words, w, delta);
    const bool lo_wrap = !hi && (old & 0xFFFFu) + k > 0xFFFFu;
    const bool carry = old > 0xFFFFFFFFu - delta;
    if (lo_wrap || carry) {
        const uint32_t i = lds_add_rtn(ev_count, 0, 1u);
        if (i < kEventCap) evlist[i] = w | (lo_wrap ? kEvLoWrap : 0u) | (carry ? kEvCarry : 0u);
    }
}

// Unaggregated 16-bit counting of N elements at once: every ds_add_rtn_u32 is
// issued before any returned value is examined, so the wave waits for LDS
// once per batch instead of once per element (N <= 15 keeps the batch within
// the LDS wait counter). An event is possible only when the half being
// incremented was 0xFFFF, which one bit-field extract tests; the rare
// events then take one wave-uniform branch.
template <int N>
__device__ __forceinline__ void count16_batch(uint32_t *words, uint32_t *evlist, uint32_t *ev_count,
                                              const uint32_t (&s)[N], const bool (&ok)[N])
{
    uint32_t old[N], sh[N];
#pragma unroll
    for (int e = 0; e < N; ++e) {
        sh[e] = (s[e] & 1u) << 4;
        old[e] = 0u;
        if (ok[e]) old[e] = lds_add_rtn(words, s[e] >> 1, 1u << sh[e]);
    }
    bool any = false;
#pragma unroll
    for (int e = 0; e < N; ++e)
        any = any || (ok[e] && __builtin_amdgcn_ubfe(old[e], sh[e], 16) == 0xFFFFu);
    if (__ballot(any)) {
#pragma unroll
        for (int e = 0; e < N; ++e) {
            if (ok[e] && __builtin_amdgcn_ubfe(old[e], sh[e], 16) == 0xFFFFu) {
                // low half full: it wraps, and the whole word carries out if the
                // high half was full too; high half full: the word carries out.
                const bool hi = sh[e] != 0u;
                const uint32_t ev = (hi ? 0u : kEvLoWrap) |
                                    ((hi || (old[e] >> 16) == 0xFFFFu) ? kEvCarry : 0u);
                const uint32_t i = lds_add_rtn(ev_count, 0, 1u);
                if (i < kEventCap) evlist[i] = (s[e] >> 1) | ev;
            }
        }
    }
}

template <int ROUNDS>
__device__ __forceinline__ void lds_count16(uint32_t *words, uint32_t *evlist, uint32_t *ev_count,
                                            uint32_t slot, bool valid)
{
    if constexpr (ROUNDS == 0) {
        if (valid) add16(words, evlist, ev_count, slot, 1u);
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
            if (mine && lane_id() == (uint32_t)leader)
                add16(words, evlist, ev_count, lead, (uint32_t)__popcll(m));
            pending = pending && !mine;
            if (__popcll(m) == 1) break;
        }
        if (pending) add16(words, evlist, ev_count, slot, 1u);
    }
}

}  // namespace pca
