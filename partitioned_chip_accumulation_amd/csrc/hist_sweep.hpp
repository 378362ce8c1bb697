// hist_sweep.hpp -- the single-pass sweep (FULL and RANGE paths)
//
// Part of the gfx950 kernels of libpca_hist.so (see hist_kernels.hpp for the
// overview).
#pragma once

#include "hist_common.hpp"
#include "hist_counters16.hpp"
#include "hist_counters8.hpp"
#include "hist_partials.hpp"

namespace pca {

// Co-owner pacing of the RANGE sweep (see k_sweep): where each workgroup keeps
// its progress word, the run's epoch (the word's top 12 bits, so that words
// left by an earlier run read as "not started"), and how many batches a
// workgroup may run ahead of the next range's owner of its chunk.
struct Pacing {
    uint32_t *prog;  // [groups][ranges], or null: plain loads without pacing
    uint32_t epoch;  // 0 .. 4095
    uint32_t window; // batches
};
constexpr uint32_t kPaceDone = 0xFFFFFu;     // batch field of a workgroup that has finished
constexpr uint32_t kPaceSpin = 4096;         // LDS polls before a wave stops waiting for good
constexpr uint32_t kPacerRounds = 1u << 20;  // rounds before the pacer wave gives up

__device__ __forceinline__ uint32_t pace_batch(uint32_t word, uint32_t epoch)
{
    return (word >> 20) == epoch ? (word & 0xFFFFFu) : 0u;
}

// ---------------------------------------------------------------------------
// Sweep: workgroup (g, r) counts chunk g of the input into bin range r.
//
// The page's kernel zeroes its slice, synchronises, accumulates, synchronises
// and flushes (section "The cluster histogram"); the same zero -> barrier ->
// accumulate -> barrier -> write shape runs here at workgroup scope, with the
// owner filter replacing the remote atomic: an element x lands in this
// workgroup's LDS iff lo <= x < lo + len, at slot x - lo (one unsigned
// compare, which also rejects negatives and values >= num_bins).
//
// With ranges == 1 every workgroup owns all bins. With ranges > 1 the R
// owners of a chunk all read it; xcds > 1 places them on one XCD
// (workgroups are dispatched to the XCDs round-robin) so that one owner's
// read brings the lines into the shared L2 for the others. Counters are
// 32-bit (CW = 32), or packed 16-bit or 8-bit ones with carry events
// (CW = 16, 8).
//
// Chunk g is body vectors [g * nvec / groups, (g + 1) * nvec / groups); the
// head scalars belong to chunk 0 and the tail scalars to the last chunk.
// The slice goes to partial row g in 256-bin blocks (range_bins is a multiple
// of 256), or straight into direct[] (the output) when there is one chunk;
// accumulate != 0 adds to direct[] instead of overwriting it. ev_cap is the
// LDS length of the 8-bit counters' carry-event list, and ev_spill (or null)
// holds kEvSpill8 more entries per workgroup, workgroup b's at b kEvSpill8.
//
// NTL: non-temporal input loads (the lines are not kept for a later reader).
// With false the loads are plain, so that when R > 1 owners read a chunk
// each at its own pace the second reader finds more of the lines still in
// the XCD's L2.
//
// PACE (RANGE, R > 1, packed counters): the owners of a chunk read it with
// plain loads, and each keeps pace with the next range's owner, which reads
// the same lines, so that the lines the first reader brings into the XCD's
// L2 are still there for the second. The last wave of the workgroup does no
// counting: it is the pacer. It publishes the workgroup's progress (the
// counting waves' average batch, which they add up in LDS) with relaxed
// device-scope stores, reads the partner's, and leaves it in LDS, where a
// counting wave that is more than pc.window batches ahead waits for it
// (s_sleep between LDS polls). The pacer's stores never hold up a counting
// wave: a wave's stores and loads share one wait counter, and a store that
// writes through takes microseconds under the input stream. Every wait is
// bounded (a counting wave stops waiting after kPaceSpin polls, the pacer
// after kPacerRounds rounds, e.g. when the partner is not resident). The
// counts do not depend on any of this: every owner counts what it loads.
template <int WG, int UNROLL, int AGG, int CW, bool PACE = false, bool NTL = true>
__global__ __launch_bounds__(WG) void k_sweep(InputView in, uint32_t num_bins, uint32_t range_bins,
                                              uint32_t ranges, uint32_t groups, uint32_t xcds,
                                              uint32_t kshift, uint32_t ev_cap,
                                              uint32_t *__restrict__ ev_spill, Partials out,
                                              uint32_t *__restrict__ direct, uint32_t accumulate,
                                              Pacing pc)
{
    extern __shared__ u32x4 lds4[];
    uint32_t *lds = reinterpret_cast<uint32_t *>(lds4);
    uint32_t *ev_count = lds + range_bins * CW / 32;  // CW < 32 only
    uint32_t *evlist = ev_count + 4;
    const EvList ev{evlist, ev_count, CW == 8 ? ev_cap : kEventCap,
                    CW == 8 && ev_spill != nullptr ? ev_spill + (uint64_t)blockIdx.x * kEvSpill8
                                                   : nullptr};
    const uint32_t tid = threadIdx.x;
    const uint32_t b = blockIdx.x;
    uint32_t g, r;
    if (xcds > 1) {
        const uint32_t x = b % xcds, k = b / xcds;
        r = k % ranges;
        g = (k / ranges) * xcds + x;
    } else {
        g = b / ranges;
        r = b % ranges;
    }
    const uint32_t lo = r * range_bins;
    const uint32_t len = min(range_bins, num_bins - lo);

    const i32x4 *body = reinterpret_cast<const i32x4 *>(in.ptr + in.head);
    const uint64_t v0 = (uint64_t)g * in.nvec / groups;
    const uint64_t v1 = (uint64_t)(g + 1) * in.nvec / groups;
    static_assert(!PACE || CW != 32, "pacing keeps its LDS words in the carry-event block");
    constexpr uint32_t CT = PACE ? WG - 64 : WG;  // counting threads (the rest: the pacer wave)
    constexpr uint32_t NCW = CT / 64;             // counting waves
    constexpr uint32_t STEP = CT * UNROLL;
    constexpr bool NT = NTL && !PACE;
    auto ld = [&](const i32x4 *a) __attribute__((always_inline)) { return load_vec<NT>(a); };
    const bool counter = !PACE || tid < CT;
    uint64_t v = v0;

    // PACE: ev_count[1] sums the counting waves' batches, ev_count[2] holds the
    // partner's batch (the pacer's copy), ev_count[3] counts finished waves
    bool pace = false;
    uint32_t kb = 0;
    if constexpr (PACE) pace = pc.prog != nullptr && ranges > 1;

    // The first batch of loads is in flight while the LDS slice is cleared,
    // and every later batch is requested before the previous one is counted,
    // so each wave keeps 2 * UNROLL vector loads outstanding.
    i32x4 nx[UNROLL];
    const bool any_full = v + STEP <= v1;
    if (any_full && counter) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) nx[u] = ld(body + v + u * CT + tid);
    }
    zero_lds<WG>(lds, CW == 32 ? (len << kshift) : CW == 16 ? (len + 1) / 2 : (len + 3) / 4);
    if (CW != 32 && tid < (PACE ? 4u : 1u)) ev_count[tid] = 0u;
    __syncthreads();
    // 32-bit counters may keep 2^kshift interleaved copies of the slice; a lane
    // adds to copy (lane mod 2^kshift), so lanes of one wave that hit the same
    // bin mostly touch different words and banks.
    const uint32_t rep = lane_id() & ((1u << kshift) - 1u);

    // AGG == 1: hot-slot register aggregation in the main loop; the ragged
    // remainder counts plainly. AGG >= 2: leader-peel rounds everywhere.
    constexpr int PEEL = AGG >= 2 ? AGG : 0;
    auto count1 = [&](uint32_t s, bool ok) {
        if constexpr (CW == 32) lds_count<PEEL>(lds, (s << kshift) | rep, ok);
        else if constexpr (CW == 16) lds_count16<PEEL>(lds, evlist, ev_count, s, ok);
        else lds_count8<PEEL>(lds, ev, s, ok);
    };
    HotSlot hs;
    auto hot_flush = [&]() {
        if constexpr (AGG == 1) {
            uint32_t t = hot_take(hs);
            if (lane_id() == 0 && t != 0u) {
                if constexpr (CW == 32) {
                    lds_add(lds, hs.h << kshift, t);
                } else {
                    while (t != 0u) {
                        const uint32_t kk = min(t, CW == 16 ? 32768u : 255u);
                        if constexpr (CW == 16) add16(lds, evlist, ev_count, hs.h, kk);
                        else add8(lds, ev, hs.h, kk);
                        t -= kk;
                    }
                }
            }
        }
    };
    auto hot_check = [&](uint32_t s0, bool v0) {
        if constexpr (AGG == 1) {
            uint32_t nxt;
            if (hot_should_switch(hs, s0, v0, &nxt)) {
                hot_flush();
                hs.h = nxt;
            }
        }
    };
    auto count4 = [&](const i32x4 q, bool ok) {
        uint32_t s;
        s = (uint32_t)q.x - lo; count1(s, ok && s < len);
        s = (uint32_t)q.y - lo; count1(s, ok && s < len);
        s = (uint32_t)q.z - lo; count1(s, ok && s < len);
        s = (uint32_t)q.w - lo; count1(s, ok && s < len);
    };

    if (counter) {
    for (; any_full && v + STEP <= v1; v += STEP) {
        if constexpr (PACE) {
            if (pace) {
                uint32_t spins = 0;
                while (kb > __hip_atomic_load(ev_count + 2, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_WORKGROUP) + pc.window) {
                    if (++spins > kPaceSpin) {
                        pace = false;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
        }
        i32x4 q[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) q[u] = nx[u];
        if (v + 2 * STEP <= v1) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) nx[u] = ld(body + v + STEP + u * CT + tid);
        }
        if constexpr (PACE) {
            if (lane_id() == 0) lds_add(ev_count, 1, 1u);
            ++kb;
        }
        if constexpr (AGG <= 1) {
            uint32_t sl[4 * UNROLL];
            bool ok[4 * UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                sl[4 * u + 0] = (uint32_t)q[u].x - lo;
                sl[4 * u + 1] = (uint32_t)q[u].y - lo;
                sl[4 * u + 2] = (uint32_t)q[u].z - lo;
                sl[4 * u + 3] = (uint32_t)q[u].w - lo;
            }
#pragma unroll
            for (int e = 0; e < 4 * UNROLL; ++e) ok[e] = sl[e] < len;
            if constexpr (AGG == 1) {
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) hot_check(sl[4 * u], ok[4 * u]);
                if (hs.h != kNoSlot) {
#pragma unroll
                    for (int e = 0; e < 4 * UNROLL; ++e) {
                        const bool m = ok[e] && sl[e] == hs.h;
                        hs.c += m ? 1u : 0u;
                        ok[e] = ok[e] && !m;
                    }
                }
            }
            if constexpr (CW == 16) {
                count16_batch<4 * UNROLL>(lds, evlist, ev_count, sl, ok);
            } else if constexpr (CW == 8) {
                count8_batch<4 * UNROLL>(ev, sl, ok);
            } else {
#pragma unroll
                for (int e = 0; e < 4 * UNROLL; ++e) lds_count<0>(lds, (sl[e] << kshift) | rep, ok[e]);
            }
        } else {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) count4(q[u], true);
        }
    }
    if constexpr (PACE) {
        if (lane_id() == 0) lds_add(ev_count, 3, 1u);  // this wave is done with the stream
    }
    // Remainder with a wave-uniform trip count.
    for (; v < v1; v += CT) {
        const bool ok = v + tid < v1;
        const i32x4 q = ok ? ld(body + v + tid) : i32x4{0, 0, 0, 0};
        count4(q, ok);
    }
    {
        const bool hok = g == 0 && tid < in.head;
        const uint32_t hs = (hok ? (uint32_t)in.ptr[tid] : 0u) - lo;
        count1(hs, hok && hs < len);
        const bool tok = g == groups - 1 && tid < in.tail;
        const uint32_t ts = (tok ? (uint32_t)in.ptr[in.head + 4 * in.nvec + tid] : 0u) - lo;
        count1(ts, tok && ts < len);
    }
    } else if constexpr (PACE) {
        // The pacer wave: publish this workgroup's progress, fetch the
        // partner's into LDS, until every counting wave is done (or, bounded,
        // kPacerRounds rounds: then the counting waves stop waiting).
        uint32_t *my_prog = pc.prog + (uint64_t)g * ranges + r;
        const uint32_t *pa_prog = pc.prog + (uint64_t)g * ranges + (r + 1) % ranges;
        for (uint32_t round = 0; pace; ++round) {
            const uint32_t done =
                __hip_atomic_load(ev_count + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            const uint32_t mine =
                __hip_atomic_load(ev_count + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) / NCW;
            if (lane_id() == 0)
                __hip_atomic_store(my_prog, (pc.epoch << 20) | (done == NCW ? kPaceDone : mine),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (done == NCW) break;
            uint32_t pk = pace_batch((uint32_t)__builtin_amdgcn_readfirstlane((int)__hip_atomic_load(
                                         pa_prog, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)),
                                     pc.epoch);
            if (round >= kPacerRounds) pk = kPaceDone;  // give up: nobody waits any more
            if (lane_id() == 0)
                __hip_atomic_store(ev_count + 2, pk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (pk == kPaceDone) break;
            __builtin_amdgcn_s_sleep(4);
        }
    }
    hot_flush();
    __syncthreads();

    // (the barrier above also makes the spilled entries, plain global stores
    // of this workgroup, visible to all its waves)
    const uint32_t nev = CW == 16 ? min(*ev_count, kEventCap) : CW == 8 ? events8_held(ev) : 0u;
    if (direct) {
        const uint32_t npairs = (len + 511) / 512;
        for (uint32_t p = tid >> 6; p < npairs; p += WG / 64) {
            uint32_t c[8];
            slice_octet<CW>(lds, ev, nev, p, len, kshift, c);
            const uint32_t b0 = lo + p * 512 + lane_id() * 8;
#pragma unroll
            for (uint32_t i = 0; i < 8; ++i)
                if (b0 + i < num_bins && b0 + i - lo < len)
                    direct[b0 + i] = (accumulate ? direct[b0 + i] : 0u) + c[i];
        }
    } else {
        flush_slice<WG, CW>(out, g, lo / kBlockBins, lds, ev, nev, len, kshift);
    }
}

}  // namespace pca
