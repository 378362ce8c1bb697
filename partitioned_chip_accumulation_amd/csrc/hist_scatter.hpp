// hist_scatter.hpp -- the two-phase path (SCATTER): partition, range scans,
// per-owner histograms, slot merge
//
// Part of the gfx950 kernels of libpca_hist.so (see hist_kernels.hpp for the
// overview).
#pragma once

#include "hist_common.hpp"
#include "hist_partials.hpp"

namespace pca {

// ---------------------------------------------------------------------------
// Two-phase path.
// WG-wide exclusive scan of one value per thread; returns this thread's
// exclusive prefix and writes the total to *total (all threads).
template <int WG>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *scratch,
                                                         uint32_t *total)
{
    constexpr int NW = WG / 64;
    const uint32_t lane = lane_id(), w = threadIdx.x >> 6;
    const uint32_t incl = wave_inclusive_scan(v);
    if (lane == 63) scratch[w] = incl;
    __syncthreads();
    if (w == 0) {
        const uint32_t s = lane < (uint32_t)NW ? scratch[lane] : 0u;
        const uint32_t si = wave_inclusive_scan(s);
        if (lane < (uint32_t)NW) scratch[NW + lane] = si - s;
        if (lane == 63) scratch[2 * NW] = si;
    }
    __syncthreads();
    *total = scratch[2 * NW];
    return scratch[NW + w] + incl - v;
}

// The same with one barrier: every wave scans the per-wave totals itself.
// scratch holds WG / 64 words, which the caller must not write again before
// its next barrier.
template <int WG>
__device__ __forceinline__ uint32_t block_exclusive_scan_1b(uint32_t v, uint32_t *scratch,
                                                            uint32_t *total)
{
    constexpr int NW = WG / 64;
    const uint32_t lane = lane_id(), w = threadIdx.x >> 6;
    const uint32_t incl = wave_inclusive_scan(v);
    if (lane == 63) scratch[w] = incl;
    __syncthreads();
    static_assert(NW <= 16, "the wave totals fit one row of 16 lanes");
    const uint32_t s = lane < (uint32_t)NW ? scratch[lane] : 0u;
    const uint32_t si = row_inclusive_scan(s);
    *total = (uint32_t)__builtin_amdgcn_readlane((int)si, NW - 1);
    const uint32_t before = (uint32_t)__builtin_amdgcn_readlane(
        (int)(si - s), __builtin_amdgcn_readfirstlane((int)w));
    return before + incl - v;
}

// Phase 1b: per range r, tpre[r][t] = sum of tcnt[r][t'] over t' < t, and
// totals[r] = the range's element count. Two passes, both spread over
// (range, segment of kScanSeg tiles) workgroups so that every CU takes part:
// k_seg_scan writes each segment's local exclusive prefix and its total,
// k_seg_fix adds the totals of the range's earlier segments (and the last
// segment's workgroup writes the range total).
constexpr uint32_t kScanSeg = 4096;

template <int WG>
__global__ __launch_bounds__(WG) void k_seg_scan(const uint32_t *__restrict__ tcnt, uint32_t tiles,
                                                 uint32_t nseg, uint32_t *__restrict__ tpre,
                                                 uint32_t *__restrict__ segtot)
{
    __shared__ uint32_t scratch[2 * (WG / 64) + 1];
    const uint32_t r = blockIdx.x / nseg, sg = blockIdx.x % nseg, tid = threadIdx.x;
    const uint32_t s0 = sg * kScanSeg, s1 = min(s0 + kScanSeg, tiles);
    const uint32_t *c = tcnt + (uint64_t)r * tiles;
    uint32_t *p = tpre + (uint64_t)r * tiles;
    constexpr uint32_t PER = kScanSeg / WG;
    const uint32_t t0 = s0 + tid * PER;
    uint32_t v[PER], sum = 0;
#pragma unroll
    for (uint32_t k = 0; k < PER; ++k) {
        v[k] = t0 + k < s1 ? c[t0 + k] : 0u;
        sum += v[k];
    }
    uint32_t total;
    uint32_t run = block_exclusive_scan<WG>(sum, scratch, &total);
#pragma unroll
    for (uint32_t k = 0; k < PER; ++k) {
        if (t0 + k < s1) p[t0 + k] = run;
        run += v[k];
    }
    if (tid == 0) segtot[(uint64_t)r * nseg + sg] = total;
}

template <int WG>
__global__ __launch_bounds__(WG) void k_seg_fix(uint32_t tiles, uint32_t nseg,
                                                uint32_t *__restrict__ tpre,
                                                const uint32_t *__restrict__ segtot,
                                                uint32_t *__restrict__ totals)
{
    const uint32_t r = blockIdx.x / nseg, sg = blockIdx.x % nseg, tid = threadIdx.x;
    const uint32_t *st = segtot + (uint64_t)r * nseg;
    uint32_t off = 0;
    for (uint32_t k = 0; k < sg; ++k) off += st[k];
    if (sg == nseg - 1 && tid == 0) totals[r] = off + st[sg];
    if (off == 0) return;
    uint32_t *p = tpre + (uint64_t)r * tiles;
    const uint32_t s0 = sg * kScanSeg, s1 = min(s0 + kScanSeg, tiles);
    for (uint32_t t = s0 + tid; t < s1; t += WG) p[t] += off;
}

// The same in one pass for a range of at most WG * PER tiles: one
// workgroup per range loads all its run lengths at once, row by row (tile k
// * WG + thread, so every load and store is one contiguous row), scans each
// row across its waves, and wave 0 scans the (row, wave) totals in row-major
// order, which is the tiles' order. Two barriers and one memory round trip,
// where the two passes above take two kernels.
template <int WG, int PER>
__global__ __launch_bounds__(WG) void k_range_scan(const uint32_t *__restrict__ tcnt, uint32_t tiles,
                                                   uint32_t *__restrict__ tpre,
                                                   uint32_t *__restrict__ totals)
{
    constexpr uint32_t NW = WG / 64, NT = PER * NW;
    static_assert(NT % 64 == 0 && NT <= 64 * 8, "wave 0 scans the totals, 8 per lane");
    __shared__ uint32_t tot[NT + 1];
    const uint32_t r = blockIdx.x, tid = threadIdx.x, w = tid >> 6, lane = lane_id();
    const uint32_t *c = tcnt + (uint64_t)r * tiles;
    uint32_t *p = tpre + (uint64_t)r * tiles;
    const uint32_t rows = (tiles + WG - 1) / WG;  // <= PER
    uint32_t v[PER], incl[PER];
#pragma unroll
    for (uint32_t k = 0; k < PER; ++k) v[k] = k < rows && k * WG + tid < tiles ? c[k * WG + tid] : 0u;
#pragma unroll
    for (uint32_t k = 0; k < PER; ++k) {
        incl[k] = 0u;
        if (k < rows) {  // uniform
            incl[k] = wave_inclusive_scan(v[k]);
            if (lane == 63) tot[k * NW + w] = incl[k];
        }
    }
    __syncthreads();
    if (w == 0) {
        constexpr uint32_t E = NT / 64;
        uint32_t a[E], sum = 0;
#pragma unroll
        for (uint32_t i = 0; i < E; ++i) {
            const uint32_t at = lane * E + i;
            a[i] = at < rows * NW ? tot[at] : 0u;
            sum += a[i];
        }
        const uint32_t in = wave_inclusive_scan(sum);
        uint32_t run = in - sum;
#pragma unroll
        for (uint32_t i = 0; i < E; ++i) {
            tot[lane * E + i] = run;
            run += a[i];
        }
        if (lane == 63) tot[NT] = in;
    }
    __syncthreads();
#pragma unroll
    for (uint32_t k = 0; k < PER; ++k)
        if (k < rows && k * WG + tid < tiles) p[k * WG + tid] = tot[k * NW + w] + incl[k] - v[k];
    if (tid == 0) totals[r] = tot[NT];
}

// Two [rows][cols] uint32 tables (blockIdx.z picks which) to [cols][rows],
// through LDS in 64 x 64 tiles: reads and writes are both 256-byte rows.
__global__ __launch_bounds__(256) void k_transpose(const uint32_t *__restrict__ src0,
                                                   uint32_t *__restrict__ dst0,
                                                   const uint32_t *__restrict__ src1,
                                                   uint32_t *__restrict__ dst1, uint32_t rows,
                                                   uint32_t cols)
{
    __shared__ uint32_t tile[64][65];  // padded: a column read hits 64 banks
    const uint32_t *src = blockIdx.z == 0 ? src0 : src1;
    uint32_t *dst = blockIdx.z == 0 ? dst0 : dst1;
    const uint32_t c0 = blockIdx.x * 64u, r0 = blockIdx.y * 64u;
    const uint32_t tx = threadIdx.x & 63u, ty = threadIdx.x >> 6;
    for (uint32_t i = ty; i < 64u; i += 4u) {
        const uint32_t r = r0 + i, c = c0 + tx;
        if (r < rows && c < cols) tile[i][tx] = src[(uint64_t)r * cols + c];
    }
    __syncthreads();
    for (uint32_t i = ty; i < 64u; i += 4u) {
        const uint32_t c = c0 + i, r = r0 + tx;
        if (c < cols && r < rows) dst[(uint64_t)c * rows + r] = tile[tx][i];
    }
}

// Exclusive prefix of totals[0..ranges) into bs[0..ranges], by wave 0.
__device__ __forceinline__ void range_starts(const uint32_t *__restrict__ totals, uint32_t ranges,
                                             uint64_t *bs)
{
    if (threadIdx.x < 64) {
        const uint32_t lane = threadIdx.x;
        uint64_t carry = 0;
        for (uint32_t c = 0; c < ranges; c += 64) {
            const uint32_t i = c + lane;
            const uint32_t v = i < ranges ? totals[i] : 0u;
            const uint32_t incl = wave_inclusive_scan(v);  // < 2^32: sum of <= 64 counts of one call
            if (i < ranges) bs[i] = carry + incl - v;
            carry += __shfl(incl, 63, 64);
        }
        if (lane == 0) bs[ranges] = carry;
    }
}

// Owner workgroup i of W covers positions [i*N/W, (i+1)*N/W) of the
// concatenation of all ranges' elements; this returns the owner of position p.
__device__ __forceinline__ uint32_t owner_of(uint64_t p, uint64_t N, uint32_t W)
{
    return (uint32_t)(((p + 1) * W - 1) / N);
}

// no in-place window (k_window_pick found none worth it, or none was asked for)
constexpr uint32_t kNoWindow = 0xFFFFFFFFu;
// k_window_pick's words: the window's first bin, whether the owners' hot slot
// has a value to take, the hot value the partition counts in registers
constexpr uint32_t kSelWindow = 0, kSelOwnersHot = 1, kSelHotValue = 2;
// a window-partials row: the window's bins, then the hot value's total
constexpr uint32_t kWindowRowPad = 64;

// Phase 1: route every element of a tile to its owning range.
//
// Tile t is body vectors [t * WG * VPT, ...) (tile 0 also takes the head
// scalars, the last tile the tail scalars). Each valid element x (x <
// num_bins) is owned by range r = x >> shift, where it is slot x & mask. The
// workgroup counts its elements per range in LDS; each element's returning
// LDS atomic gives its rank among the tile's elements of that range, and an
// exclusive scan of the counts gives each range's start, so the tile's slots
// are grouped by range in an LDS staging buffer and copied out with full
// 16-byte stores to stage[t * stage_cap ...]. Only the 16-bit slot is kept:
// the range is implied by the position. Counters and staging buffers come in
// pairs that alternate between tiles, so a tile's copy-out and the clearing
// of its counters wait for no barrier of their own: they run after the next
// tile's ranks, and a tile takes three barriers (ranks done, wave totals
// posted, starts posted).
//
// Returning atomics on one LDS word are served one lane at a time (each lane
// needs its own rank), so every range's counter is split into 2^qlog
// sub-counters chosen by lane (lane mod 2^qlog): lanes that route to the same
// range then rarely share a word. The scan runs over [range][sub] order, so a
// range's elements stay contiguous. Per tile and range the kernel writes the
// run's length and start (tcnt, tbase) at r * rstride + t * tstride: range-
// major ([range][tile], rstride = tiles, tstride = 1) for few ranges. With
// many ranges those are 4-byte stores a whole row apart, each a partial-line
// write, so the tables are written tile-major (rstride = 1, tstride = ranges)
// and k_transpose turns them range-major. Element order inside a run is
// whatever the atomics gave; counts do not depend on it.

template <int WG, int VPT, bool NTS = true>
__global__ __launch_bounds__(WG) void k_partition(InputView in, uint32_t num_bins, uint32_t shift,
                                                  uint32_t ranges, uint32_t qlog, uint32_t tiles,
                                                  uint16_t *__restrict__ stage, uint32_t stage_cap,
                                                  uint32_t *__restrict__ tcnt,
                                                  uint32_t *__restrict__ tbase, uint32_t rstride,
                                                  uint32_t tstride, const uint32_t *__restrict__ wsel,
                                                  uint32_t wbins, uint32_t *__restrict__ wpart)
{
    extern __shared__ u32x4 smem4[];
    const uint32_t nsub = ranges << qlog;  // <= 2 * WG
    const uint32_t npad = (nsub + 3u) & ~3u;
    uint32_t *cnt = reinterpret_cast<uint32_t *>(smem4);  // two sets of npad
    uint32_t *base = cnt + 2 * npad;
    uint32_t *scratch = base + npad;  // block scan scratch
    uint16_t *st = reinterpret_cast<uint16_t *>(scratch + 64);  // two buffers of stage_cap
    // the in-place window: bins [w0, w0 + hw) are counted here, not staged;
    // so is the hot value hv (k_window_pick), in a register of each lane
    uint32_t *win = reinterpret_cast<uint32_t *>(st + 2 * stage_cap);  // [wbins], then the hot total
    const uint32_t w0 = wsel ? wsel[kSelWindow] : kNoWindow;
    const uint32_t hw = w0 == kNoWindow ? 0u : min(wbins, num_bins - w0);
    const uint32_t hv = wsel ? wsel[kSelHotValue] : kNoWindow;
    uint32_t hc = 0;
    const uint32_t tid = threadIdx.x;
    const uint32_t mask = (1u << shift) - 1u;
    const uint32_t q = lane_id() & ((1u << qlog) - 1u);
    constexpr int E = VPT * 4;
    const i32x4 *body = reinterpret_cast<const i32x4 *>(in.ptr + in.head);

    // A persistent workgroup walks tiles blockIdx.x, + gridDim.x, ...; the
    // next tile's elements are loaded while the current one is counted.
    uint32_t nx[E + 2];
    auto load_tile = [&](uint32_t t) {
        const uint64_t vb = (uint64_t)t * (WG * VPT);
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const uint64_t v = vb + (uint64_t)u * WG + tid;
            const i32x4 qv = v < in.nvec ? body[v] : i32x4{-1, -1, -1, -1};
            nx[4 * u + 0] = (uint32_t)qv.x;
            nx[4 * u + 1] = (uint32_t)qv.y;
            nx[4 * u + 2] = (uint32_t)qv.z;
            nx[4 * u + 3] = (uint32_t)qv.w;
        }
        nx[E] = (t == 0 && tid < in.head) ? (uint32_t)in.ptr[tid] : 0xFFFFFFFFu;
        nx[E + 1] = (t == tiles - 1 && tid < in.tail) ? (uint32_t)in.ptr[in.head + 4 * in.nvec + tid]
                                                      : 0xFFFFFFFFu;
    };
    // the previous tile's slots, still in its staging buffer: 16-byte vectors, tile
    uint32_t prev_nv = 0, prev_t = 0;
    // NTS: non-temporal stores, for staged slots that outgrow the
    // Infinity Cache (the host's choice); plain ones keep smaller runs there
    // for the owners
    auto copy_out = [&](uint32_t buf) {
        const u32x4 *s4 = reinterpret_cast<const u32x4 *>(st + buf * stage_cap);
        u32x4 *d4 = reinterpret_cast<u32x4 *>(stage + (uint64_t)prev_t * stage_cap);
        for (uint32_t i = tid; i < prev_nv; i += WG) {
            if constexpr (NTS) __builtin_nontemporal_store(s4[i], d4 + i);
            else d4[i] = s4[i];
        }
    };
    uint32_t t = blockIdx.x;
    if (t < tiles) load_tile(t);
    for (uint32_t i = tid; i < 2 * npad; i += WG) cnt[i] = 0u;
    for (uint32_t i = tid; i < hw; i += WG) win[i] = 0u;
    if (wsel && tid == 0) win[wbins] = 0u;
    __syncthreads();

    uint32_t b = 0;  // this tile's counters and staging buffer
    for (; t < tiles; t += gridDim.x, b ^= 1u) {
        uint32_t *cb = cnt + b * npad;
        uint16_t *sb = st + b * stage_cap;
        uint32_t x[E + 2], rk[E + 2];
#pragma unroll
        for (int e = 0; e < E + 2; ++e) x[e] = nx[e];
        if (t + gridDim.x < tiles) load_tile(t + gridDim.x);
        if (hw) {
            // the window's elements first: counted, then neither ranked nor
            // staged. The add alone sits under the branch and the marking is
            // a select: a register written under a branch would make the
            // compiler copy the whole array there and wait for the next
            // tile's loads.
#pragma unroll
            for (int e = 0; e < E + 2; ++e) {
                const uint32_t wi = x[e] - w0;
                if (wi < hw) lds_add(win, wi, 1u);
            }
#pragma unroll
            for (int e = 0; e < E + 2; ++e) x[e] = x[e] - w0 < hw ? 0xFFFFFFFFu : x[e];
        }
        if (hv != kNoWindow) {  // the hot value's copies: a register count, no LDS
#pragma unroll
            for (int e = 0; e < E + 2; ++e) {
                const bool m = x[e] == hv;
                hc += m ? 1u : 0u;
                x[e] = m ? 0xFFFFFFFFu : x[e];
            }
        }
#pragma unroll
        for (int e = 0; e < E + 2; ++e) {
            rk[e] = 0u;
            if (x[e] < num_bins) rk[e] = lds_add_rtn(cb, ((x[e] >> shift) << qlog) | q, 1u);
        }
        __syncthreads();  // this tile's ranks are in; the previous tile's slots are staged

        // the previous tile goes out, and its counters are cleared for the next
        copy_out(b ^ 1u);
        {
            uint32_t *co = cnt + (b ^ 1u) * npad;
            for (uint32_t i = tid; i < nsub; i += WG) co[i] = 0u;
        }
        uint32_t nvalid;
        {
            const uint32_t i0 = 2 * tid, i1 = 2 * tid + 1;
            const uint32_t c0 = i0 < nsub ? cb[i0] : 0u, c1 = i1 < nsub ? cb[i1] : 0u;
            const uint32_t ex = block_exclusive_scan_1b<WG>(c0 + c1, scratch, &nvalid);
            if (i0 < nsub) base[i0] = ex;
            if (i1 < nsub) base[i1] = ex + c0;
        }
        __syncthreads();  // the starts are posted
        for (uint32_t r = tid; r < ranges; r += WG) {
            const uint32_t b0 = base[r << qlog];
            const uint32_t b1 = r + 1 < ranges ? base[(r + 1) << qlog] : nvalid;
            const uint64_t at = (uint64_t)r * rstride + (uint64_t)t * tstride;
            tcnt[at] = b1 - b0;
            tbase[at] = b0;
        }
        // every element's start is read, its own counter's or counter 0's, so
        // that a group of reads waits once; then the valid ones are stored
        constexpr int G = (E + 2) % 6 == 0 ? 6 : 1;
#pragma unroll
        for (int g = 0; g < E + 2; g += G) {
            uint32_t at[G];
#pragma unroll
            for (int k = 0; k < G; ++k) {
                const uint32_t xe = x[g + k];
                at[k] = base[xe < num_bins ? ((xe >> shift) << qlog) | q : 0u] + rk[g + k];
            }
#pragma unroll
            for (int k = 0; k < G; ++k)
                if (x[g + k] < num_bins) sb[at[k]] = (uint16_t)(x[g + k] & mask);
        }
        prev_nv = (nvalid + 7u) >> 3;
        prev_t = t;
    }
    // the last tile's slots
    __syncthreads();
    copy_out(b ^ 1u);
    // the workgroup's window counts and hot-value total: its row of the
    // window partials (kWindowRowPad words past the window's bins)
    if (wsel) {
        const uint32_t hsum = wave_sum(hc);
        if (lane_id() == 0 && hsum) lds_add(win, wbins, hsum);
        __syncthreads();
        uint32_t *row = wpart + (uint64_t)blockIdx.x * (wbins + kWindowRowPad);
        for (uint32_t i = tid; i < hw; i += WG) row[i] = win[i];
        if (tid == 0) row[wbins] = win[wbins];
    }
}

// The heaviest window of wbins consecutive bins, from a sample of the input,
// for k_partition to count in place, and the hottest value outside it. One
// workgroup samples 1,024 elements, 64 runs of 16 S consecutive ones at
// evenly spaced places (S = 1024 / WG per thread; with WG = 1024, 64 lines on
// 64 pages, which one CU fetches in a few microseconds while the rest of the
// GPU waits; single elements from 1,024 pages took the half-Gaussian 2^19-bin
// workload 652 against 644 us, the page walks setting the time). For input in
// random order a share's standard error stays under 1.6%; on ordered input
// the runs make the estimate coarser, which can only cost time, never
// exactness. The samples are counted into coarse buckets (256
// bins, or more so that there are at most 8,192) and, by value, into an LDS
// hash table; the window is the run of wbins / bucket buckets with the most
// samples (the first such, from a prefix sum). wsel[kSelWindow] gets its
// first bin when it holds at least samples / min_div of the sample (min_div
// 0: always), else kNoWindow. Among the values outside the window, the one
// with the most copies (the largest such value on a tie, so the choice does
// not depend on the order of the atomics), when it holds at least 1/32 of
// the samples, is the hot value (wsel[kSelHotValue], else kNoWindow) that the
// partition counts in registers; wsel[kSelOwnersHot] says whether the next
// value holds at least 1/32 of them too (0: the owners leave their hot slot
// off for this run; its checks would find nothing to take: on Zipf s = 1.1
// over 2^18 bins, whose second value holds 6%, the slot still took a run
// from 598 to 489 us, while on the half-Gaussian it cost 8 us).
template <int WG>
__global__ __launch_bounds__(WG) void k_window_pick(const int32_t *__restrict__ x, uint64_t n,
                                                   uint32_t num_bins, uint32_t wbins,
                                                   uint32_t min_div, uint32_t *__restrict__ wsel)
{
    constexpr uint32_t S = 1024 / WG, kSamples = S * WG, kMaxBuckets = 8192, PER = kMaxBuckets / WG;
    constexpr uint32_t kSlots = 2 * kSamples, kEmpty = 0xFFFFFFFFu, NW = WG / 64;
    static_assert(kSlots == 2048, "the hash gives 11 bits");
    __shared__ uint32_t hist[kMaxBuckets];
    __shared__ uint32_t keys[kSlots], cnts[kSlots];
    __shared__ uint32_t scratch[64];
    const uint32_t tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    // every sample's load goes out before the tables are cleared
    uint32_t v[S];
    const uint64_t at = (uint64_t)(tid >> 4) * n / (WG >> 4) + (tid & 15u) * S;
#pragma unroll
    for (uint32_t k = 0; k < S; ++k) v[k] = (uint32_t)x[min(at + k, n - 1u)];
    uint32_t blog = 8;
    while ((((uint64_t)num_bins + (1u << blog) - 1u) >> blog) > kMaxBuckets) ++blog;
    const uint32_t nb = (uint32_t)(((uint64_t)num_bins + (1u << blog) - 1u) >> blog);
    for (uint32_t i = tid; i < kMaxBuckets; i += WG) hist[i] = 0u;
    for (uint32_t i = tid; i < kSlots; i += WG) {
        keys[i] = kEmpty;
        cnts[i] = 0u;
    }
    __syncthreads();
    // buckets, and counts by value (linear probing; at most kSamples of the
    // 2 * kSamples slots fill, so every probe ends)
#pragma unroll
    for (uint32_t k = 0; k < S; ++k) {
        const uint32_t val = v[k];
        if (val < num_bins) {
            lds_add(hist, val >> blog, 1u);
            uint32_t h = (val * 2654435761u) >> (32 - 11);  // Knuth's multiplicative hash
            for (;;) {
                uint32_t old = kEmpty;
                const bool took = __hip_atomic_compare_exchange_strong(
                    keys + h, &old, val, __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if (took || old == val) {
                    lds_add(cnts, h, 1u);
                    break;
                }
                h = (h + 1u) & (kSlots - 1u);
            }
        }
    }
    __syncthreads();
    // inclusive prefix over the buckets, PER per thread
    uint32_t local[PER], run = 0;
#pragma unroll
    for (uint32_t k = 0; k < PER; ++k) {
        run += hist[tid * PER + k];
        local[k] = run;
    }
    uint32_t total;
    const uint32_t before = block_exclusive_scan<WG>(run, scratch, &total);
    __syncthreads();
#pragma unroll
    for (uint32_t k = 0; k < PER; ++k) hist[tid * PER + k] = before + local[k];
    __syncthreads();
    // window sums: buckets [j, j + wb) = P[j + wb - 1] - P[j - 1]
    const uint32_t wb = max(1u, wbins >> blog);
    uint32_t best = 0;  // sum << 13 | (8191 - j): the largest sum, then the first j
#pragma unroll
    for (uint32_t k = 0; k < PER; ++k) {
        const uint32_t j = tid * PER + k;
        if (j < nb) {
            const uint32_t hi = hist[min(j + wb, nb) - 1u], lo = j ? hist[j - 1u] : 0u;
            best = max(best, ((hi - lo) << 13) | (kMaxBuckets - 1u - j));
        }
    }
    for (int d = 32; d >= 1; d >>= 1) best = max(best, (uint32_t)__shfl_xor((int)best, d, 64));
    if (lane == 0) scratch[w] = best;
    __syncthreads();
    uint32_t m = 0;
#pragma unroll
    for (uint32_t i = 0; i < NW; ++i) m = max(m, scratch[i]);
    const uint32_t bsum = m >> 13, bj = kMaxBuckets - 1u - (m & (kMaxBuckets - 1u));
    const uint32_t w0 = (min_div == 0 || (uint64_t)bsum * min_div >= kSamples) ? (bj << blog) : kNoWindow;
    const uint32_t hw = w0 == kNoWindow ? 0u : min(wbins, num_bins - w0);
    // the two (copies << 32 | value) maxima among the values outside the window
    uint64_t a1 = 0, a2 = 0;
    for (uint32_t i = tid; i < kSlots; i += WG) {
        const uint32_t c = cnts[i], key = keys[i];
        if (c && !(key - w0 < hw)) {
            const uint64_t e = ((uint64_t)c << 32) | key;
            a2 = max(a2, min(a1, e));
            a1 = max(a1, e);
        }
    }
    auto merge2 = [&](uint64_t b1, uint64_t b2) {
        a2 = max(max(a2, b2), min(a1, b1));
        a1 = max(a1, b1);
    };
    for (int d = 32; d >= 1; d >>= 1) {
        auto xchg = [&](uint64_t q) {
            const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)q, d, 64);
            const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(q >> 32), d, 64);
            return ((uint64_t)hi << 32) | lo;
        };
        const uint64_t b1 = xchg(a1), b2 = xchg(a2);
        merge2(b1, b2);
    }
    __syncthreads();  // every wave has read the window maxima
    if (lane == 0) {
        scratch[4 * w + 0] = (uint32_t)a1;
        scratch[4 * w + 1] = (uint32_t)(a1 >> 32);
        scratch[4 * w + 2] = (uint32_t)a2;
        scratch[4 * w + 3] = (uint32_t)(a2 >> 32);
    }
    __syncthreads();
    if (tid == 0) {
        a1 = a2 = 0;
        for (uint32_t i = 0; i < NW; ++i)
            merge2(((uint64_t)scratch[4 * i + 1] << 32) | scratch[4 * i],
                   ((uint64_t)scratch[4 * i + 3] << 32) | scratch[4 * i + 2]);
        const bool hot = (uint32_t)(a1 >> 32) * 32u >= kSamples;
        wsel[kSelWindow] = w0;
        wsel[kSelHotValue] = hot ? (uint32_t)a1 : kNoWindow;
        // the next value: the second maximum, or the first when there is no hot one
        wsel[kSelOwnersHot] = (uint32_t)((hot ? a2 : a1) >> 32) * 32u >= kSamples ? 1u : 0u;
    }
}

// counts[w0 + b] += the sum of the window partials' rows at b, for the bins
// of the window k_window_pick chose (none: nothing). Each workgroup takes
// kWindowMergeBins bins; its thread groups sum every (WG / kWindowMergeBins)-th
// row, 8 loads in flight per lane, then one group adds the partial sums: the
// counts of a bin are written by one thread, with no atomic.
constexpr uint32_t kWindowMergeBins = 64;
template <int WG>
__global__ __launch_bounds__(WG) void k_window_merge(const uint32_t *__restrict__ wsel,
                                                    const uint32_t *__restrict__ wpart, uint32_t rows,
                                                    uint32_t wbins, uint32_t num_bins,
                                                    uint32_t *__restrict__ counts)
{
    constexpr uint32_t NB = kWindowMergeBins, PH = WG / NB, U = 8;
    __shared__ uint32_t part[WG];
    const uint32_t w0 = wsel[kSelWindow], hv = wsel[kSelHotValue];
    if (w0 == kNoWindow && hv == kNoWindow) return;
    const uint64_t stride = wbins + kWindowRowPad;
    if (blockIdx.x == 0 && hv != kNoWindow) {
        // the hot value's total over the rows, by the first workgroup
        uint32_t h = 0;
        for (uint32_t r = threadIdx.x; r < rows; r += WG) h += wpart[(uint64_t)r * stride + wbins];
        h = wave_sum(h);
        if (lane_id() == 0) part[threadIdx.x >> 6] = h;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t t = 0;
            for (uint32_t k = 0; k < WG / 64; ++k) t += part[k];
            counts[hv] += t;
        }
        __syncthreads();  // part is reused below
    }
    if (w0 == kNoWindow) return;
    const uint32_t hw = min(wbins, num_bins - w0);
    const uint32_t b = blockIdx.x * NB + (threadIdx.x & (NB - 1u)), ph = threadIdx.x / NB;
    uint32_t sum = 0;
    if (b < hw) {
        uint32_t r = ph;
        for (; r + PH * (U - 1) < rows; r += PH * U) {
            uint32_t v[U];
#pragma unroll
            for (uint32_t u = 0; u < U; ++u) v[u] = wpart[(uint64_t)(r + PH * u) * stride + b];
#pragma unroll
            for (uint32_t u = 0; u < U; ++u) sum += v[u];
        }
        for (; r < rows; r += PH) sum += wpart[(uint64_t)r * stride + b];
    }
    part[threadIdx.x] = sum;
    __syncthreads();
    if (ph == 0 && b < hw) {
        for (uint32_t k = 1; k < PH; ++k) sum += part[k * NB + threadIdx.x];
        counts[w0 + b] += sum;
    }
}

// Wave-cooperative search in a non-decreasing array: the last index i in
// [0, n) with a[i] <= key (0 if none). Each round samples 64 evenly spaced
// entries with one load per lane, so a search costs log64(n) round trips.
__device__ __forceinline__ uint32_t wave_find_last_le(const uint32_t *__restrict__ a, uint32_t n,
                                                      uint32_t key)
{
    const uint32_t lane = lane_id();
    uint32_t lo = 0, hi = n;  // answer in [lo, hi)
    while (hi - lo > 1) {
        const uint32_t step = (hi - lo + 63) / 64;
        const uint32_t idx = lo + lane * step;
        const bool le = idx < hi && a[idx] <= key;
        const uint64_t m = __ballot(le);
        const uint32_t j = m ? 63u - (uint32_t)__builtin_clzll(m) : 0u;
        lo = lo + j * step;
        hi = min(lo + step, hi);
    }
    return lo;
}

// An owner counts a range with one run per lane when the range's runs over
// its span average fewer than this many elements (24 staged vectors). Timed on
// 2^26 uniform elements: runs of 128 take 87.6 us one per lane against 103.8
// striped, runs of 256 take 89.0 against 67.5.
constexpr uint32_t kSparseRun = 192;
// In that mode a run of more than this many staged vectors is counted by its
// whole wave rather than by one lane.
constexpr uint32_t kLaneRunVecs = 64;

// Count the slots of one staged vector (8 uint16 slots as 4 words) whose
// index e lies in [first, last), through the wave's hot slot when AGG == 1.
template <int AGG>
__device__ __forceinline__ void count_slots(uint32_t *lds, HotSlot &hs, const uint32_t (&words)[4],
                                            uint32_t first, uint32_t last)
{
    // the hot slot is wave-uniform: read it as a scalar so that this test is one branch
    const uint32_t h = AGG == 1 ? (uint32_t)__builtin_amdgcn_readfirstlane((int)hs.h) : kNoSlot;
    if (AGG == 1 && h != kNoSlot) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t s = (e & 1) ? (words[e >> 1] >> 16) : (words[e >> 1] & 0xFFFFu);
            const bool ok = (uint32_t)e >= first && (uint32_t)e < last;
            const bool m = ok && s == h;
            hs.c += m ? 1u : 0u;
            lds_count<0>(lds, s, ok && !m);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t s = (e & 1) ? (words[e >> 1] >> 16) : (words[e >> 1] & 0xFFFFu);
            const bool ok = (uint32_t)e >= first && (uint32_t)e < last;
            lds_count<AGG == 1 ? 0 : AGG>(lds, s, ok);
        }
    }
}

// An owner's finished slice of one range. When the owner's span holds the
// whole range it is the range's only owner: it writes the counts itself
// (adds them when accumulating), and the slot merge skips the range.
// Otherwise the slice goes to partial slot `row` for the slot merge.
template <int WG>
__device__ __forceinline__ void finish_range(const Partials &out, uint32_t row, const uint32_t *lds,
                                             uint32_t len, uint32_t *__restrict__ dst, bool whole,
                                             uint32_t accumulate)
{
    if (!whole) {
        flush_slice<WG, 32>(out, row, 0, lds, EvList{nullptr, nullptr, 0u, nullptr}, 0, len, 0);
        return;
    }
    // 16-byte stores where the range's counts start 16-byte aligned (counts
    // itself needs only 4-byte alignment); the tail and other bases by word
    uint32_t done = 0;
    if ((reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
        const uint32_t nv = len >> 2;
        const u32x4 *l4 = reinterpret_cast<const u32x4 *>(lds);
        u32x4 *d4 = reinterpret_cast<u32x4 *>(dst);
        if (accumulate)
            for (uint32_t v = threadIdx.x; v < nv; v += WG) d4[v] = d4[v] + l4[v];
        else
            for (uint32_t v = threadIdx.x; v < nv; v += WG) d4[v] = l4[v];
        done = nv << 2;
    }
    if (accumulate)
        for (uint32_t b = done + threadIdx.x; b < len; b += WG) dst[b] += lds[b];
    else
        for (uint32_t b = done + threadIdx.x; b < len; b += WG) dst[b] = lds[b];
}

// Phase 2: owner workgroups build LDS histograms from the routed slots.
//
// All ranges' elements, concatenated in range order, are split evenly over
// W owner workgroups, so a range holding most of the input (a hot bin, a
// Gaussian bump) is shared by as many owners as its size calls for. Owner i
// takes positions [i*N/W, (i+1)*N/W); for every range r it overlaps it
// zeroes an LDS slice of the range's bins, counts the overlapped elements,
// and writes the slice to partial slot i + r (i + r is distinct for every
// (owner, range) pair that occurs, because both grow along the
// concatenation). Inside one range the elements are the tiles' runs in tile
// order. Waves work without barriers, in teams: a team takes groups of RPW
// consecutive tiles (every (NW / S)-th group of the owner's span) and each
// of its S waves reads the group's run metadata with one lane per tile. Run
// m then feeds slot m of every lane's batch of RPW 16-byte loads (the team's
// lanes stripe each run's vectors), so every run parameter is wave-uniform
// and a vector costs a compare, an address and two bounds. The runs of one range are
// about equally long for shuffled inputs, so the slots stay busy and the
// waves balanced. With no workgroup barrier until the slice is flushed, the
// waves drift apart and one wave's loads overlap the others' counting.
template <int WG, int UNROLL, int AGG, bool NTS = true>
__global__ __launch_bounds__(WG) void k_bucket_hist(
    const uint16_t *__restrict__ stage, uint32_t stage_cap, const uint32_t *__restrict__ tcnt,
    const uint32_t *__restrict__ tbase, const uint32_t *__restrict__ tpre,
    const uint32_t *__restrict__ totals, uint32_t ranges, uint32_t tiles, uint32_t range_bins,
    uint32_t num_bins, uint32_t owners, Partials out, uint64_t *__restrict__ starts,
    uint32_t *__restrict__ counts, uint32_t accumulate, const uint32_t *__restrict__ hot_seen)
{
    extern __shared__ u32x4 lds4[];
    uint32_t *lds = reinterpret_cast<uint32_t *>(lds4);
    // the hot slot, unless this run's sample showed no value that it would
    // take (k_window_pick): then its checks would cost and find nothing
    const bool hot_on = AGG == 1 && (!hot_seen || *hot_seen != 0u);
    uint64_t *bs = reinterpret_cast<uint64_t *>(lds + range_bins);  // [ranges + 1]
    uint32_t *misc = reinterpret_cast<uint32_t *>(bs + ranges + 1);  // [0] ta [1] tb
    const uint32_t tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    constexpr uint32_t NW = WG / 64;  // waves
    constexpr uint32_t RPW = UNROLL;  // tiles (runs) per wave group = loads in flight per lane

    range_starts(totals, ranges, bs);
    __syncthreads();
    // the slot merge reads every range's start from here
    if (blockIdx.x == 0)
        for (uint32_t k = threadIdx.x; k <= ranges; k += WG) starts[k] = bs[k];
    const uint64_t N = bs[ranges];
    const uint32_t i = blockIdx.x;
    const uint64_t e0 = (uint64_t)i * N / owners, e1 = (uint64_t)(i + 1) * N / owners;
    if (e0 >= e1) return;  // whole workgroup: no element to count

    uint32_t r;  // first range overlapping [e0, e1): the last r with bs[r] <= e0
    {
        uint32_t lo = 0, hi = ranges - 1;
        while (lo < hi) {
            const uint32_t mid = (lo + hi + 1) >> 1;
            if (bs[mid] <= e0) lo = mid; else hi = mid - 1;
        }
        r = lo;
    }
    // The staged slots are read once, here: NTS, non-temporal loads, for
    // slots that outgrow the Infinity Cache (the host's choice, as for the
    // partition's stores).
    const i32x4 *stage_vec = reinterpret_cast<const i32x4 *>(stage);
    for (; r < ranges && bs[r] < e1; ++r) {
        const uint64_t rb = bs[r], re = bs[r + 1];
        if (re <= e0 || rb == re) continue;  // uniform
        const uint32_t p0 = (uint32_t)(max(e0, rb) - rb), p1 = (uint32_t)(min(e1, re) - rb);
        const uint32_t len = min(range_bins, num_bins - r * range_bins);
        const uint32_t *rc = tcnt + (uint64_t)r * tiles;
        const uint32_t *rbase = tbase + (uint64_t)r * tiles;
        const uint32_t *rpre = tpre + (uint64_t)r * tiles;
        zero_lds<WG>(lds, len);
        if (w == 0) {
            // runs overlapping [p0, p1): from the last t with rpre[t] <= p0 to the
            // first t with rpre[t] >= p1
            const uint32_t ta = wave_find_last_le(rpre, tiles, p0);
            uint32_t tb = wave_find_last_le(rpre, tiles, p1 - 1) + 1;
            if (lane == 0) {
                misc[0] = ta;
                misc[1] = tb;
            }
        }
        __syncthreads();
        const uint32_t ta = misc[0], tb = misc[1];
        HotSlot hs;

        if ((uint64_t)(p1 - p0) < (uint64_t)kSparseRun * (tb - ta)) {
            // Short runs (many ranges, few elements per tile and range): one run
            // per lane, 64 consecutive tiles per wave and WG tiles per pass, with
            // the next pass's run table requested before this pass's vectors. A
            // lane walks its run's vectors two at a time and counts each element
            // with one LDS atomic; duplicates are rare at these densities.
            uint32_t nc = 0, nq = 0, nb = 0;
            auto load_run = [&](uint32_t t) {
                if (t < tb) {
                    nc = rc[t];
                    nq = rpre[t];
                    nb = rbase[t];
                }
            };
            load_run(ta + tid);
            for (uint32_t t0 = ta + w * 64u; t0 < tb; t0 += WG) {
                const uint32_t t = t0 + lane;
                uint32_t vlo = 0, nv = 0, skip = 0, used = 0;
                if (t < tb) {
                    const uint32_t lo_e = max(p0, nq) - nq, hi_e = min(p1, nq + nc) - nq;
                    if (nc != 0u && hi_e > lo_e) {
                        const uint64_t g_lo = (uint64_t)t * stage_cap + nb + lo_e;
                        const uint64_t g_hi = g_lo + (hi_e - lo_e);
                        vlo = (uint32_t)(g_lo >> 3);
                        nv = (uint32_t)(((g_hi + 7) >> 3) - (g_lo >> 3));
                        skip = (uint32_t)(g_lo & 7u);
                        used = hi_e - lo_e;
                    }
                }
                load_run(t0 + WG + lane);
                // A run far longer than the average (part of the input sorted,
                // say) would keep one lane busy while the rest of the workgroup
                // waits: the wave takes such runs together after its own runs.
                const uint32_t nv_run = nv;
                uint64_t longm = __ballot(nv > kLaneRunVecs);
                if (nv > kLaneRunVecs) nv = 0u;
                for (uint32_t v = 0; v < nv; v += 2u) {
                    const bool two = v + 1u < nv;
                    const i32x4 qa = load_vec<NTS>(stage_vec + ((uint64_t)vlo + v));
                    const i32x4 qb = two ? load_vec<NTS>(stage_vec + ((uint64_t)vlo + v + 1u)) : i32x4{0, 0, 0, 0};
#pragma unroll
                    for (uint32_t k = 0; k < 2; ++k) {
                        const i32x4 q = k == 0 ? qa : qb;
                        const uint32_t k8 = (v + k) * 8u;
                        const uint32_t first = k8 < skip ? skip - k8 : 0u;
                        const uint32_t last = (k == 0 || two) ? min(8u, skip + used - k8) : 0u;
                        const uint32_t words[4] = {(uint32_t)q.x, (uint32_t)q.y, (uint32_t)q.z,
                                                   (uint32_t)q.w};
                        count_slots<0>(lds, hs, words, first, last);
                    }
                }
                while (longm) {
                    const int m = __builtin_ctzll(longm);
                    longm &= longm - 1u;
                    const uint32_t lv = (uint32_t)__builtin_amdgcn_readlane((int)vlo, m);
                    const uint32_t ln = (uint32_t)__builtin_amdgcn_readlane((int)nv_run, m);
                    const uint32_t ls = (uint32_t)__builtin_amdgcn_readlane((int)skip, m);
                    const uint32_t lu = (uint32_t)__builtin_amdgcn_readlane((int)used, m);
                    for (uint32_t d = lane; d < ln; d += 64u) {
                        const i32x4 q = load_vec<NTS>(stage_vec + ((uint64_t)lv + d));
                        const uint32_t k8 = d * 8u;
                        const uint32_t first = k8 < ls ? ls - k8 : 0u;
                        const uint32_t last = min(8u, ls + lu - k8);
                        const uint32_t words[4] = {(uint32_t)q.x, (uint32_t)q.y, (uint32_t)q.z,
                                                   (uint32_t)q.w};
                        count_slots<0>(lds, hs, words, first, last);
                    }
                }
            }
            __syncthreads();
            finish_range<WG>(out, i + r, lds, len, counts + (uint64_t)r * range_bins,
                             rb >= e0 && re <= e1, accumulate);
            __syncthreads();
            continue;
        }

        // Teams of S waves: team w / S takes groups of RPW tiles (every NW / S-th
        // group), and its S waves stripe each run's vectors. S is the smallest
        // power of two that still leaves every team two groups, so long runs
        // (few ranges, or an input piled into one range) keep all waves busy.
        const uint32_t ngroups = (tb - ta + RPW - 1) / RPW;
        uint32_t S = 1;
        while (S < NW && ngroups < 2u * (NW / S)) S *= 2u;
        const uint32_t team = w / S, member = w % S;
        // The next group's run table is requested before this group's vectors,
        // so both are in flight together and a group costs one memory round trip.
        const uint32_t gstride = (NW / S) * RPW;
        uint32_t nc = 0, nq = 0, nb = 0;
        auto load_runs = [&](uint32_t g) {
            const uint32_t t = g + lane;
            if (lane < RPW && t < tb) {
                nc = rc[t];
                nq = rpre[t];
                nb = rbase[t];
            }
        };
        load_runs(ta + team * RPW);
        for (uint32_t g0 = ta + team * RPW; g0 < tb; g0 += gstride) {
            // lane m < RPW: the run of tile g0 + m, clipped to [p0, p1)
            uint32_t vlo = 0, nv = 0, skip = 0, used = 0;
            const uint32_t t = g0 + lane;
            if (lane < RPW && t < tb) {
                const uint32_t c = nc, q = nq, bse = nb;
                const uint32_t lo_e = max(p0, q) - q;
                const uint32_t hi_e = min(p1, q + c) - q;
                if (c != 0u && hi_e > lo_e) {
                    const uint64_t g_lo = (uint64_t)t * stage_cap + bse + lo_e;
                    const uint64_t g_hi = g_lo + (hi_e - lo_e);
                    vlo = (uint32_t)(g_lo >> 3);
                    nv = (uint32_t)(((g_hi + 7) >> 3) - (g_lo >> 3));
                    skip = (uint32_t)(g_lo & 7u);
                    used = hi_e - lo_e;
                }
            }
            load_runs(g0 + gstride);
            // Run m of the group takes slot m of every lane's batch of RPW vector
            // loads, so all run parameters stay wave-uniform (scalar registers).
            uint32_t run_n[RPW], run_v[RPW], run_s[RPW], run_u[RPW], steps = 0;
#pragma unroll
            for (uint32_t m = 0; m < RPW; ++m) {
                run_n[m] = (uint32_t)__builtin_amdgcn_readlane((int)nv, (int)m);
                run_v[m] = (uint32_t)__builtin_amdgcn_readlane((int)vlo, (int)m);
                run_s[m] = (uint32_t)__builtin_amdgcn_readlane((int)skip, (int)m);
                run_u[m] = (uint32_t)__builtin_amdgcn_readlane((int)used, (int)m);
                steps = max(steps, (run_n[m] + 64u * S - 1u) / (64u * S));
            }
            for (uint32_t it = 0; it < steps; ++it) {
                const uint32_t d = (it * S + member) * 64u + lane;  // this lane's vector in each run
                const uint32_t k8 = d * 8u;          // run element of vector element e is k8 + e - skip
                i32x4 qv[RPW];
                uint32_t first[RPW], last[RPW];
#pragma unroll
                for (uint32_t m = 0; m < RPW; ++m) {
                    const bool ok = d < run_n[m];
                    first[m] = ok ? (k8 < run_s[m] ? run_s[m] - k8 : 0u) : 8u;
                    last[m] = ok ? min(8u, run_s[m] + run_u[m] - k8) : 0u;
                    qv[m] = ok ? load_vec<NTS>(stage_vec + ((uint64_t)run_v[m] + d)) : i32x4{0, 0, 0, 0};
                }
#pragma unroll
                for (uint32_t k = 0; k < RPW; ++k) {
                    const uint32_t words[4] = {(uint32_t)qv[k].x, (uint32_t)qv[k].y,
                                               (uint32_t)qv[k].z, (uint32_t)qv[k].w};
                    if constexpr (AGG == 1) {
                        uint32_t nxt;
                        if (hot_on && hot_should_switch(hs, words[0] & 0xFFFFu,
                                                        first[k] == 0u && last[k] > 0u, &nxt)) {
                            const uint32_t tk = hot_take(hs);
                            if (lane == 0 && tk != 0u) lds_add(lds, hs.h, tk);
                            hs.h = nxt;
                        }
                    }
                    count_slots<AGG>(lds, hs, words, first[k], last[k]);
                }
            }
        }
        {
            const uint32_t t = hot_take(hs);
            if (lane == 0 && t != 0u) lds_add(lds, hs.h, t);
        }
        __syncthreads();
        finish_range<WG>(out, i + r, lds, len, counts + (uint64_t)r * range_bins,
                         rb >= e0 && re <= e1, accumulate);
        __syncthreads();
    }
}

// Phase 2b: counts[b] for the bins of one range = the sum of the slots that
// the owners overlapping the range wrote for it (exclusive owner per bin, no
// global atomics). A workgroup handles BPW 256-bin blocks of one range. Owner
// i wrote the range's slot to row i + r, so the slots of the overlapping
// owners first..last are consecutive rows, summed by merge_block. An owner
// that took no element (possible only when there are fewer elements than
// owners) wrote no slot and is skipped. A range with a single owner was
// written to counts by that owner and is skipped whole. Empty ranges give
// zeros.
template <int WAVES, bool ACC, uint32_t ROUNDS, uint32_t BPW>
__global__ __launch_bounds__(WAVES * 64) void k_merge_slots(Partials P, const uint64_t *__restrict__ starts,
                                                            uint32_t ranges, uint32_t range_bins,
                                                            uint32_t num_bins, uint32_t owners,
                                                            uint32_t *__restrict__ counts)
{
    const uint32_t lane = lane_id(), w = threadIdx.x >> 6;
    // a workgroup takes BPW consecutive blocks of one range (BPW divides the
    // range's 128 blocks), so that a range with one owner is skipped once
    const uint32_t wpr = range_bins / kBlockBins / BPW;  // workgroups per range
    const uint32_t r = blockIdx.x / wpr, lb0 = (blockIdx.x % wpr) * BPW;
    // start of range r, its end, and the grand total (the owner phase's prefix)
    const uint64_t rb = starts[r], re = starts[r + 1], N = starts[ranges];
    uint32_t first = 0, rows = 0;
    if (re > rb) {
        first = owner_of(rb, N, owners);
        rows = owner_of(re - 1, N, owners) - first + 1;
        if (rows == 1) return;  // one owner held the whole range and wrote its counts
    }
    // every owner took at least one element when N >= owners
    const bool all_nonempty = N >= owners;
    auto row_ok = [&](uint32_t k) {
        const uint64_t i = (uint64_t)first + k;
        return all_nonempty || i * N / owners < (i + 1) * N / owners;
    };
    for (uint32_t lb = lb0; lb < lb0 + BPW; ++lb) {
        const u32x4 t = merge_block<WAVES, ROUNDS>(P, (uint64_t)first + r, rows, lb, row_ok);
        if (w == 0)
            store_counts<ACC>(counts, (uint64_t)r * range_bins + lb * kBlockBins + lane * 4u, num_bins,
                              t);
        if (BPW > 1) __syncthreads();  // merge_block's LDS is reused by the next block
    }
}

}  // namespace pca
