// hist_kernels.hpp -- gfx950 kernels of the partitioned LDS histogram.
//
// Internal to libpca_hist.so. The operation is the one on the page
// "Distributed Shared Memory", section "The cluster histogram": every input
// element adds one to the bin it names, each bin is accumulated on-chip by
// the workgroup that owns it, and owned slices are merged into the global
// bins. What changes for CDNA4 is how ownership is reached. There is no
// cross-CU shared memory on gfx950, so instead of sending an atomic to the
// owner's LDS, either
//   * the owner reads the input itself and keeps only its own bins
//     (k_sweep: a workgroup owns all bins, or one range of them), or
//   * the input is first routed by owner in a cheap coarse pass
//     (k_partition), and owners then read only their own elements
//     (k_bucket_hist).
// Slices are merged by exclusive owners (k_merge, k_merge_slots): one thread
// writes each output bin once, so no global atomics and no memset of the
// output are needed.
//
// Conventions: wave64 (gfx950), 16-byte (dwordx4) global loads on the input
// body, uint32 LDS counters, ds_add_u32 for accumulation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pca {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// popcount of the bits of m below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v)
{
    const uint32_t lane = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t o = __shfl_up(v, d, 64);
        if (lane >= (uint32_t)d) v += o;
    }
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

// Like lds_count, but returns each valid lane's rank: the value lds[slot]
// had before this lane's increment (distinct lanes of one slot get distinct,
// consecutive ranks). Invalid lanes get 0.
template <int ROUNDS>
__device__ __forceinline__ uint32_t lds_rank(uint32_t *lds, uint32_t slot, bool valid)
{
    uint32_t rank = 0;
    bool pending = valid;
    if constexpr (ROUNDS > 0) {
#pragma unroll
        for (int k = 0; k < ROUNDS; ++k) {
            const uint64_t act = __ballot(pending);
            if (act == 0) return rank;
            const int leader = __builtin_ctzll(act);
            const uint32_t lead = __builtin_amdgcn_readlane(slot, leader);
            const bool mine = pending && slot == lead;
            const uint64_t m = __ballot(mine);
            uint32_t base = 0;
            if (mine && lane_id() == (uint32_t)leader)
                base = lds_add_rtn(lds, lead, (uint32_t)__popcll(m));
            base = __builtin_amdgcn_readlane(base, leader);
            if (mine) rank = base + lanes_below(m);
            pending = pending && !mine;
            if (__popcll(m) == 1) break;
        }
    }
    if (pending) rank = lds_add_rtn(lds, slot, 1u);
    return rank;
}

template <bool NT>
__device__ __forceinline__ i32x4 load_vec(const i32x4 *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// Copy lds[0..len) to dst[0..len). 16-byte stores when dst is aligned; the
// store never writes past dst[len - 1].
template <int WG>
__device__ __forceinline__ void store_slice(uint32_t *__restrict__ dst, const uint32_t *lds,
                                            uint32_t len)
{
    const uint32_t tid = threadIdx.x;
    if ((reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
        const uint32_t full = len >> 2;
        const u32x4 *s4 = reinterpret_cast<const u32x4 *>(lds);
        u32x4 *d4 = reinterpret_cast<u32x4 *>(dst);
        for (uint32_t i = tid; i < full; i += WG) d4[i] = s4[i];
        for (uint32_t i = full * 4 + tid; i < len; i += WG) dst[i] = lds[i];
    } else {
        for (uint32_t i = tid; i < len; i += WG) dst[i] = lds[i];
    }
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
// With ranges == 1 every workgroup owns all bins (LDS holds num_bins
// counters). With ranges > 1 the R owners of a chunk all read it; xcds > 1
// places them on one XCD (workgroups are dispatched to the XCDs round-robin)
// so that one owner's read brings the lines into the shared L2 for the
// others. The chunk's slice of range r goes to dst + g * dst_row + lo.
//
// Chunk g is body vectors [g * nvec / groups, (g + 1) * nvec / groups); the
// head scalars belong to chunk 0 and the tail scalars to the last chunk.
template <int WG, int UNROLL, int AGG, bool NT>
__global__ __launch_bounds__(WG) void k_sweep(InputView in, uint32_t num_bins, uint32_t range_bins,
                                              uint32_t ranges, uint32_t groups, uint32_t xcds,
                                              uint32_t *__restrict__ dst, uint64_t dst_row)
{
    extern __shared__ u32x4 lds4[];
    uint32_t *lds = reinterpret_cast<uint32_t *>(lds4);
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

    zero_lds<WG>(lds, len);
    __syncthreads();

    const i32x4 *body = reinterpret_cast<const i32x4 *>(in.ptr + in.head);
    const uint64_t v0 = (uint64_t)g * in.nvec / groups;
    const uint64_t v1 = (uint64_t)(g + 1) * in.nvec / groups;

    auto count4 = [&](const i32x4 q, bool ok) {
        uint32_t s;
        s = (uint32_t)q.x - lo; lds_count<AGG>(lds, s, ok && s < len);
        s = (uint32_t)q.y - lo; lds_count<AGG>(lds, s, ok && s < len);
        s = (uint32_t)q.z - lo; lds_count<AGG>(lds, s, ok && s < len);
        s = (uint32_t)q.w - lo; lds_count<AGG>(lds, s, ok && s < len);
    };

    constexpr uint32_t STEP = WG * UNROLL;
    uint64_t v = v0;
    for (; v + STEP <= v1; v += STEP) {
        i32x4 q[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) q[u] = load_vec<NT>(body + v + u * WG + tid);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) count4(q[u], true);
    }
    // Remainder with a wave-uniform trip count.
    for (; v < v1; v += WG) {
        const bool ok = v + tid < v1;
        const i32x4 q = ok ? load_vec<NT>(body + v + tid) : i32x4{0, 0, 0, 0};
        count4(q, ok);
    }
    {
        const bool hok = g == 0 && tid < in.head;
        const uint32_t hs = (hok ? (uint32_t)in.ptr[tid] : 0u) - lo;
        lds_count<AGG>(lds, hs, hok && hs < len);
        const bool tok = g == groups - 1 && tid < in.tail;
        const uint32_t ts = (tok ? (uint32_t)in.ptr[in.head + 4 * in.nvec + tid] : 0u) - lo;
        lds_count<AGG>(lds, ts, tok && ts < len);
    }
    __syncthreads();
    store_slice<WG>(dst + (uint64_t)g * dst_row + lo, lds, len);
}

// ---------------------------------------------------------------------------
// Exclusive-owner merge: counts[b] = sum over g < groups of partials[g][b].
// A workgroup owns 256 consecutive bins; lane l holds bins 4l..4l+3 as one
// 16-byte load per row, the WAVES waves split the rows, and wave 0 adds the
// waves' sums and writes each of its bins once. row (the partial row
// stride) is a multiple of 4.
template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_merge(const uint32_t *__restrict__ partials,
                                                      uint32_t groups, uint64_t row,
                                                      uint32_t num_bins,
                                                      uint32_t *__restrict__ counts)
{
    __shared__ u32x4 red[WAVES][64];
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    const uint64_t b0 = (uint64_t)blockIdx.x * 256u + lane * 4u;
    u32x4 acc = {0u, 0u, 0u, 0u};
    if (b0 < row) {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(partials + b0);
        const uint64_t s4 = row >> 2;
        uint32_t g = w;
        for (; g + 3 * WAVES < groups; g += 4 * WAVES) {
            const u32x4 a = p[(uint64_t)g * s4];
            const u32x4 bq = p[(uint64_t)(g + WAVES) * s4];
            const u32x4 c = p[(uint64_t)(g + 2 * WAVES) * s4];
            const u32x4 d = p[(uint64_t)(g + 3 * WAVES) * s4];
            acc += (a + bq) + (c + d);
        }
        for (; g < groups; g += WAVES) acc += p[(uint64_t)g * s4];
    }
    red[w][lane] = acc;
    __syncthreads();
    if (w == 0) {
#pragma unroll
        for (int k = 1; k < WAVES; ++k) acc += red[k][lane];
        if (b0 + 0 < num_bins) counts[b0 + 0] = acc.x;
        if (b0 + 1 < num_bins) counts[b0 + 1] = acc.y;
        if (b0 + 2 < num_bins) counts[b0 + 2] = acc.z;
        if (b0 + 3 < num_bins) counts[b0 + 3] = acc.w;
    }
}

// ---------------------------------------------------------------------------
// Two-phase path, phase 1: route every element of a tile to its owning range.
//
// Tile t is body vectors [t * WG * VPT, ...) (tile 0 also takes the head
// scalars, the last tile the tail scalars). Each valid element x (x <
// num_bins) is owned by range r = x >> shift, where it is slot x & mask. The
// workgroup counts its elements per range in LDS, and each element's LDS
// atomic returns its rank among the tile's elements of that range; an
// exclusive scan of the counts gives each range's start, so the tile's
// slots can be written to an LDS staging buffer grouped by range and copied
// to stage[t * stage_cap ...] with full 16-byte stores. Only the 16-bit slot
// is kept: the range is implied by the position. Per tile and range the
// kernel writes the count and the start of its run (tcnt, tbase; layout
// [range][tile]). Element order inside a run is whatever the atomics gave;
// counts do not depend on it.
template <int WG, int VPT, int AGG>
__global__ __launch_bounds__(WG) void k_partition(InputView in, uint32_t num_bins, uint32_t shift,
                                                  uint32_t ranges, uint32_t tiles,
                                                  uint16_t *__restrict__ stage, uint32_t stage_cap,
                                                  uint32_t *__restrict__ tcnt,
                                                  uint32_t *__restrict__ tbase)
{
    extern __shared__ u32x4 smem4[];
    const uint32_t rpad = (ranges + 3u) & ~3u;
    uint32_t *cnt = reinterpret_cast<uint32_t *>(smem4);
    uint32_t *base = cnt + rpad;
    uint32_t *nvalid = base + rpad;  // one word, padded to 16 bytes
    uint16_t *st = reinterpret_cast<uint16_t *>(nvalid + 4);
    const uint32_t tid = threadIdx.x, t = blockIdx.x;
    const uint32_t mask = (1u << shift) - 1u;

    for (uint32_t i = tid; i < ranges; i += WG) cnt[i] = 0u;
    __syncthreads();

    constexpr int E = VPT * 4;
    uint32_t x[E + 2], rk[E + 2];
    const i32x4 *body = reinterpret_cast<const i32x4 *>(in.ptr + in.head);
    const uint64_t vb = (uint64_t)t * (WG * VPT);
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        const uint64_t v = vb + (uint64_t)u * WG + tid;
        const i32x4 q = v < in.nvec ? body[v] : i32x4{-1, -1, -1, -1};
        x[4 * u + 0] = (uint32_t)q.x;
        x[4 * u + 1] = (uint32_t)q.y;
        x[4 * u + 2] = (uint32_t)q.z;
        x[4 * u + 3] = (uint32_t)q.w;
    }
    x[E] = (t == 0 && tid < in.head) ? (uint32_t)in.ptr[tid] : 0xFFFFFFFFu;
    x[E + 1] = (t == tiles - 1 && tid < in.tail) ? (uint32_t)in.ptr[in.head + 4 * in.nvec + tid]
                                                 : 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < E + 2; ++e) {
        const bool ok = x[e] < num_bins;
        rk[e] = lds_rank<AGG>(cnt, ok ? x[e] >> shift : 0u, ok);
    }
    __syncthreads();

    if (tid < 64) {
        uint32_t carry = 0;
        for (uint32_t c = 0; c < ranges; c += 64) {
            const uint32_t i = c + tid;
            const uint32_t v = i < ranges ? cnt[i] : 0u;
            const uint32_t incl = wave_inclusive_scan(v);
            if (i < ranges) {
                base[i] = carry + incl - v;
                tcnt[(uint64_t)i * tiles + t] = v;
                tbase[(uint64_t)i * tiles + t] = carry + incl - v;
            }
            carry += __shfl(incl, 63, 64);
        }
        if (tid == 0) *nvalid = carry;
    }
    __syncthreads();

#pragma unroll
    for (int e = 0; e < E + 2; ++e)
        if (x[e] < num_bins) st[base[x[e] >> shift] + rk[e]] = (uint16_t)(x[e] & mask);
    __syncthreads();

    const uint32_t nv = (*nvalid + 7u) >> 3;
    const u32x4 *s4 = reinterpret_cast<const u32x4 *>(st);
    u32x4 *d4 = reinterpret_cast<u32x4 *>(stage + (uint64_t)t * stage_cap);
    for (uint32_t i = tid; i < nv; i += WG) d4[i] = s4[i];
}

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

// Phase 1b: per range r, tpre[r][t] = sum of tcnt[r][t'] over t' < t, and
// totals[r] = the range's element count. One workgroup per range.
template <int WG>
__global__ __launch_bounds__(WG) void k_bucket_scan(const uint32_t *__restrict__ tcnt,
                                                    uint32_t tiles, uint32_t *__restrict__ tpre,
                                                    uint32_t *__restrict__ totals)
{
    __shared__ uint32_t scratch[2 * (WG / 64) + 1];
    const uint32_t r = blockIdx.x, tid = threadIdx.x;
    const uint32_t *c = tcnt + (uint64_t)r * tiles;
    uint32_t *p = tpre + (uint64_t)r * tiles;
    const uint32_t per = (tiles + WG - 1) / WG;
    const uint32_t t0 = min(tid * per, tiles), t1 = min(t0 + per, tiles);
    uint32_t s = 0;
    for (uint32_t t = t0; t < t1; ++t) s += c[t];
    uint32_t total;
    uint32_t run = block_exclusive_scan<WG>(s, scratch, &total);
    for (uint32_t t = t0; t < t1; ++t) {
        p[t] = run;
        run += c[t];
    }
    if (tid == 0) totals[r] = total;
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

// Phase 2: owner workgroups build LDS histograms from the routed slots.
//
// All ranges' elements, concatenated in range order, are split evenly over
// W owner workgroups, so a range holding most of the input (a hot bin, a
// Gaussian bump) is shared by as many owners as its size calls for. Owner i
// takes positions [i*N/W, (i+1)*N/W); for every range r it overlaps it
// zeroes an LDS slice of the range's bins, counts the overlapped elements,
// and writes the slice to partial slot i + r (i + r is distinct for every
// (owner, range) pair that occurs, because both grow along the
// concatenation). Inside one range the elements are the runs of the tiles in
// tile order; each wave takes 64 tiles at a time, lays their runs end to end
// with a wave scan of their vector counts, and spreads the resulting 16-byte
// vectors over its lanes, so short and long runs both keep every lane busy.
template <int WG, int UNROLL, int AGG>
__global__ __launch_bounds__(WG) void k_bucket_hist(
    const uint16_t *__restrict__ stage, uint32_t stage_cap, const uint32_t *__restrict__ tcnt,
    const uint32_t *__restrict__ tbase, const uint32_t *__restrict__ tpre,
    const uint32_t *__restrict__ totals, uint32_t ranges, uint32_t tiles, uint32_t range_bins,
    uint32_t num_bins, uint32_t owners, uint32_t *__restrict__ partials)
{
    constexpr uint32_t NW = WG / 64;
    extern __shared__ u32x4 lds4[];
    uint32_t *lds = reinterpret_cast<uint32_t *>(lds4);
    uint64_t *bs = reinterpret_cast<uint64_t *>(lds + range_bins);
    const uint32_t tid = threadIdx.x, lane = lane_id(), w = tid >> 6;

    range_starts(totals, ranges, bs);
    __syncthreads();
    const uint64_t N = bs[ranges];
    const uint32_t i = blockIdx.x;
    const uint64_t e0 = (uint64_t)i * N / owners, e1 = (uint64_t)(i + 1) * N / owners;
    if (e0 >= e1) return;  // whole workgroup: no element to count

    // First range overlapping [e0, e1): the last r with bs[r] <= e0.
    uint32_t r = 0;
    {
        uint32_t lo = 0, hi = ranges - 1;
        while (lo < hi) {
            const uint32_t mid = (lo + hi + 1) >> 1;
            if (bs[mid] <= e0) lo = mid; else hi = mid - 1;
        }
        r = lo;
    }
    const i32x4 *stage_vec = reinterpret_cast<const i32x4 *>(stage);
    for (; r < ranges && bs[r] < e1; ++r) {
        const uint64_t rb = bs[r], re = bs[r + 1];
        if (re <= e0 || rb == re) continue;  // uniform
        const uint32_t p0 = (uint32_t)(max(e0, rb) - rb), p1 = (uint32_t)(min(e1, re) - rb);
        const uint32_t len = min(range_bins, num_bins - r * range_bins);
        zero_lds<WG>(lds, len);
        __syncthreads();

        const uint32_t *rc = tcnt + (uint64_t)r * tiles;
        const uint32_t *rbase = tbase + (uint64_t)r * tiles;
        const uint32_t *rpre = tpre + (uint64_t)r * tiles;
        // Tiles whose runs overlap [p0, p1): from the last t with rpre[t] <= p0
        // up to (excluding) the first t with rpre[t] >= p1.
        uint32_t ta, tb;
        {
            uint32_t lo = 0, hi = tiles - 1;
            while (lo < hi) {
                const uint32_t mid = (lo + hi + 1) >> 1;
                if (rpre[mid] <= p0) lo = mid; else hi = mid - 1;
            }
            ta = lo;
            lo = ta;
            hi = tiles;
            while (lo < hi) {
                const uint32_t mid = (lo + hi) >> 1;
                if (rpre[mid] >= p1) hi = mid; else lo = mid + 1;
            }
            tb = lo;
        }
        for (uint32_t t0 = ta + w * 64; t0 < tb; t0 += NW * 64) {
            const uint32_t t = t0 + lane;
            uint32_t vlo = 0, nv = 0, skip = 0, cnt = 0;
            if (t < tb) {
                const uint32_t c = rc[t], q = rpre[t];
                const uint32_t lo_e = max(p0, q) - q;
                const uint32_t hi_e = min(p1, q + c) - q;
                if (c != 0 && hi_e > lo_e) {
                    const uint64_t g_lo = (uint64_t)t * stage_cap + rbase[t] + lo_e;
                    const uint64_t g_hi = g_lo + (hi_e - lo_e);
                    vlo = (uint32_t)(g_lo >> 3);
                    nv = (uint32_t)(((g_hi + 7) >> 3) - (g_lo >> 3));
                    skip = (uint32_t)(g_lo & 7u);
                    cnt = hi_e - lo_e;
                }
            }
            const uint32_t P = wave_inclusive_scan(nv);
            const uint32_t E = P - nv;
            const uint32_t total = __shfl(P, 63, 64);
            for (uint32_t u0 = 0; u0 < total; u0 += 64 * UNROLL) {
                i32x4 q[UNROLL];
                uint32_t first[UNROLL], last[UNROLL];
#pragma unroll
                for (int k = 0; k < UNROLL; ++k) {
                    const uint32_t u = u0 + k * 64 + lane;
                    // owner lane j: the first lane whose inclusive prefix exceeds u
                    uint32_t j = 0;
#pragma unroll
                    for (uint32_t step = 32; step >= 1; step >>= 1) {
                        const uint32_t pj = __shfl(P, (int)(j + step - 1), 64);
                        if (pj <= u) j += step;
                    }
                    const uint32_t jv = __shfl(vlo, (int)j, 64);
                    const uint32_t je = __shfl(E, (int)j, 64);
                    const uint32_t js = __shfl(skip, (int)j, 64);
                    const uint32_t jc = __shfl(cnt, (int)j, 64);
                    const bool ok = u < total;
                    const uint32_t k8 = (u - je) * 8u;  // element offset of this vector in the run, + skip
                    // element e of the vector is run element k8 + e - skip
                    first[k] = ok ? (k8 < js ? js - k8 : 0u) : 8u;
                    last[k] = ok ? min(8u, js + jc - k8) : 0u;
                    q[k] = ok ? stage_vec[jv + (u - je)] : i32x4{0, 0, 0, 0};
                }
#pragma unroll
                for (int k = 0; k < UNROLL; ++k) {
                    const uint32_t words[4] = {(uint32_t)q[k].x, (uint32_t)q[k].y, (uint32_t)q[k].z,
                                               (uint32_t)q[k].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t s = (e & 1) ? (words[e >> 1] >> 16) : (words[e >> 1] & 0xFFFFu);
                        const bool ok = (uint32_t)e >= first[k] && (uint32_t)e < last[k];
                        lds_count<AGG>(lds, s, ok);
                    }
                }
            }
        }
        __syncthreads();
        store_slice<WG>(partials + (uint64_t)(i + r) * range_bins, lds, len);
        __syncthreads();
    }
}

// Phase 2b: counts[b] for the bins of one range = the sum of the slots that
// the owners overlapping the range wrote for it (exclusive owner per bin, no
// global atomics). A workgroup handles 256 bins of one range; range_bins is
// a multiple of 256. Empty ranges give zeros.
template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_merge_slots(const uint32_t *__restrict__ partials,
                                                            const uint32_t *__restrict__ totals,
                                                            uint32_t ranges, uint32_t range_bins,
                                                            uint32_t num_bins, uint32_t owners,
                                                            uint32_t *__restrict__ counts)
{
    __shared__ u32x4 red[WAVES][64];
    __shared__ uint64_t se[3];
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    const uint64_t bin0 = (uint64_t)blockIdx.x * 256u;
    const uint32_t r = (uint32_t)(bin0 / range_bins);
    const uint32_t s0 = (uint32_t)(bin0 % range_bins) + lane * 4u;
    if (w == 0) {
        // start of range r, its end, and the grand total
        uint64_t before = 0, all = 0;
        for (uint32_t c = 0; c < ranges; c += 64) {
            const uint32_t k = c + lane;
            const uint64_t v = k < ranges ? totals[k] : 0u;
            uint64_t a = v, bsum = k < r ? v : 0u;
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) {
                a += __shfl_xor(a, d, 64);
                bsum += __shfl_xor(bsum, d, 64);
            }
            all += a;
            before += bsum;
        }
        if (lane == 0) {
            se[0] = before;
            se[1] = before + totals[r];
            se[2] = all;
        }
    }
    __syncthreads();
    const uint64_t rb = se[0], re = se[1], N = se[2];
    u32x4 acc = {0u, 0u, 0u, 0u};
    if (re > rb) {
        const uint32_t first = owner_of(rb, N, owners), last = owner_of(re - 1, N, owners);
        for (uint32_t i = first + w; i <= last; i += WAVES) {
            const uint64_t a = (uint64_t)i * N / owners, b = (uint64_t)(i + 1) * N / owners;
            if (a < b)
                acc += *reinterpret_cast<const u32x4 *>(partials + (uint64_t)(i + r) * range_bins + s0);
        }
    }
    red[w][lane] = acc;
    __syncthreads();
    if (w == 0) {
#pragma unroll
        for (int k = 1; k < WAVES; ++k) acc += red[k][lane];
        const uint64_t b = (uint64_t)r * range_bins + s0;
        if (b + 0 < num_bins) counts[b + 0] = acc.x;
        if (b + 1 < num_bins) counts[b + 1] = acc.y;
        if (b + 2 < num_bins) counts[b + 2] = acc.z;
        if (b + 3 < num_bins) counts[b + 3] = acc.w;
    }
}

}  // namespace pca
