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
// writes (or, when accumulating, reads and writes) each output bin once, so
// no global atomics and no memset of the output are needed.
//
// Conventions: wave64 (gfx950), 16-byte (dwordx4) global loads on the input
// body; LDS counters are uint32 (ds_add_u32) or two 16-bit halves of a word
// kept exact by carry events (ds_add_rtn_u32).
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

__device__ __forceinline__ uint32_t wave_sum(uint32_t v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
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

// ---------------------------------------------------------------------------
// Partial slices.
//
// A workgroup's slice is flushed in blocks of 256 bins, stored nibble-planar:
// plane q of a block (128 bytes) holds bits 4q..4q+3 of its 256 counts, bin b
// of the block in byte b / 2 (low nibble for even b). A block keeps only as
// many planes as its largest count needs (1, 2, 4 or 8 planes for 4, 8, 16
// or 32 bits, chosen by wave ballots). Plane 0 of every block of a row is
// stored densely (row after row, 128 bytes per block), planes 1..7 in a
// per-block slot of their own, and a byte per block records planes - 1. A
// histogram's partial slices hold small counts for most inputs (a
// 65,536-bin slice of 262,144 uniform elements averages 4 per bin), so plane
// 0 alone carries nearly all of it: an eighth of the 32-bit bytes, written
// and read as whole cache lines, while staying exact for any count.
constexpr uint32_t kBlockBins = 256;
constexpr uint32_t kPlaneBytes = 128;
constexpr uint32_t kUpperPlanes = 7;
// bytes of partial storage per (row, block): plane 0, planes 1..7, width code
constexpr uint32_t kBlockStoreBytes = kPlaneBytes * (1 + kUpperPlanes) + 1;


struct Partials {
    uint8_t *plane0;  // [rows][nblk][128 bytes]
    uint8_t *upper;   // [rows][nblk][7 planes][128 bytes]
    uint8_t *width;   // [rows][nblk]: number of planes - 1 (0, 1, 3 or 7)
    uint32_t nblk;    // blocks per row = ceil(num_bins / 256)
};

// Store that writes through the XCD's L2 (device scope): the partial slices
// are read by other XCDs in the next kernel, and written-through lines leave
// nothing for the end-of-kernel L2 write-back to do.
__device__ __forceinline__ void store_through(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bits 4q..4q+3 of eight counts, packed as the nibbles of one word.
__device__ __forceinline__ uint32_t plane_word(const uint32_t (&c)[8], uint32_t q)
{
    uint32_t d = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) d |= ((c[i] >> (4u * q)) & 0xFu) << (4 * i);
    return d;
}

// Store a pair of blocks: lane l holds the counts of bins 8l..8l+7 of the
// pair (lanes 0-31 the even block kb0, lanes 32-63 the odd one). blocks_left
// is the number of blocks of the pair that exist (1 or 2). Whole wave,
// convergent.
__device__ __forceinline__ void write_pair(const Partials &P, uint64_t blk_even,
                                           uint32_t blocks_left, const uint32_t (&c)[8])
{
    const uint32_t lane = lane_id();
    // a count needs more than 4k bits iff the OR of the counts does
    uint32_t any = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) any |= c[i];
    const uint32_t sh = lane & 32u;
    const uint32_t b4 = (uint32_t)(__ballot(any > 0xFu) >> sh);
    const uint32_t b8 = (uint32_t)(__ballot(any > 0xFFu) >> sh);
    const uint32_t b16 = (uint32_t)(__ballot(any > 0xFFFFu) >> sh);
    const uint32_t planes = b16 ? 8u : b8 ? 4u : b4 ? 2u : 1u;
    if ((lane >> 5) >= blocks_left) return;
    const uint64_t blk = blk_even + (lane >> 5);
    const uint32_t sub = lane & 31u;
    // both blocks' plane 0 are 256 contiguous bytes
    store_through(reinterpret_cast<uint32_t *>(P.plane0 + blk_even * kPlaneBytes) + lane,
                  plane_word(c, 0));
    for (uint32_t q = 1; q < planes; ++q)
        store_through(reinterpret_cast<uint32_t *>(P.upper + (blk * kUpperPlanes + q - 1) * kPlaneBytes) + sub,
                      plane_word(c, q));
    if (sub == 0) P.width[blk] = (uint8_t)(planes - 1);
}

// Plane q of eight 16-bit counts held two per word (count 2k in the low half
// of word k, count 2k+1 in its high half), as one word of nibbles.
__device__ __forceinline__ uint32_t plane_word16(u32x4 w, uint32_t q)
{
    const uint32_t sh = 4u * q;
    // y: nibbles of counts 0, 2, 1, 3 at bits 0, 8, 16, 24 (z likewise for 4..7)
    const uint32_t y = ((w.x >> sh) & 0x000F000Fu) | (((w.y >> sh) & 0x000F000Fu) << 8);
    const uint32_t z = ((w.z >> sh) & 0x000F000Fu) | (((w.w >> sh) & 0x000F000Fu) << 8);
    return ((y | (y >> 12)) & 0xFFFFu) | ((z | (z >> 12)) << 16);
}

// write_pair for counts that are exact in 16 bits, read straight from packed
// LDS words (lane l: bins 8l..8l+7 of the pair as four words). Both blocks of
// the pair exist. Whole wave, convergent.
__device__ __forceinline__ void write_pair16(const Partials &P, uint64_t blk_even, u32x4 w)
{
    const uint32_t lane = lane_id();
    const uint32_t any = w.x | w.y | w.z | w.w;
    const uint64_t wide = __ballot((any & 0xFFF0FFF0u) != 0u);
    if (wide == 0) {
        // the common case: both blocks fit 4 bits, plane 0 only
        store_through(reinterpret_cast<uint32_t *>(P.plane0 + blk_even * kPlaneBytes) + lane,
                      plane_word16(w, 0));
        if ((lane & 31u) == 0) P.width[blk_even + (lane >> 5)] = 0;
        return;
    }
    const uint32_t sh = lane & 32u;
    const uint32_t b4 = (uint32_t)(wide >> sh);
    const uint32_t b8 = (uint32_t)(__ballot((any & 0xFF00FF00u) != 0u) >> sh);
    const uint32_t planes = b8 ? 4u : b4 ? 2u : 1u;
    const uint64_t blk = blk_even + (lane >> 5);
    const uint32_t sub = lane & 31u;
    store_through(reinterpret_cast<uint32_t *>(P.plane0 + blk_even * kPlaneBytes) + lane,
                  plane_word16(w, 0));
    for (uint32_t q = 1; q < planes; ++q)
        store_through(reinterpret_cast<uint32_t *>(P.upper + (blk * kUpperPlanes + q - 1) * kPlaneBytes) + sub,
                      plane_word16(w, q));
    if (sub == 0) P.width[blk] = (uint8_t)(planes - 1);
}

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

// Counts of bins 8l..8l+7 (l = lane) of pair p (bins 512p..512p+511) of a
// slice, from 32-bit or 16-bit LDS counters. Bins at or beyond len read as
// zero; a lane whose bins all lie beyond len reads no LDS. The slice's LDS
// holds at least round_up(len, 256) counters, so a partly valid lane stays
// inside it.
template <int CW>
__device__ __forceinline__ void slice_octet(const uint32_t *lds, const uint32_t *evlist,
                                            uint32_t nev, uint32_t p, uint32_t len,
                                            uint32_t kshift, uint32_t (&c)[8])
{
    const uint32_t b0 = p * 512u + lane_id() * 8u;
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = 0u;
    if (b0 >= len) return;
    if constexpr (CW == 32) {
        if (kshift == 0) {
            const u32x4 a = reinterpret_cast<const u32x4 *>(lds)[b0 / 4];
            const u32x4 b = reinterpret_cast<const u32x4 *>(lds)[b0 / 4 + 1];
            c[0] = a.x; c[1] = a.y; c[2] = a.z; c[3] = a.w;
            c[4] = b.x; c[5] = b.y; c[6] = b.z; c[7] = b.w;
        } else {
            // K = 2^kshift interleaved copies: bin s, copy j at word s*K + j
            const uint32_t K = 1u << kshift;
            for (uint32_t i = 0; i < 8; ++i) {
                const uint32_t *src = lds + ((b0 + i) << kshift);
                uint32_t t = 0u;
                for (uint32_t cp = 0; cp < K; ++cp) t += src[cp];
                c[i] = t;
            }
        }
    } else {
        const u32x4 ww = reinterpret_cast<const u32x4 *>(lds)[b0 / 8];
        c[0] = ww.x & 0xFFFFu; c[1] = ww.x >> 16;
        c[2] = ww.y & 0xFFFFu; c[3] = ww.y >> 16;
        c[4] = ww.z & 0xFFFFu; c[5] = ww.z >> 16;
        c[6] = ww.w & 0xFFFFu; c[7] = ww.w >> 16;
        const uint32_t w0 = b0 / 2;
        // constant indices only: a variable index would move c[] to scratch memory
        for (uint32_t e = 0; e < nev; ++e) {
            const uint32_t ent = evlist[e];
            const uint32_t d = (ent & 0x3FFFFFFFu) - w0;
            const uint32_t add_lo = (ent & kEvLoWrap) ? 65536u : 0u;
            const uint32_t add_hi = ((ent & kEvCarry) ? 65536u : 0u) - ((ent & kEvLoWrap) ? 1u : 0u);
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k) {
                if (d == k) {
                    c[2 * k] += add_lo;
                    c[2 * k + 1] += add_hi;
                }
            }
        }
    }
#pragma unroll
    for (uint32_t i = 0; i < 8; ++i)
        if (b0 + i >= len) c[i] = 0u;
}

// Flush an LDS slice of len bins to partial row `row`, starting at block
// blk0 of the row: each wave takes pairs of blocks, kFlushBatch pairs at a
// time with their LDS reads issued together. Whole workgroup.
constexpr uint32_t kFlushBatch = 4;

template <int WG, int CW>
__device__ __forceinline__ void flush_slice(const Partials &P, uint64_t row, uint32_t blk0,
                                            const uint32_t *lds, const uint32_t *evlist,
                                            uint32_t nev, uint32_t len, uint32_t kshift)
{
    const uint32_t nblk_slice = (len + kBlockBins - 1) / kBlockBins;
    const uint32_t npairs = (nblk_slice + 1) / 2;
    const uint32_t w = threadIdx.x >> 6;
    constexpr uint32_t NW = WG / 64;
    const uint64_t row_blk = row * P.nblk + blk0;
    if constexpr (CW == 16) {
        // No carry events: every count is its 16-bit half. Whole pairs inside
        // the slice go straight from the packed LDS words.
        if (nev == 0) {
            const uint32_t full = len / 512;
            for (uint32_t p0 = w * kFlushBatch; p0 < full; p0 += NW * kFlushBatch) {
                u32x4 ww[kFlushBatch];
#pragma unroll
                for (uint32_t j = 0; j < kFlushBatch; ++j)
                    ww[j] = reinterpret_cast<const u32x4 *>(lds)[min(p0 + j, full - 1) * 64 + lane_id()];
#pragma unroll
                for (uint32_t j = 0; j < kFlushBatch; ++j) {
                    if (p0 + j >= full) break;  // uniform
                    write_pair16(P, row_blk + 2 * (p0 + j), ww[j]);
                }
            }
            if (full < npairs && w == (full / kFlushBatch) % NW) {
                uint32_t c[8];
                slice_octet<CW>(lds, evlist, nev, full, len, kshift, c);
                write_pair(P, row_blk + 2 * full, min(2u, nblk_slice - 2 * full), c);
            }
            return;
        }
    }
    for (uint32_t p0 = w * kFlushBatch; p0 < npairs; p0 += NW * kFlushBatch) {
        uint32_t c[kFlushBatch][8];
#pragma unroll
        for (uint32_t j = 0; j < kFlushBatch; ++j)
            slice_octet<CW>(lds, evlist, nev, p0 + j < npairs ? p0 + j : npairs, len, kshift, c[j]);
#pragma unroll
        for (uint32_t j = 0; j < kFlushBatch; ++j) {
            if (p0 + j >= npairs) break;  // uniform
            const uint32_t kb = 2 * (p0 + j);
            write_pair(P, row_blk + kb, min(2u, nblk_slice - kb), c[j]);
        }
    }
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
// 32-bit (CW = 32) or packed 16-bit with carry events (CW = 16).
//
// Chunk g is body vectors [g * nvec / groups, (g + 1) * nvec / groups); the
// head scalars belong to chunk 0 and the tail scalars to the last chunk.
// The slice goes to partial row g in 256-bin blocks (range_bins is a multiple
// of 256), or straight into direct[] (the output) when there is one chunk;
// accumulate != 0 adds to direct[] instead of overwriting it.
template <int WG, int UNROLL, int AGG, int CW>
__global__ __launch_bounds__(WG) void k_sweep(InputView in, uint32_t num_bins, uint32_t range_bins,
                                              uint32_t ranges, uint32_t groups, uint32_t xcds,
                                              uint32_t kshift, Partials out,
                                              uint32_t *__restrict__ direct, uint32_t accumulate)
{
    extern __shared__ u32x4 lds4[];
    uint32_t *lds = reinterpret_cast<uint32_t *>(lds4);
    uint32_t *ev_count = lds + range_bins / 2;  // CW == 16 only
    uint32_t *evlist = ev_count + 4;
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
    constexpr uint32_t STEP = WG * UNROLL;
    uint64_t v = v0;

    // The first batch of loads is in flight while the LDS slice is cleared,
    // and every later batch is requested before the previous one is counted,
    // so each wave keeps 2 * UNROLL vector loads outstanding.
    i32x4 nx[UNROLL];
    const bool any_full = v + STEP <= v1;
    if (any_full) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) nx[u] = load_vec<true>(body + v + u * WG + tid);
    }
    zero_lds<WG>(lds, CW == 32 ? (len << kshift) : (len + 1) / 2);
    if (CW == 16 && tid == 0) *ev_count = 0u;
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
        else lds_count16<PEEL>(lds, evlist, ev_count, s, ok);
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
                        const uint32_t kk = min(t, 32768u);
                        add16(lds, evlist, ev_count, hs.h, kk);
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

    for (; any_full && v + STEP <= v1; v += STEP) {
        i32x4 q[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) q[u] = nx[u];
        if (v + 2 * STEP <= v1) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) nx[u] = load_vec<true>(body + v + STEP + u * WG + tid);
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
            } else {
#pragma unroll
                for (int e = 0; e < 4 * UNROLL; ++e) lds_count<0>(lds, (sl[e] << kshift) | rep, ok[e]);
            }
        } else {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) count4(q[u], true);
        }
    }
    // Remainder with a wave-uniform trip count.
    for (; v < v1; v += WG) {
        const bool ok = v + tid < v1;
        const i32x4 q = ok ? load_vec<true>(body + v + tid) : i32x4{0, 0, 0, 0};
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
    hot_flush();
    __syncthreads();

    const uint32_t nev = CW == 16 ? min(*ev_count, kEventCap) : 0u;
    if (direct) {
        const uint32_t npairs = (len + 511) / 512;
        for (uint32_t p = tid >> 6; p < npairs; p += WG / 64) {
            uint32_t c[8];
            slice_octet<CW>(lds, evlist, nev, p, len, kshift, c);
            const uint32_t b0 = lo + p * 512 + lane_id() * 8;
#pragma unroll
            for (uint32_t i = 0; i < 8; ++i)
                if (b0 + i < num_bins && b0 + i - lo < len)
                    direct[b0 + i] = (accumulate ? direct[b0 + i] : 0u) + c[i];
        }
    } else {
        flush_slice<WG, CW>(out, g, lo / kBlockBins, lds, evlist, nev, len, kshift);
    }
}

// The exclusive owner's write of bins b0..b0+3 (those below num_bins):
// counts = t, or counts += t (mod 2^32) when ACC.
template <bool ACC>
__device__ __forceinline__ void store_counts(uint32_t *__restrict__ counts, uint64_t b0,
                                             uint32_t num_bins, u32x4 t)
{
    const uint32_t v[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (b0 + k < num_bins) counts[b0 + k] = (ACC ? counts[b0 + k] : 0u) + v[k];
}

// ---------------------------------------------------------------------------
// Exclusive-owner merge: counts[b] = sum over rows g < rows of partial[g][b].
//
// A workgroup owns one 256-bin block and writes each of its bins once
// (merge_block does the reading and summing, k_merge_slots uses it too). Lane
// l of wave w reads 16 bytes of a plane per row: the 32 bins of chunk
// c = l / 8 of the block, from row slot i = l mod 8 of the wave's 8 rows of
// a round (8 * WAVES rows per round). A batch is kMergeRounds rounds, and
// all of its loads of one plane are issued before any is used. A lane sums
// its rows' nibbles bytewise, then widens them into 32 counters. Plane 0
// exists for every row; planes 1..7 are fetched only when the batch's width
// codes (one ballot) ask for them, each lane for its own rows. Finally the 8
// lanes of a chunk are summed with DPP, the waves through LDS.
constexpr uint32_t kMergeRounds = 8;

// acc[j] += sum over t of nibble j of v[t] (32 nibbles as 4 words), shifted
// to plane q's weight 16^q. The nibbles are first summed bytewise, even and
// odd nibbles apart; kMergeRounds * 15 < 256 keeps each byte exact.
__device__ __forceinline__ void add_nibbles_bytewise(uint32_t (&acc)[32],
                                                     const u32x4 (&v)[kMergeRounds], uint32_t q)
{
    u32x4 se = {0u, 0u, 0u, 0u}, so = {0u, 0u, 0u, 0u};
#pragma unroll
    for (uint32_t t = 0; t < kMergeRounds; ++t) {
        se += v[t] & 0x0F0F0F0Fu;
        so += (v[t] >> 4) & 0x0F0F0F0Fu;
    }
    const uint32_t e4[4] = {se.x, se.y, se.z, se.w}, o4[4] = {so.x, so.y, so.z, so.w};
    const uint32_t sh = 4u * q;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            acc[8 * k + 2 * bb] += ((e4[k] >> (8 * bb)) & 0xFFu) << sh;
            acc[8 * k + 2 * bb + 1] += ((o4[k] >> (8 * bb)) & 0xFFu) << sh;
        }
    }
}

// Sum over rows row0 .. row0 + rows - 1 of block blk of the partial rows
// (rows whose row_ok(k) is false, k the row's index from row0, are skipped).
// Whole workgroup of WAVES waves, convergent; the sums are valid in wave 0,
// lane l holding bins 4l..4l+3 of the block.
template <int WAVES, typename RowOk>
__device__ __forceinline__ u32x4 merge_block(const Partials &P, uint64_t row0, uint32_t rows,
                                             uint64_t blk, RowOk row_ok)
{
    constexpr uint32_t RPR = 8 * WAVES;  // rows per round
    __shared__ u32x4 red[WAVES][64];
    const uint32_t lane = lane_id(), w = threadIdx.x >> 6;
    const uint32_t c = lane >> 3, i = lane & 7u;
    uint32_t acc[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[j] = 0u;
    for (uint32_t base = 0; base < rows; base += kMergeRounds * RPR) {
        // lane l: the width code of round l / 8, slot l mod 8
        const uint32_t crow = base + (lane >> 3) * RPR + w * 8 + i;
        const uint32_t code =
            crow < rows && row_ok(crow) ? P.width[(row0 + crow) * P.nblk + blk] : 0u;
        u32x4 v[kMergeRounds];
#pragma unroll
        for (uint32_t t = 0; t < kMergeRounds; ++t) {
            const uint32_t k = base + t * RPR + w * 8 + i;
            v[t] = k < rows && row_ok(k)
                       ? *reinterpret_cast<const u32x4 *>(
                             P.plane0 + ((row0 + k) * P.nblk + blk) * kPlaneBytes + 16u * c)
                       : u32x4{0u, 0u, 0u, 0u};
        }
        add_nibbles_bytewise(acc, v, 0);
        // Planes beyond 0: each lane fetches them for its own rows of the batch,
        // all rows of one plane at once (plane q of a row exists iff q < planes).
        if (__ballot(code != 0u)) {
            const uint32_t maxp = __ballot(code == 7u) ? 8u : __ballot(code == 3u) ? 4u : 2u;
            uint32_t pl[kMergeRounds];
#pragma unroll
            for (uint32_t t = 0; t < kMergeRounds; ++t)
                pl[t] = (uint32_t)__shfl((int)code, (int)(8 * t + i), 64) + 1u;
            for (uint32_t q = 1; q < maxp; ++q) {
#pragma unroll
                for (uint32_t t = 0; t < kMergeRounds; ++t) {
                    const uint64_t row = row0 + base + t * RPR + w * 8 + i;
                    v[t] = q < pl[t] ? *reinterpret_cast<const u32x4 *>(
                                           P.upper + ((row * P.nblk + blk) * kUpperPlanes + q - 1) *
                                                         kPlaneBytes + 16u * c)
                                     : u32x4{0u, 0u, 0u, 0u};
                }
                add_nibbles_bytewise(acc, v, q);
            }
        }
    }
    // sum over the 8 lanes of each chunk: swap pairs, swap pair halves, mirror halves of 8
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        acc[j] += (uint32_t)__builtin_amdgcn_mov_dpp((int)acc[j], 0xB1, 0xF, 0xF, false);
        acc[j] += (uint32_t)__builtin_amdgcn_mov_dpp((int)acc[j], 0x4E, 0xF, 0xF, false);
        acc[j] += (uint32_t)__builtin_amdgcn_mov_dpp((int)acc[j], 0x141, 0xF, 0xF, false);
    }
    // lane 8c + i keeps bins 32c + 4i .. 32c + 4i + 3: red[w] holds the block in bin order
    u32x4 mine = {acc[0], acc[1], acc[2], acc[3]};
#pragma unroll
    for (uint32_t k = 1; k < 8; ++k)
        if (i == k) mine = u32x4{acc[4 * k], acc[4 * k + 1], acc[4 * k + 2], acc[4 * k + 3]};
    red[w][lane] = mine;
    __syncthreads();
    u32x4 t = {0u, 0u, 0u, 0u};
    if (w == 0) {
#pragma unroll
        for (int k = 0; k < WAVES; ++k) t += red[k][lane];
    }
    return t;
}

struct AllRows {
    __device__ bool operator()(uint32_t) const { return true; }
};

// ACC: add into counts instead of overwriting it (a template parameter, so
// that the overwriting kernel carries no branch around its stores).
template <int WAVES, bool ACC>
__global__ __launch_bounds__(WAVES * 64) void k_merge(Partials P, uint32_t rows, uint32_t num_bins,
                                                      uint32_t *__restrict__ counts)
{
    const u32x4 t = merge_block<WAVES>(P, 0, rows, blockIdx.x, AllRows{});
    if ((threadIdx.x >> 6) == 0)
        store_counts<ACC>(counts, (uint64_t)blockIdx.x * kBlockBins + lane_id() * 4u, num_bins, t);
}

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
// the range is implied by the position.
//
// Returning atomics on one LDS word are served one lane at a time (each lane
// needs its own rank), so every range's counter is split into 2^qlog
// sub-counters chosen by lane (lane mod 2^qlog): lanes that route to the same
// range then rarely share a word. The scan runs over [range][sub] order, so a
// range's elements stay contiguous. Per tile and range the kernel writes the
// run's length and start (tcnt, tbase; layout [range][tile]). Element order
// inside a run is whatever the atomics gave; counts do not depend on it.
template <int WG, int VPT>
__global__ __launch_bounds__(WG) void k_partition(InputView in, uint32_t num_bins, uint32_t shift,
                                                  uint32_t ranges, uint32_t qlog, uint32_t tiles,
                                                  uint16_t *__restrict__ stage, uint32_t stage_cap,
                                                  uint32_t *__restrict__ tcnt,
                                                  uint32_t *__restrict__ tbase)
{
    extern __shared__ u32x4 smem4[];
    const uint32_t nsub = ranges << qlog;  // <= 2 * WG
    const uint32_t npad = (nsub + 3u) & ~3u;
    uint32_t *cnt = reinterpret_cast<uint32_t *>(smem4);
    uint32_t *base = cnt + npad;
    uint32_t *scratch = base + npad;  // block scan scratch + total
    uint16_t *st = reinterpret_cast<uint16_t *>(scratch + 64);
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
    uint32_t t = blockIdx.x;
    if (t < tiles) load_tile(t);
    for (uint32_t i = tid; i < nsub; i += WG) cnt[i] = 0u;
    __syncthreads();

    for (; t < tiles; t += gridDim.x) {
        uint32_t x[E + 2], rk[E + 2];
#pragma unroll
        for (int e = 0; e < E + 2; ++e) x[e] = nx[e];
        if (t + gridDim.x < tiles) load_tile(t + gridDim.x);
#pragma unroll
        for (int e = 0; e < E + 2; ++e) {
            rk[e] = 0u;
            if (x[e] < num_bins) rk[e] = lds_add_rtn(cnt, ((x[e] >> shift) << qlog) | q, 1u);
        }
        __syncthreads();

        {
            const uint32_t i0 = 2 * tid, i1 = 2 * tid + 1;
            const uint32_t c0 = i0 < nsub ? cnt[i0] : 0u, c1 = i1 < nsub ? cnt[i1] : 0u;
            uint32_t total;
            const uint32_t ex = block_exclusive_scan<WG>(c0 + c1, scratch, &total);
            if (i0 < nsub) base[i0] = ex;
            if (i1 < nsub) base[i1] = ex + c0;
            if (tid == 0) scratch[63] = total;
        }
        __syncthreads();
        const uint32_t nvalid = scratch[63];
        for (uint32_t r = tid; r < ranges; r += WG) {
            const uint32_t b0 = base[r << qlog];
            const uint32_t b1 = r + 1 < ranges ? base[(r + 1) << qlog] : nvalid;
            tcnt[(uint64_t)r * tiles + t] = b1 - b0;
            tbase[(uint64_t)r * tiles + t] = b0;
        }
#pragma unroll
        for (int e = 0; e < E + 2; ++e)
            if (x[e] < num_bins) st[base[((x[e] >> shift) << qlog) | q] + rk[e]] = (uint16_t)(x[e] & mask);
        __syncthreads();

        // counters are free again: clear them for the next tile while copying out
        for (uint32_t i = tid; i < nsub; i += WG) cnt[i] = 0u;
        const uint32_t nv = (nvalid + 7u) >> 3;
        const u32x4 *s4 = reinterpret_cast<const u32x4 *>(st);
        u32x4 *d4 = reinterpret_cast<u32x4 *>(stage + (uint64_t)t * stage_cap);
        for (uint32_t i = tid; i < nv; i += WG) d4[i] = s4[i];
        __syncthreads();  // staging and counters are reused by the next tile
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
template <int WG, int UNROLL, int AGG>
__global__ __launch_bounds__(WG) void k_bucket_hist(
    const uint16_t *__restrict__ stage, uint32_t stage_cap, const uint32_t *__restrict__ tcnt,
    const uint32_t *__restrict__ tbase, const uint32_t *__restrict__ tpre,
    const uint32_t *__restrict__ totals, uint32_t ranges, uint32_t tiles, uint32_t range_bins,
    uint32_t num_bins, uint32_t owners, Partials out)
{
    extern __shared__ u32x4 lds4[];
    uint32_t *lds = reinterpret_cast<uint32_t *>(lds4);
    uint64_t *bs = reinterpret_cast<uint64_t *>(lds + range_bins);  // [ranges + 1]
    uint32_t *misc = reinterpret_cast<uint32_t *>(bs + ranges + 1);  // [0] ta [1] tb
    const uint32_t tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    constexpr uint32_t NW = WG / 64;  // waves
    constexpr uint32_t RPW = UNROLL;  // tiles (runs) per wave group = loads in flight per lane

    range_starts(totals, ranges, bs);
    __syncthreads();
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

        // Teams of S waves: team w / S takes groups of RPW tiles (every NW / S-th
        // group), and its S waves stripe each run's vectors. S is the smallest
        // power of two that still leaves every team two groups, so long runs
        // (few ranges, or an input piled into one range) keep all waves busy.
        const uint32_t ngroups = (tb - ta + RPW - 1) / RPW;
        uint32_t S = 1;
        while (S < NW && ngroups < 2u * (NW / S)) S *= 2u;
        const uint32_t team = w / S, member = w % S;
        for (uint32_t g0 = ta + team * RPW; g0 < tb; g0 += (NW / S) * RPW) {
            // lane m < RPW: the run of tile g0 + m, clipped to [p0, p1)
            uint32_t vlo = 0, nv = 0, skip = 0, used = 0;
            const uint32_t t = g0 + lane;
            if (lane < RPW && t < tb) {
                const uint32_t c = rc[t], q = rpre[t], bse = rbase[t];
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
                    qv[m] = ok ? stage_vec[(uint64_t)run_v[m] + d] : i32x4{0, 0, 0, 0};
                }
#pragma unroll
                for (uint32_t k = 0; k < RPW; ++k) {
                    const uint32_t words[4] = {(uint32_t)qv[k].x, (uint32_t)qv[k].y,
                                               (uint32_t)qv[k].z, (uint32_t)qv[k].w};
                    if constexpr (AGG == 1) {
                        uint32_t nxt;
                        if (hot_should_switch(hs, words[0] & 0xFFFFu, first[k] == 0u && last[k] > 0u,
                                              &nxt)) {
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
        flush_slice<WG, 32>(out, i + r, 0, lds, nullptr, 0, len, 0);
        __syncthreads();
    }
}

// Phase 2b: counts[b] for the bins of one range = the sum of the slots that
// the owners overlapping the range wrote for it (exclusive owner per bin, no
// global atomics). A workgroup handles one 256-bin block of one range. Owner
// i wrote the range's slot to row i + r, so the slots of the overlapping
// owners first..last are consecutive rows, summed by merge_block. An owner
// that took no element (possible only when there are fewer elements than
// owners) wrote no slot and is skipped. Empty ranges give zeros.
template <int WAVES, bool ACC>
__global__ __launch_bounds__(WAVES * 64) void k_merge_slots(Partials P, const uint32_t *__restrict__ totals,
                                                            uint32_t ranges, uint32_t range_bins,
                                                            uint32_t num_bins, uint32_t owners,
                                                            uint32_t *__restrict__ counts)
{
    __shared__ uint64_t se[3];
    const uint32_t lane = lane_id(), w = threadIdx.x >> 6;
    const uint32_t bpr = range_bins / kBlockBins;  // blocks per range
    const uint32_t r = blockIdx.x / bpr, lb = blockIdx.x % bpr;
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
    uint32_t first = 0, rows = 0;
    if (re > rb) {
        first = owner_of(rb, N, owners);
        rows = owner_of(re - 1, N, owners) - first + 1;
    }
    // every owner took at least one element when N >= owners
    const bool all_nonempty = N >= owners;
    auto row_ok = [&](uint32_t k) {
        const uint64_t i = (uint64_t)first + k;
        return all_nonempty || i * N / owners < (i + 1) * N / owners;
    };
    const u32x4 t = merge_block<WAVES>(P, (uint64_t)first + r, rows, lb, row_ok);
    if (w == 0)
        store_counts<ACC>(counts, (uint64_t)r * range_bins + lb * kBlockBins + lane * 4u, num_bins, t);
}

}  // namespace pca
