// hist_partials.hpp -- partial slices: nibble-planar layout, flush from LDS,
// exclusive-owner merge
//
// Part of the gfx950 kernels of libpca_hist.so (see hist_kernels.hpp for the
// overview).
#pragma once

#include "hist_common.hpp"
#include "hist_counters16.hpp"
#include "hist_counters8.hpp"

namespace pca {

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

// Plane q (0 or 1) of eight 8-bit counts held four per word (count 4k + i in
// byte i of word k), as one word of nibbles.
__device__ __forceinline__ uint32_t plane_word8(u32x2 w, uint32_t q)
{
    const uint32_t sh = 4u * q;
    // nibbles of counts 0..3 at bits 0, 8, 16, 24 (z likewise for 4..7), then
    // each even nibble joined with its odd neighbour and the two bytes packed
    uint32_t y = (w.x >> sh) & 0x0F0F0F0Fu, z = (w.y >> sh) & 0x0F0F0F0Fu;
    y |= y >> 4;
    z |= z >> 4;
    return (y & 0xFFu) | ((y >> 8) & 0xFF00u) | ((z & 0xFFu) << 16) | ((z << 8) & 0xFF000000u);
}

// write_pair for counts that are exact in 8 bits, read straight from packed
// LDS words (lane l: bins 8l..8l+7 of the pair as two words). Both blocks of
// the pair exist. Whole wave, convergent.
__device__ __forceinline__ void write_pair8(const Partials &P, uint64_t blk_even, u32x2 w)
{
    const uint32_t lane = lane_id();
    const uint64_t wide = __ballot(((w.x | w.y) & 0xF0F0F0F0u) != 0u);
    store_through(reinterpret_cast<uint32_t *>(P.plane0 + blk_even * kPlaneBytes) + lane,
                  plane_word8(w, 0));
    if (wide == 0) {
        // the common case: both blocks fit 4 bits, plane 0 only
        if ((lane & 31u) == 0) P.width[blk_even + (lane >> 5)] = 0;
        return;
    }
    const uint32_t planes = (uint32_t)(wide >> (lane & 32u)) ? 2u : 1u;
    const uint64_t blk = blk_even + (lane >> 5);
    if (planes == 2u)
        store_through(reinterpret_cast<uint32_t *>(P.upper + blk * kUpperPlanes * kPlaneBytes) +
                          (lane & 31u),
                      plane_word8(w, 1));
    if ((lane & 31u) == 0) P.width[blk] = (uint8_t)(planes - 1);
}

// The eight bytes of bins 8l..8l+7 (l = lane) of pair p, as stored in 8-bit
// LDS counters (before carry events), into c[8j..8j+7]; zero for a lane
// whose bins all lie at or beyond len. j is a compile-time index.
template <int J>
__device__ __forceinline__ void octet8_raw(const uint32_t *lds, uint32_t p, uint32_t len,
                                           Counts32 &cv)
{
    const uint32_t b0 = p * 512u + lane_id() * 8u;
    u32x2 w = {0u, 0u};
    if (b0 < len) w = reinterpret_cast<const u32x2 *>(lds)[b0 / 8];
    count_at<8 * J + 0>(cv) = w.x & 0xFFu;
    count_at<8 * J + 1>(cv) = (w.x >> 8) & 0xFFu;
    count_at<8 * J + 2>(cv) = (w.x >> 16) & 0xFFu;
    count_at<8 * J + 3>(cv) = w.x >> 24;
    count_at<8 * J + 4>(cv) = w.y & 0xFFu;
    count_at<8 * J + 5>(cv) = (w.y >> 8) & 0xFFu;
    count_at<8 * J + 6>(cv) = (w.y >> 16) & 0xFFu;
    count_at<8 * J + 7>(cv) = w.y >> 24;
}

// c[0..7] = counts 8j..8j+7 of cv.
template <int J>
__device__ __forceinline__ void octet_of(Counts32 &cv, uint32_t (&c)[8])
{
    c[0] = count_at<8 * J + 0>(cv); c[1] = count_at<8 * J + 1>(cv);
    c[2] = count_at<8 * J + 2>(cv); c[3] = count_at<8 * J + 3>(cv);
    c[4] = count_at<8 * J + 4>(cv); c[5] = count_at<8 * J + 5>(cv);
    c[6] = count_at<8 * J + 6>(cv); c[7] = count_at<8 * J + 7>(cv);
}

__device__ __forceinline__ void mask_octet(uint32_t p, uint32_t len, uint32_t (&c)[8])
{
    const uint32_t b0 = p * 512u + lane_id() * 8u;
#pragma unroll
    for (uint32_t i = 0; i < 8; ++i)
        if (b0 + i >= len) c[i] = 0u;
}

// Counts of bins 8l..8l+7 (l = lane) of pair p (bins 512p..512p+511) of a
// slice, from 32-bit, 16-bit or 8-bit LDS counters. Bins at or beyond len
// read as zero; a lane whose bins all lie beyond len reads no LDS. The
// slice's LDS holds at least round_up(len, 256) counters, so a partly valid
// lane stays inside it. With 8-bit counters the whole wave must call it
// (uniform p): the carry events are applied by the wave together.
template <int CW>
__device__ __forceinline__ void slice_octet(const uint32_t *lds, const EvList &ev,
                                            uint32_t nev, uint32_t p, uint32_t len,
                                            uint32_t kshift, uint32_t (&c)[8])
{
    const uint32_t b0 = p * 512u + lane_id() * 8u;
    if constexpr (CW == 8) {
        Counts32 cv;
        octet8_raw<0>(lds, p, len, cv);
        // a carry out of the last valid byte lands in an invalid one: mask after
        apply_events8<1, 1>(ev, nev, p, cv);
        octet_of<0>(cv, c);
        mask_octet(p, len, c);
        return;
    }
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
            const uint32_t ent = ev.lds[e];
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
                                            const uint32_t *lds, const EvList &ev,
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
                slice_octet<CW>(lds, ev, nev, full, len, kshift, c);
                write_pair(P, row_blk + 2 * full, min(2u, nblk_slice - 2 * full), c);
            }
            return;
        }
    }
    if constexpr (CW == 8) {
        if (nev == 0) {
            // no carry events: every count is its byte
            const uint32_t full = len / 512;
            for (uint32_t p0 = w * kFlushBatch; p0 < full; p0 += NW * kFlushBatch) {
                u32x2 ww[kFlushBatch];
#pragma unroll
                for (uint32_t j = 0; j < kFlushBatch; ++j)
                    ww[j] = reinterpret_cast<const u32x2 *>(lds)[min(p0 + j, full - 1) * 64 + lane_id()];
#pragma unroll
                for (uint32_t j = 0; j < kFlushBatch; ++j) {
                    if (p0 + j >= full) break;  // uniform
                    write_pair8(P, row_blk + 2 * (p0 + j), ww[j]);
                }
            }
            if (full < npairs && w == (full / kFlushBatch) % NW) {
                uint32_t c[8];
                slice_octet<CW>(lds, ev, nev, full, len, kshift, c);
                write_pair(P, row_blk + 2 * full, min(2u, nblk_slice - 2 * full), c);
            }
            return;
        }
        // One pass over the event list per batch of pairs. A batch is four
        // pairs NW apart, so that a contiguous run of event-heavy pairs (the
        // hot core of a skewed input) is spread over up to NW waves, each of
        // which applies its events one at a time.
        for (uint32_t p0 = w; p0 < npairs; p0 += NW * kFlushBatch) {
            static_assert(kFlushBatch == 4, "Counts32 holds four pairs");
            Counts32 cv;
            octet8_raw<0>(lds, p0 + 0 * NW, len, cv);
            octet8_raw<1>(lds, p0 + 1 * NW, len, cv);
            octet8_raw<2>(lds, p0 + 2 * NW, len, cv);
            octet8_raw<3>(lds, p0 + 3 * NW, len, cv);
            apply_events8<kFlushBatch, NW>(ev, nev, p0, cv);
            uint32_t c[kFlushBatch][8];
            octet_of<0>(cv, c[0]);
            octet_of<1>(cv, c[1]);
            octet_of<2>(cv, c[2]);
            octet_of<3>(cv, c[3]);
#pragma unroll
            for (uint32_t j = 0; j < kFlushBatch; ++j) {
                const uint32_t p = p0 + j * NW;
                if (p >= npairs) break;  // uniform
                mask_octet(p, len, c[j]);
                write_pair(P, row_blk + 2 * p, min(2u, nblk_slice - 2 * p), c[j]);
            }
        }
        return;
    }
    for (uint32_t p0 = w * kFlushBatch; p0 < npairs; p0 += NW * kFlushBatch) {
        uint32_t c[kFlushBatch][8];
#pragma unroll
        for (uint32_t j = 0; j < kFlushBatch; ++j)
            slice_octet<CW>(lds, ev, nev, p0 + j < npairs ? p0 + j : npairs, len, kshift, c[j]);
#pragma unroll
        for (uint32_t j = 0; j < kFlushBatch; ++j) {
            if (p0 + j >= npairs) break;  // uniform
            const uint32_t kb = 2 * (p0 + j);
            write_pair(P, row_blk + kb, min(2u, nblk_slice - kb), c[j]);
        }
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
// a round (8 * WAVES rows per round). A batch is kMergeRounds rounds (or fewer), and
// all of its loads of one plane are issued before any is used. A lane sums
// its rows' nibbles bytewise, then widens them into 32 counters. Plane 0
// exists for every row; planes 1..7 are fetched only when the batch's width
// codes (one ballot) ask for them, each lane for its own rows. Finally the 8
// lanes of a chunk are summed with DPP, the waves through LDS.
constexpr uint32_t kMergeRounds = 8;

// acc[j] += sum over t of nibble j of v[t] (32 nibbles as 4 words), shifted
// to plane q's weight 16^q. The nibbles are first summed bytewise, even and
// odd nibbles apart; ROUNDS * 15 < 256 keeps each byte exact.
template <uint32_t ROUNDS>
__device__ __forceinline__ void add_nibbles_bytewise(uint32_t (&acc)[32], const u32x4 (&v)[ROUNDS],
                                                     uint32_t q)
{
    static_assert(ROUNDS * 15u < 256u, "bytewise nibble sums must not carry");
    u32x4 se = {0u, 0u, 0u, 0u}, so = {0u, 0u, 0u, 0u};
#pragma unroll
    for (uint32_t t = 0; t < ROUNDS; ++t) {
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
// lane l holding bins 4l..4l+3 of the block. A batch is ROUNDS rounds: fewer
// rounds hold fewer loads in flight per wave but need fewer registers, so
// more waves fit when there are few rows to sum.
template <int WAVES, uint32_t ROUNDS = kMergeRounds, typename RowOk>
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
    for (uint32_t base = 0; base < rows; base += ROUNDS * RPR) {
        // lane l: the width code of round l / 8, slot l mod 8
        const uint32_t crow = base + (lane >> 3) * RPR + w * 8 + i;
        const uint32_t code = (lane >> 3) < ROUNDS && crow < rows && row_ok(crow)
                                  ? P.width[(row0 + crow) * P.nblk + blk]
                                  : 0u;
        u32x4 v[ROUNDS];
#pragma unroll
        for (uint32_t t = 0; t < ROUNDS; ++t) {
            const uint32_t k = base + t * RPR + w * 8 + i;
            v[t] = k < rows && row_ok(k)
                       ? *reinterpret_cast<const u32x4 *>(
                             P.plane0 + ((row0 + k) * P.nblk + blk) * kPlaneBytes + 16u * c)
                       : u32x4{0u, 0u, 0u, 0u};
        }
        add_nibbles_bytewise<ROUNDS>(acc, v, 0);
        // Planes beyond 0: each lane fetches them for its own rows of the batch,
        // all rows of one plane at once (plane q of a row exists iff q < planes).
        if (__ballot(code != 0u)) {
            const uint32_t maxp = __ballot(code == 7u) ? 8u : __ballot(code == 3u) ? 4u : 2u;
            uint32_t pl[ROUNDS];
#pragma unroll
            for (uint32_t t = 0; t < ROUNDS; ++t)
                pl[t] = (uint32_t)__shfl((int)code, (int)(8 * t + i), 64) + 1u;
            for (uint32_t q = 1; q < maxp; ++q) {
#pragma unroll
                for (uint32_t t = 0; t < ROUNDS; ++t) {
                    const uint64_t row = row0 + base + t * RPR + w * 8 + i;
                    v[t] = q < pl[t] ? *reinterpret_cast<const u32x4 *>(
                                           P.upper + ((row * P.nblk + blk) * kUpperPlanes + q - 1) *
                                                         kPlaneBytes + 16u * c)
                                     : u32x4{0u, 0u, 0u, 0u};
                }
                add_nibbles_bytewise<ROUNDS>(acc, v, q);
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

}  // namespace pca
