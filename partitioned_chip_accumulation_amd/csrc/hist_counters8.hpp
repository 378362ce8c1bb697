// hist_counters8.hpp -- 8-bit LDS counters kept exact by carry events
//
// Part of the gfx950 kernels of libpca_hist.so (see hist_kernels.hpp for the
// overview).
#pragma once

#include "hist_common.hpp"

namespace pca {

// ---------------------------------------------------------------------------
// 8-bit LDS counters.
//
// Four bins share one 32-bit LDS word, bin 4w + p in byte p of word w, so a
// workgroup's 160 KiB hold about 155,000 bins. An add of k (1 <= k <= 255) to
// bin 4w + p is ds_add_rtn_u32 of k << 8p. A byte that overflows carries into
// the next byte of the word (which can overflow in turn), and a carry out of
// byte 3 leaves the word. The returned old value shows every carry: with
// new = old + delta, bit 8q + 8 of old ^ delta ^ new is the carry out of byte
// q < 3, and new < old is the carry out of byte 3. Each carry out of byte q
// is appended to an LDS list as the entry 4w + q. With C_q the carries out of
// byte q of the final word W, the true counts are
//     A_q = byte_q(W) + 256 C_q - C_(q-1)   (C_(-1) = 0).
// Every carry out of a byte takes 256 units into it, and the units into byte
// q are the adds to bin q plus the carries out of byte q - 1, so from zero a
// workgroup that counts E elements logs at most E / 255 events. The list
// takes the LDS the slice leaves (at least kMinEventCap8 entries, cap in
// all) and goes on for kEvSpill8 entries in the workgroup's own area of the
// workspace, and the host keeps E <= 255 (cap + kEvSpill8 - 16), which
// bounds it.
constexpr uint32_t kMinEventCap8 = 2048;
constexpr uint32_t kEvSpill8 = 512;

// A workgroup's carry-event list: cap entries in LDS, then (spill not null)
// kEvSpill8 more in global memory, written with plain stores and read by the
// same workgroup after a barrier. The 16-bit counters use lds, count and cap
// only.
struct EvList {
    uint32_t *lds;
    uint32_t *count;  // LDS word: entries logged
    uint32_t cap;
    uint32_t *spill;
};

__device__ __forceinline__ void put_event8(const EvList &ev, uint32_t i, uint32_t x)
{
    if (i < ev.cap) ev.lds[i] = x;
    else if (ev.spill != nullptr && i - ev.cap < kEvSpill8) ev.spill[i - ev.cap] = x;
}

__device__ __forceinline__ uint32_t event8_at(const EvList &ev, uint32_t e)
{
    return e < ev.cap ? ev.lds[e] : ev.spill[e - ev.cap];
}

// Entries logged that the list holds.
__device__ __forceinline__ uint32_t events8_held(const EvList &ev)
{
    return min(*ev.count, ev.cap + (ev.spill != nullptr ? kEvSpill8 : 0u));
}

// Bit q set: the add of delta to a word that held old carried out of byte q.
__device__ __forceinline__ uint32_t carry_bits8(uint32_t old, uint32_t delta)
{
    const uint32_t nw = old + delta;
    const uint32_t x = old ^ delta ^ nw;  // the carry into every bit
    return ((x >> 8) & 1u) | ((x >> 15) & 2u) | ((x >> 22) & 4u) | (nw < old ? 8u : 0u);
}

// Log the carries of an add of delta = k << 8p to word w that returned old
// (one lane on its own).
__device__ __forceinline__ void log_carries8(const EvList &ev, uint32_t w, uint32_t old,
                                             uint32_t delta)
{
    const uint32_t bits = carry_bits8(old, delta);
    if (bits == 0u) return;
    uint32_t i = lds_add_rtn(ev.count, 0, (uint32_t)__popc(bits));
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q) {
        if ((bits >> q) & 1u) {
            put_event8(ev, i, (w << 2) | q);
            ++i;
        }
    }
}

__device__ __forceinline__ void add8(uint32_t *words, const EvList &ev, uint32_t s, uint32_t k)
{
    const uint32_t delta = k << ((s & 3u) << 3);
    const uint32_t old = lds_add_rtn(words, s >> 2, delta);
    log_carries8(ev, s >> 2, old, delta);
}

// Log the carries of an add of one to byte q0 = t / 8 (t mod 32 its bit
// offset) of the word at slot offset a (a multiple of 4), which returned old
// with that byte 0xFF (one lane on its own). The carry leaves byte q0 and runs
// on through every 0xFF byte above it, up to byte 3: n >= 1 events, entries
// a | q0 .. a | (q0 + n - 1). The bytes of ~old above bit t are zero exactly
// where old's are 0xFF, so n is the count of whole zero bytes at the bottom
// of ~old >> t, capped at the word's top byte.
__device__ __forceinline__ void log_carry_chain8(const EvList &ev, uint32_t a, uint32_t old,
                                                 uint32_t t)
{
    const uint32_t q0 = (t >> 3) & 3u;
    const uint32_t y = ~old >> (t & 31u);
    const uint32_t n = y == 0u ? 4u - q0 : min((uint32_t)__builtin_ctz(y) >> 3, 4u - q0);
    uint32_t i = lds_add_rtn(ev.count, 0, n);
    put_event8(ev, i, a | q0);
    for (uint32_t j = 1; j < n; ++j) put_event8(ev, i + j, a | (q0 + j));
}

// Unaggregated 8-bit counting of N elements at once (all ds_add_rtn_u32 are
// issued before any returned value is examined; N <= 15), into the counters
// at the start of the dynamic LDS block. The byte of slot s sits at bit
// 8 (s mod 4) of the word at byte offset s & ~3, and t = 8 s holds that bit
// offset in its low five bits, the only ones the shift and the bit-field
// extract below read. An add of 1 can carry only when the byte it increments
// was 0xFF. A batch in which some lane carried takes one wave-uniform branch,
// where each lane logs its own carries with one LDS atomic on the list length
// per element that carried (mostly one element of one lane). Skewed input,
// whose hot bins wrap a byte every 256 counts, takes this branch often, so it
// stays short.
template <int N>
__device__ __forceinline__ void count8_batch(const EvList &ev, const uint32_t (&s)[N],
                                             const bool (&ok)[N])
{
    uint32_t old[N], t[N], a[N];
#pragma unroll
    for (int e = 0; e < N; ++e) {
        t[e] = s[e] << 3;
        a[e] = s[e] & ~3u;
        // a lane that does not count keeps the increment, which is dead after
        // the add (the returned value can take its register: no copy)
        old[e] = shl_mod32(1u, t[e]);
        if (ok[e]) old[e] = dyn_lds_add_rtn(a[e], old[e]);
    }
    bool hit[N], any = false;
#pragma unroll
    for (int e = 0; e < N; ++e) {
        hit[e] = ok[e] && __builtin_amdgcn_ubfe(old[e], t[e], 8) == 0xFFu;
        any = any || hit[e];
    }
    if (__ballot(any)) {
#pragma unroll
        for (int e = 0; e < N; ++e)
            if (hit[e]) log_carry_chain8(ev, a[e], old[e], t[e]);
    }
}

template <int ROUNDS>
__device__ __forceinline__ void lds_count8(uint32_t *words, const EvList &ev, uint32_t slot,
                                           bool valid)
{
    if constexpr (ROUNDS == 0) {
        if (valid) add8(words, ev, slot, 1u);
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
                add8(words, ev, lead, (uint32_t)__popcll(m));  // <= 64
            pending = pending && !mine;
            if (__popcll(m) == 1) break;
        }
        if (pending) add8(words, ev, slot, 1u);
    }
}

// The counts a lane holds for up to four pairs of blocks, as 32 named
// scalars rather than an array: the compiler keeps an array of this size as
// one 32-register tuple, which a branch that changes one element copies
// whole.
struct Counts32 {
    uint32_t v0, v1, v2, v3, v4, v5, v6, v7;          // pair 0 of the batch
    uint32_t v8, v9, v10, v11, v12, v13, v14, v15;    // pair 1
    uint32_t v16, v17, v18, v19, v20, v21, v22, v23;  // pair 2
    uint32_t v24, v25, v26, v27, v28, v29, v30, v31;  // pair 3
};
constexpr uint32_t Counts32::*kCountMember[32] = {
    &Counts32::v0,  &Counts32::v1,  &Counts32::v2,  &Counts32::v3,
    &Counts32::v4,  &Counts32::v5,  &Counts32::v6,  &Counts32::v7,
    &Counts32::v8,  &Counts32::v9,  &Counts32::v10, &Counts32::v11,
    &Counts32::v12, &Counts32::v13, &Counts32::v14, &Counts32::v15,
    &Counts32::v16, &Counts32::v17, &Counts32::v18, &Counts32::v19,
    &Counts32::v20, &Counts32::v21, &Counts32::v22, &Counts32::v23,
    &Counts32::v24, &Counts32::v25, &Counts32::v26, &Counts32::v27,
    &Counts32::v28, &Counts32::v29, &Counts32::v30, &Counts32::v31};

template <int K>
__device__ __forceinline__ uint32_t &count_at(Counts32 &c)
{
    return c.*kCountMember[K];
}

// One carry event out of count k (wave-uniform, k in [LO, HI)): c[k] += add
// and, unless k is byte 3 of its word (whose carry leaves the word),
// c[k + 1] -= sub. A binary tree of scalar branches leads to a leaf that
// updates its registers by constant names; the updates are opaque
// instructions so that the compiler cannot merge the leaves back into one
// update at a run-time register index (GPR indexing mode), which it would
// otherwise do and which this code must not depend on.
template <int LO, int HI>
__device__ __forceinline__ void carry_at(Counts32 &c, uint32_t k, uint32_t add, uint32_t sub)
{
    if constexpr (HI - LO == 1) {
        asm volatile("v_add_u32 %0, %0, %1" : "+v"(count_at<LO>(c)) : "v"(add));
        if constexpr ((LO & 3) != 3)
            asm volatile("v_sub_u32 %0, %0, %1" : "+v"(count_at<LO + 1>(c)) : "v"(sub));
    } else {
        constexpr int MID = (LO + HI) / 2;
        if (k < (uint32_t)MID) carry_at<LO, MID>(c, k, add, sub);
        else carry_at<MID, HI>(c, k, add, sub);
    }
}

// Apply the carry events to the counts of J <= 4 pairs of blocks, pairs
// p0 + STRIDE j (j < J): c[8j + i] is bin 8l + i of pair p0 + STRIDE j
// (l = lane), byte i % 4 of its word 2l + i / 4. The wave reads the list 64
// entries at a time and takes only the entries in its pairs; an entry names
// one count, whose index in c is wave-uniform, so each distinct matching
// entry of a window costs a few scalar branches and two register updates in
// which only the owning lane's values change (its copies in the window are
// added at once). Whole wave, convergent; p0 uniform.
template <int J, int STRIDE>
__device__ __forceinline__ void apply_events8(const EvList &ev, uint32_t nev, uint32_t p0,
                                              Counts32 &c)
{
    const uint32_t lane = lane_id();
    // uniform in fact (derived from the wave index); said so, the entry index
    // below is computed in scalar registers
    p0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)p0);
    for (uint32_t e0 = 0; e0 < nev; e0 += 64) {
        const uint32_t e = e0 + lane;
        const uint32_t ent = e < nev ? event8_at(ev, e) : 0xFFFFFFFFu;
        const uint32_t dp = (ent >> 9) - p0;  // pair of the entry's word, from p0
        uint64_t m = __ballot(dp < (uint32_t)(STRIDE * J) && dp % STRIDE == 0u);
        while (m != 0) {
            const int k = __builtin_ctzll(m);
            const uint32_t ev = (uint32_t)__builtin_amdgcn_readlane((int)ent, k);
            // the window's copies of this entry (hot bytes repeat) are applied
            // together: mult events, +256 mult and -mult
            const uint64_t same = __ballot(ent == ev) & m;
            m &= ~same;
            const uint32_t mult = (uint32_t)__popcll(same);
            const uint32_t word = ev >> 2;
            const uint32_t idx = (((ev >> 9) - p0) / STRIDE) * 8u + (word & 1u) * 4u + (ev & 3u);
            const uint32_t hit = lane == ((word & 127u) >> 1) ? mult : 0u;
            carry_at<0, 8 * J>(c, idx, hit << 8, hit);
        }
    }
}

}  // namespace pca
