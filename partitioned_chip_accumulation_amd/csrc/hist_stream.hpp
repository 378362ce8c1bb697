// hist_stream.hpp -- the streaming owner-queue path (STREAM): one persistent
// kernel in which producer waves route input tiles to the ranges that own
// their bins and owner workgroups count each range's elements in LDS as the
// tiles are published.
//
// Part of the gfx950 kernels of libpca_hist.so (see hist_kernels.hpp for the
// overview).
#pragma once

#include "hist_common.hpp"

namespace pca {

// ---------------------------------------------------------------------------
// Streaming path.
//
// The page "Distributed Shared Memory", section "The cluster histogram", has
// every element's increment sent to the block that owns its bin; the page
// "Hopper DSMEM vs HBM" hands data from one block to another through memory
// and a flag (its latency test). Here, in one persistent kernel:
//   - the first P workgroups to start are producers, and each of their waves
//     works on its own, with no workgroup barrier: it claims input tiles of
//     16,384 elements in turn (an atomic tile counter) and routes a tile in
//     sub-tiles of 2,048 elements. For a sub-tile it ranks every
//     element within its range with wave-private LDS counters, lays the
//     ranges' runs of 16-bit slots (bin & (S - 1)) out one after another,
//     each padded to whole 16-byte chunks with the slot kStreamPad, and
//     writes the slots and the sub-tile's run-table row (per range, start
//     << 16 | length). After the eighth sub-tile it publishes the tile with
//     one release store of the tile's flag. The loads of the next sub-tile
//     are in flight while the current one is routed;
//   - every other workgroup, and every producer once the tiles run out, is an
//     owner. An owner holds one range of S = 32,768 bins in LDS (32-bit
//     counters) and claims that range's blocks of BT consecutive tiles in
//     turn (an atomic per range). For each block one wave waits for the
//     tiles' flags, 64 at a time (an acquire after the last); then groups of
//     G lanes count the range's runs of the block's sub-tiles, one run per
//     group, four 16-byte chunks per lane in flight (G from the expected run
//     length). When the range has no block left, the owner writes its
//     counts (its stint) to a slot of a pool, takes the next slot from an
//     atomic counter and records the slot's range, and moves to the range
//     with the most blocks left, so the owners of a skewed input's heavy
//     ranges multiply as the light ones run out. Moves come from a budget
//     (an atomic counter): an owner denied one ends, which bounds the stints
//     by workgroups + budget, the pool's size. A range is never left with
//     blocks unclaimed: an owner leaves a range only when its last block is
//     claimed, and every range has an owner from the start or once the
//     producers turn owners (tickets cover every range).
//   - k_stream_merge then adds each range's stints (the sum of the slots
//     recorded for it) into the output, or writes them when not accumulating.
//     It runs after the persistent kernel, so it reads the pool with plain
//     loads; no lock or atomic touches the counts.
// Every wait can end: producers wait on nothing, and owners wait only on
// tiles that a producer which has started (it holds one of the first P
// tickets) will publish. No workgroup needs another to be resident. Every
// wait also gives up after `spin` polls (setting ctl[kCtlError]), so a run
// can never hang.
//
// Coherence across the XCDs' L2 caches: what one workgroup writes for another
// (a tile's slots and run table, a range's counts) is written with
// device-scope stores and read with device-scope loads (sc1), never plain
// ones, and no 128-byte line holds data of two sub-tiles (run-table rows and
// stage areas are whole lines). A hand-over is then: wait until this wave's
// stores have completed (they are visible device-wide once they have), then
// store the flag at device scope; the reader polls at device scope and
// acquires. No L2 writeback (buffer_wbl2) is needed, which a
// release at agent scope would issue once per tile: with thousands of tiles
// those writebacks of whole L2s were the path's bottleneck.
//
// Workspace, zeroed by k_stream_prepare at the start of every run:
//   ctl[0..63]: ticket, tile counter, error, stint counter, move counter;
//   claim[R], flag[T]. Then the pool's slots (S counters each) and the
//   range of each slot, which need no clearing.
// Each workgroup also leaves a timeline of its run, kStreamTraceWords words
// at trace[ticket * kStreamTraceWords] (times in ticks of the 100 MHz
// constant clock, low 32 bits): the StreamTrace fields below.
constexpr uint32_t kCtlTicket = 0, kCtlTile = 1, kCtlError = 2, kCtlSlots = 3, kCtlMoves = 4, kCtlWords = 64;
enum StreamTrace : uint32_t {
    kTrTicket = 0, kTrStart, kTrProduced, kTrEnd, kTrTiles, kTrBlocks, kTrStints,
    kTrFlagWait, kTrMovesDenied, kTrStintWrite, kTrCount, kTrScans, kStreamTraceWords = 16
};
constexpr uint32_t kStreamShWords = 8 + kStreamTraceWords;  // LDS words after the shared area
// the slot value that pads a run (slots hold bin & (S - 1) < S)
constexpr uint16_t kStreamPad = 0xFFFFu;
__device__ __forceinline__ uint32_t ceil_div_u(uint32_t a, uint32_t b) { return (a + b - 1u) / b; }
// A producer wave's sub-tile: kStreamLaneVecs vectors per lane, a tile
// (4,096 vectors, 16,384 elements) in kStreamSubsPerTile of them. Its stage
// area holds its elements, a head or tail of up to 3 + 3 elements and up to 7
// padding slots for each of up to 64 ranges, in whole 256-byte units, and is
// copied out as at most kStreamSubChunksPerLane chunks of 16 bytes per lane.
// The workgroup size goes with it: a lane holds two sub-tiles' elements and
// their positions in registers, which 8 vectors per lane fit only with
// 256-VGPR waves (512 threads), 4 with 128-VGPR waves (1,024 threads).
constexpr uint32_t kStreamLaneVecs = 8;
constexpr uint32_t kStreamWG = kStreamLaneVecs > 4 ? 512 : 1024;
constexpr uint32_t kStreamLaneElems = 4 * kStreamLaneVecs + 1;
constexpr uint32_t kStreamSubVecs = 64 * kStreamLaneVecs;
constexpr uint32_t kStreamTileVecs = 4096, kStreamSubsPerTile = kStreamTileVecs / kStreamSubVecs;
constexpr uint32_t kStreamSubCap = (4 * kStreamSubVecs + 8 + 7 * 64 + 127) / 128 * 128;
constexpr uint32_t kStreamSubChunksPerLane = (kStreamSubCap / 8 + 63) / 64;
// per producer wave, in LDS: counters [65][4] (ranges 0..63, and 64 for the
// elements to drop), their bases (range 64's all the trash slot), the
// staged slots (whose last slot takes the dropped elements: a sub-tile
// stages at most 4 kStreamSubVecs + 3 + 7 x 64 slots). A counter ranks at
// most 16 lanes x kStreamLaneElems elements, so a rank fits 10 bits.
constexpr uint32_t kStreamWaveCnt = 260;
constexpr uint32_t kStreamWaveWords = 2 * kStreamWaveCnt + kStreamSubCap / 2;
constexpr uint32_t kStreamTrashSlot = kStreamSubCap - 1;
static_assert(16 * kStreamLaneElems < 1024, "ranks must fit 10 bits");
static_assert(4 * kStreamSubVecs + 3 + 7 * 64 < kStreamTrashSlot, "the trash slot must stay unused");
// owner runs per lane in a set (each one 16-byte chunk load per pass); two
// sets in flight take 2 x 6 U VGPRs
constexpr uint32_t kStreamOwnerU = kStreamWG == 512 ? 8 : 4;
constexpr uint32_t kStreamDropRange = 64;

struct StreamArgs {
    InputView in;
    uint32_t num_bins, ranges, tiles;
    uint32_t bt;       // tiles per owner block
    uint32_t nblocks;  // blocks per range = ceil(tiles / bt)
    uint32_t producers;
    uint32_t spin;     // polls a wait makes before it gives up
    uint32_t uwords;   // LDS words shared by the producer's and the owner's state
    uint32_t rstride;  // words per run-table row (ranges, padded to 32)
    uint32_t *ctl;     // control words, then claim[R], flag[T]
    uint32_t *pool;    // [pool_slots][S] stints' counts
    uint32_t *slot_range;  // [pool_slots] the range of each written slot
    uint32_t pool_slots, move_budget;
    uint32_t *rows;    // [tiles * kStreamSubsPerTile][rstride] per range: start << 16 | length
    uint16_t *stage;   // [tiles * kStreamSubsPerTile][kStreamSubCap] slots grouped by range
    uint32_t *counts;
    uint32_t accumulate;
    uint32_t *trace;  // [workgroups][kStreamTraceWords]
};

__global__ void k_stream_prepare(uint32_t *__restrict__ ctl, uint32_t words)
{
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < words; i += gridDim.x * blockDim.x)
        ctl[i] = 0u;
}

__device__ __forceinline__ uint32_t dev_load(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16 bytes at byte offset `off` of a buffer, loaded at device scope (sc1);
// offsets at or past the buffer's size read as zero.
constexpr int kCpolDevice = 16;
__device__ __forceinline__ u32x4 dev_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolDevice));
}
constexpr uint32_t kRawBufferWord3 = 0x00020000u;  // raw (unformatted, unswizzled) buffer

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, kRawBufferWord3);
}

// Orders this wave's LDS accesses on either side (no instruction: a wave's
// LDS operations execute in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_order() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// Waits until every memory operation this wave issued has completed (stores
// included: on gfx9 they count in vmcnt); the compiler keeps memory
// operations on their side of it.
__device__ __forceinline__ void wait_memory()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ void dev_store(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Vectors of tile t in the body (kStreamTileVecs but for the last tile).
__device__ __forceinline__ uint32_t tile_vecs(const StreamArgs &a, uint32_t t)
{
    const uint64_t v0 = (uint64_t)t * kStreamTileVecs;
    const uint64_t left = a.in.nvec > v0 ? a.in.nvec - v0 : 0;
    return (uint32_t)(left < kStreamTileVecs ? left : kStreamTileVecs);
}

// One producer wave's sub-tile `sub` of tile t into w[0..31] (vector u of the
// lane in w[4u..4u+3]; vectors past the body read as zero, which the ranking
// step drops by index, so that no use follows a load at once) and w[32], the
// head (tile 0, sub-tile 0) or tail (last tile, last sub-tile) element of
// the first lanes, else -1.
__device__ __forceinline__ void load_sub(uint32_t (&w)[kStreamLaneElems], const StreamArgs &a, uint32_t t,
                                         uint32_t sub, uint32_t lane, int32_t head_x, int32_t tail_x)
{
    const __amdgpu_buffer_rsrc_t r =
        buffer_of(a.in.ptr + a.in.head + (uint64_t)t * kStreamTileVecs * 4, tile_vecs(a, t) * 16u);
#pragma unroll
    for (uint32_t u = 0; u < kStreamLaneVecs; ++u) {
        const u32x4 q = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (sub * kStreamSubVecs + u * 64 + lane) * 16, 0, 0));
        w[4 * u + 0] = q.x;
        w[4 * u + 1] = q.y;
        w[4 * u + 2] = q.z;
        w[4 * u + 3] = q.w;
    }
    w[kStreamLaneElems - 1] = (uint32_t)((t == 0 && sub == 0) ? head_x
                       : (t == a.tiles - 1 && sub == kStreamSubsPerTile - 1) ? tail_x : -1);
}


template <int WG>
__global__ __launch_bounds__(WG) void k_stream(StreamArgs a)
{
    constexpr uint32_t S = 32768;  // bins an owner holds
    extern __shared__ u32x4 smem4[];
    uint32_t *const slice = reinterpret_cast<uint32_t *>(smem4);  // owner: S counters
    uint32_t *const sh = slice + a.uwords;  // broadcast words (past the owner's S + 64 trash words)
    uint32_t *const tr = sh + 8;            // this workgroup's timeline (thread 0)
    auto now = []() { return (uint32_t)wall_clock64(); };
    const uint32_t tid = threadIdx.x, lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t R = a.ranges, T = a.tiles;
    uint32_t *const claim = a.ctl + kCtlWords;
    uint32_t *const flag = claim + R;

    if (tid == 0) {
        sh[0] = __hip_atomic_fetch_add(a.ctl + kCtlTicket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (uint32_t k = 0; k < kStreamTraceWords; ++k) tr[k] = 0u;
        tr[kTrTicket] = sh[0];
        tr[kTrStart] = now();
    }
    __syncthreads();
    const uint32_t ticket = sh[0];

    if (ticket < a.producers) {
        // ---- producer: every wave on its own ----
        uint32_t *const wcnt = slice + wave * kStreamWaveWords;  // [range][4] counters
        uint32_t *const wbase = wcnt + kStreamWaveCnt;            // their run positions
        uint16_t *const wst = reinterpret_cast<uint16_t *>(wbase + kStreamWaveCnt);
        const uint32_t q = lane & 3u;
        reinterpret_cast<u32x4 *>(wcnt)[lane] = u32x4{0, 0, 0, 0};
        if (lane == 0) {
            reinterpret_cast<u32x4 *>(wcnt)[64] = u32x4{0, 0, 0, 0};
            reinterpret_cast<u32x4 *>(wbase)[64] =
                u32x4{kStreamTrashSlot, kStreamTrashSlot, kStreamTrashSlot, kStreamTrashSlot};
        }
        const int32_t head_x = lane < a.in.head ? a.in.ptr[lane] : -1;
        const int32_t tail_x = lane < a.in.tail ? a.in.ptr[a.in.head + 4 * a.in.nvec + lane] : -1;
        auto claim_issue = [&]() {
            uint32_t c = 0;
            if (lane == 0)
                c = __hip_atomic_fetch_add(a.ctl + kCtlTile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return c;  // lane 0's
        };
        // Route sub-tile `sub` of tile t, held in cur, after sending out the
        // loads of the one after it (sub + 1 of t, or the first of tile tn,
        // which reads as empty past the last tile) into nxt.
        auto route = [&](uint32_t (&cur)[kStreamLaneElems], uint32_t (&nxt)[kStreamLaneElems], uint32_t t,
                         uint32_t sub, uint32_t tn,
                         uint32_t nv) {
            const bool last = sub + 1 == kStreamSubsPerTile;
            load_sub(nxt, a, last ? tn : t, last ? 0u : sub + 1, lane, head_x, tail_x);
            // rank each element within its range's counter q and pack range
            // (bits 25..31; kStreamDropRange for an element outside the bins
            // or past the body), rank (15..24) and slot (0..14) into one
            // word. No branch, so that the atomics go out back to back.
#pragma unroll
            for (uint32_t k = 0; k < kStreamLaneElems; ++k) {
                const uint32_t x = cur[k];
                const bool ok = (k == kStreamLaneElems - 1 || sub * kStreamSubVecs + (k >> 2) * 64 + lane < nv) &&
                                x < a.num_bins;
                const uint32_t r = ok ? x >> 15 : kStreamDropRange;
                const uint32_t rk = lds_add_rtn(wcnt, (r << 2) | q, 1u);
                cur[k] = (r << 25) | ((rk & 1023u) << 15) | (x & (S - 1u));
            }
            wave_lds_order();
            // lane r lays out range r's run: start, the four counters'
            // positions, padding slots; row word start << 16 | length
            const u32x4 c4 = reinterpret_cast<const u32x4 *>(wcnt)[lane];
            const uint32_t len = c4.x + c4.y + c4.z + c4.w;
            const uint32_t pad = (8u - (len & 7u)) & 7u;
            const uint32_t incl = wave_inclusive_scan(len + pad);
            const uint32_t start = incl - len - pad;
            reinterpret_cast<u32x4 *>(wbase)[lane] =
                u32x4{start, start + c4.x, start + c4.x + c4.y, start + c4.x + c4.y + c4.z};
            reinterpret_cast<u32x4 *>(wcnt)[lane] = u32x4{0, 0, 0, 0};
            for (uint32_t k = 0; k < pad; ++k) wst[start + len + k] = kStreamPad;
            const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
            const uint64_t sub_id = (uint64_t)t * kStreamSubsPerTile + sub;
            if (lane < R) dev_store(a.rows + sub_id * a.rstride + lane, (start << 16) | len);
            wave_lds_order();
            // every position first, then every slot: the reads of the bases
            // and the writes of the slots each go out back to back (a dropped
            // element's base is the trash slot, so min() keeps it there)
            uint32_t pos[kStreamLaneElems];
#pragma unroll
            for (uint32_t k = 0; k < kStreamLaneElems; ++k) {
                const uint32_t e = cur[k];
                pos[k] = min(wbase[((e >> 25) << 2) | q] + ((e >> 15) & 1023u), kStreamTrashSlot);
            }
#pragma unroll
            for (uint32_t k = 0; k < kStreamLaneElems; ++k) wst[pos[k]] = (uint16_t)(cur[k] & (S - 1u));
            wave_lds_order();
            // copy the staged slots out: chunks past the total are dropped
            const __amdgpu_buffer_rsrc_t out = buffer_of(a.stage + sub_id * kStreamSubCap, total * 2);
#pragma unroll
            for (uint32_t c = 0; c < kStreamSubChunksPerLane; ++c) {
                const uint32_t ch = lane + 64 * c;
                const u32x4 v = reinterpret_cast<const u32x4 *>(wst)[ch];
                __builtin_amdgcn_raw_buffer_store_b128(v, out, ch * 16, 0, kCpolDevice);
            }
            wave_lds_order();
        };
        uint32_t t = __builtin_amdgcn_readfirstlane(claim_issue());
        uint32_t ea[kStreamLaneElems], eb[kStreamLaneElems];
        load_sub(ea, a, t, 0, lane, head_x, tail_x);  // reads as empty when t >= T
        while (t < T) {
            // sub-tiles in pairs, ea and eb taking turns; the next tile is
            // claimed two sub-tiles before its first loads go out. Tile
            // numbers stay wave-uniform (readfirstlane), so that the buffer
            // descriptors built from them are scalar.
            const uint32_t nv = tile_vecs(a, t);
            uint32_t tn = T;
            for (uint32_t sub = 0; sub < kStreamSubsPerTile; sub += 2) {
                uint32_t claimed = 0;
                if (sub == kStreamSubsPerTile - 2) claimed = claim_issue();
                route(ea, eb, t, sub, T, nv);
                if (sub == kStreamSubsPerTile - 2) tn = __builtin_amdgcn_readfirstlane(claimed);
                route(eb, ea, t, sub + 1, tn, nv);
            }
            // publish: once this wave's device-scope stores have completed
            wait_memory();
            if (lane == 0) {
                dev_store(flag + t, 1u);
                __hip_atomic_fetch_add(tr + kTrTiles, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            t = __builtin_amdgcn_readfirstlane(tn);
        }
        __syncthreads();  // the shared words become the owner's slice
        if (tid == 0) tr[kTrProduced] = now();
    }

    // ---- owner ----
    HotSlot hs;  // per wave, kept across blocks (its count is added at each block's end)
    uint32_t cur = ticket % R;
    bool have = false;  // the slice holds counts of a stint on cur
    for (uint32_t i = tid; i < S; i += WG) slice[i] = 0u;
    __syncthreads();
    for (;;) {
        if (tid == 0)
            sh[2] = __hip_atomic_fetch_add(claim + cur, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const uint32_t b = sh[2];
        if (b < a.nblocks) {
            const uint32_t t0 = b * a.bt, t1 = min(t0 + a.bt, T), nt = t1 - t0;
            if (wave == 0) {
                // wait for the block's tiles, 64 flags per poll, then acquire
                // what their producers wrote
                const uint32_t w0 = now();
                uint32_t spins = 0;
                bool ok = true;
                for (uint32_t k = 0; k < nt && ok; k += 64) {
                    const uint32_t t = t0 + k + lane;
                    while (!__all(t >= t1 || dev_load(flag + t) != 0u)) {
                        if (++spins > a.spin) {
                            ok = false;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
                if (!ok && lane == 0)
                    __hip_atomic_store(a.ctl + kCtlError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                // lanes per run for this block: the next power of two at or
                // above the mean chunks per run of range cur in 16 sampled
                // sub-tiles (runs of a heavy range are longer than the mean
                // over the ranges)
                const uint32_t nsub_b = nt * kStreamSubsPerTile;
                uint32_t nch = 0;
                if (ok && lane < 16) {
                    const uint64_t js = (uint64_t)t0 * kStreamSubsPerTile + (uint64_t)lane * nsub_b / 16;
                    nch = ((dev_load(a.rows + js * a.rstride + cur) & 0xFFFFu) + 7u) >> 3;
                }
                const uint32_t mean = (wave_sum(nch) + 15u) / 16u;
                uint32_t glog = 0;
                while (glog < 6 && (1u << glog) < mean) ++glog;
                if (lane == 0) {
                    sh[3] = ok;
                    sh[5] = glog;
                    const uint32_t w1 = now();
                    tr[kTrFlagWait] += w1 - w0;
                    tr[kTrCount] -= w1;  // plus the time after the block's closing barrier
                    ++tr[kTrBlocks];
                }
            }
            __syncthreads();
            if (sh[3]) {
                // G = 1 << glog lanes share a run (about one 16-byte chunk per
                // lane), so that one load instruction reads whole runs; each
                // lane carries U runs: in set k of wave w, group gi's u-th run
                // is that of sub-tile (w + NW k) U NG + gi + NG u (NG = 64 / G
                // groups), its lane gl taking chunks gl, gl + G, ... One pass
                // per set covers runs of up to G chunks; longer ones take more.
                // Two sets take turns in registers: the next set's row words
                // and first pass are in flight while one is counted.
                constexpr uint32_t U = kStreamOwnerU, NW = WG / 64;
                const uint32_t glog = sh[5], G = 1u << glog, gl = lane & (G - 1u), gi = lane >> glog;
                const uint32_t NG = 64u >> glog, per = NG * U, nsub = nt * kStreamSubsPerTile;
                const uint64_t sub0 = (uint64_t)t0 * kStreamSubsPerTile;
                const __amdgpu_buffer_rsrc_t rs =
                    buffer_of(a.stage + sub0 * kStreamSubCap, nsub * kStreamSubCap * 2);
                const uint32_t *const rowb = a.rows + sub0 * a.rstride + cur;
                auto rows = [&](uint32_t (&pk)[U], uint32_t k) {
                    const uint32_t j0 = (wave + NW * k) * per + gi;
#pragma unroll
                    for (uint32_t u = 0; u < U; ++u) {
                        const uint32_t j = j0 + NG * u;
                        pk[u] = j < nsub ? dev_load(rowb + (uint64_t)j * a.rstride) : 0u;
                    }
                };
                // a set in flight: its runs' chunk counts and byte offsets
                // (this lane's first chunk), and the first pass's chunks
                struct Set {
                    u32x4 v[U];
                    uint32_t nch[U], off[U];
                };
                auto load_pass = [&](Set &st, uint32_t pass) {
#pragma unroll
                    for (uint32_t u = 0; u < U; ++u) {
                        const uint32_t c = gl + G * pass;
                        st.v[u] = c < st.nch[u] ? dev_load16(rs, st.off[u] + G * pass * 16)
                                                : u32x4{~0u, ~0u, ~0u, ~0u};
                    }
                };
                auto start = [&](Set &st, const uint32_t (&pk)[U], uint32_t k) {
                    const uint32_t j0 = (wave + NW * k) * per + gi;
#pragma unroll
                    for (uint32_t u = 0; u < U; ++u) {
                        st.nch[u] = ((pk[u] & 0xFFFFu) + 7u) >> 3;
                        st.off[u] = ((j0 + NG * u) * kStreamSubCap + (pk[u] >> 16)) * 2 + gl * 16;
                    }
                    load_pass(st, 0);
                };
                // a hot slot (a bin holding many lanes of a wave) is counted in
                // registers and added once per switch (HotSlot), as the
                // two-phase path's owners do. Every other slot is one LDS add
                // with no branch: a padding slot (>= S) or a hot one adds into
                // the lane's own word past the slice, so that nothing waits
                // on an exec-mask change (with two waves per SIMD, those
                // dependencies were what bound the loop)
                auto count = [&](const u32x4 (&v)[U]) {
#pragma unroll
                    for (uint32_t u = 0; u < U; ++u) {
                        const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                        uint32_t nxt;
                        if (hot_should_switch(hs, w4[0] & 0xFFFFu, (w4[0] & 0xFFFFu) < S, &nxt)) {
                            const uint32_t tk = hot_take(hs);
                            if (lane == 0 && tk != 0u) lds_add(slice, hs.h, tk);
                            hs.h = nxt;
                        }
                        const uint32_t h = (uint32_t)__builtin_amdgcn_readfirstlane((int)hs.h);
#pragma unroll
                        for (uint32_t e = 0; e < 8; ++e) {
                            const uint32_t slot = (w4[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                            const bool m = slot == h;
                            hs.c += m ? 1u : 0u;
                            lds_add(slice, slot < S && !m ? slot : S + lane, 1u);
                        }
                    }
                };
                // count a set: its first pass, then the passes of runs longer than G chunks
                auto finish = [&](Set &st) {
                    count(st.v);
                    uint32_t most = 0;
#pragma unroll
                    for (uint32_t u = 0; u < U; ++u) most = max(most, st.nch[u]);
                    for (uint32_t pass = 1; __any(gl + G * pass < most); ++pass) {
                        load_pass(st, pass);
                        count(st.v);
                    }
                };
                // sets k and k + 1 take turns in sa and sb; the row words of the
                // set after next load while one set is counted
                const uint32_t sets = ceil_div_u(nsub, per);  // sets over the workgroup
                Set sa, sb;
                uint32_t pr[U];
                uint32_t k = 0;
                rows(pr, k);
                start(sa, pr, k);
                rows(pr, k + 1);
                for (; wave + NW * k < sets; k += 2) {
                    start(sb, pr, k + 1);
                    rows(pr, k + 2);
                    finish(sa);
                    if (wave + NW * (k + 1) >= sets) break;
                    start(sa, pr, k + 2);
                    rows(pr, k + 3);
                    finish(sb);
                }
                const uint32_t tk = hot_take(hs);
                if (lane == 0 && tk != 0u) lds_add(slice, hs.h, tk);
            }
            have = true;
            __syncthreads();
            if (tid == 0) tr[kTrCount] += now();
            continue;
        }
        // cur has no block left: write the stint's counts to the next pool slot
        if (have) {
            if (tid == 0) {
                sh[4] = __hip_atomic_fetch_add(a.ctl + kCtlSlots, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                tr[kTrStintWrite] -= now();
            }
            __syncthreads();
            const uint32_t slot = sh[4];
            if (slot < a.pool_slots) {  // always, by the move budget
                u32x4 *dst = reinterpret_cast<u32x4 *>(a.pool + (uint64_t)slot * S);
                const u32x4 *src = reinterpret_cast<const u32x4 *>(slice);
                for (uint32_t i = tid; i < S / 4; i += WG) dst[i] = src[i];
                if (tid == 0) a.slot_range[slot] = cur;
            } else if (tid == 0) {
                __hip_atomic_store(a.ctl + kCtlError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
            for (uint32_t i = tid; i < S; i += WG) slice[i] = 0u;
            have = false;
            if (tid == 0) {
                tr[kTrStintWrite] += now();
                ++tr[kTrStints];
            }
        }
        // the range with the most blocks left, if any, and a move from the budget
        if (tid == 0) {
            uint32_t best = R, left = 0;
            for (uint32_t r = 0; r < R; ++r) {
                const uint32_t c = dev_load(claim + r);
                if (c < a.nblocks && a.nblocks - c > left) {
                    left = a.nblocks - c;
                    best = r;
                }
            }
            if (best < R &&
                __hip_atomic_fetch_add(a.ctl + kCtlMoves, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
                    a.move_budget) {
                best = R;
                ++tr[kTrMovesDenied];
            }
            sh[6] = best;
            ++tr[kTrScans];
        }
        __syncthreads();
        const uint32_t nxt = sh[6];
        __syncthreads();
        if (nxt >= R) break;
        cur = nxt;
    }
    if (tid == 0) {
        tr[kTrEnd] = now();
        for (uint32_t k = 0; k < kStreamTraceWords; ++k) a.trace[ticket * kStreamTraceWords + k] = tr[k];
    }
}

// Adds each range's stints into the output: workgroup (r, part) sums the
// pool slots recorded for range r over its kMergeBins bins, then writes the
// sum, or adds it when accumulating. used = the stint counter (slots past
// pool_slots were never written).
constexpr uint32_t kStreamMergeBins = 1024;
template <int WG>
__global__ __launch_bounds__(WG) void k_stream_merge(const uint32_t *__restrict__ ctl,
                                                    const uint32_t *__restrict__ pool,
                                                    const uint32_t *__restrict__ slot_range,
                                                    uint32_t pool_slots, uint32_t num_bins,
                                                    uint32_t *__restrict__ counts, uint32_t accumulate)
{
    constexpr uint32_t S = 32768, PER = kStreamMergeBins / WG;
    constexpr uint32_t parts = S / kStreamMergeBins;
    const uint32_t r = blockIdx.x / parts, part = blockIdx.x % parts;
    const uint32_t used = min(ctl[kCtlSlots], pool_slots);
    const uint32_t b0 = r * S + part * kStreamMergeBins;
    uint32_t acc[PER];
#pragma unroll
    for (uint32_t k = 0; k < PER; ++k) acc[k] = 0u;
    for (uint32_t s = 0; s < used; ++s) {
        if (slot_range[s] != r) continue;
        const uint32_t *src = pool + (uint64_t)s * S + part * kStreamMergeBins;
#pragma unroll
        for (uint32_t k = 0; k < PER; ++k) acc[k] += src[k * WG + threadIdx.x];
    }
#pragma unroll
    for (uint32_t k = 0; k < PER; ++k) {
        const uint32_t b = b0 + k * WG + threadIdx.x;
        if (b < num_bins) counts[b] = accumulate ? counts[b] + acc[k] : acc[k];
    }
}

}  // namespace pca
