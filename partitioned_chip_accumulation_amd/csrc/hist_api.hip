// hist_api.hip -- host side of libpca_hist.so: plans, argument checks and
// kernel launches for the partitioned LDS histogram (declared in hist.h).
//
// Path choice follows the page "Distributed Shared Memory": when the bins fit
// one workgroup's on-chip memory every workgroup privatises all of them
// (FULL); when they do not, the bins are partitioned so that each workgroup
// owns a slice (section "The cluster histogram") -- on gfx950 by bin-range
// ownership (RANGE) or, when the ranges get many, by routing elements to
// their owners first (SCATTER). Section "When it beats global atomics" gives
// the capacity argument: R cooperating workgroups hold R slices on-chip.
#include "hist.h"

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "hist_host.hpp"
#include "hist_kernels.hpp"

namespace {

constexpr uint32_t kMaxLdsBins = 40960;      // 160 KiB of uint32 counters
constexpr uint32_t kMaxLdsBins16 = 79616;    // 16-bit counters + the carry-event list
constexpr uint64_t kMaxElemsPerWG16 = 1ull << 24;  // bounds the carry-event list
constexpr uint32_t kMaxLdsBins8 = 155392;    // 8-bit counters + the shortest carry-event list
constexpr uint32_t kScatterShift = 15;
constexpr uint32_t S_STREAM = 1u << kScatterShift;       // SCATTER range = 32768 bins (128 KiB)
// From this many ranges the partition writes its run tables tile-major and a
// transpose makes them range-major. Range-major stores from a tile land a row
// apart: at 2,048 ranges (2^26 bins) the partition wrote 827 MiB for 192 MiB
// of slots and tables. Measured on 2^26 uniform elements, tile-major against
// range-major: 2^26 bins 567 vs 672 us, 2^25 360 vs 404, 2^24 263.3 vs 262.2
// (the transpose's cost equals the partition's saving there).
constexpr uint32_t kTileMajorRanges = 1024;
constexpr uint32_t kScatterWG = 1024;        // the owners' workgroup
// The one-pass range scan up to this many ranges (each one workgroup); at
// 2,048 ranges of 4,096 tiles the two passes were faster (61 against 69 us).
constexpr uint32_t kRangeScanMaxRanges = 256;
// The MI355X's Infinity Cache (the memory-side cache in front of HBM). Data
// read once is loaded or stored non-temporally only when it outgrows it;
// smaller buffers stay cacheable, so that their later readers can find them
// there. Measured on the two-phase path's staged slots (2 bytes per element):
// non-temporal stores and loads took the hot-bin 2^20-bin workload (2^28
// elements) from 446 to 430 us and the half-Gaussian one (2^29) from 673 to
// 655 us, but 2^22 uniform bins at 2^26 elements from 199 to 247 us. On the
// RANGE sweep's input with R > 1 owners plain loads took the Zipf 2^18-bin
// workload (1 GiB) from 381-384 to 374-376 us but 2^18 uniform bins at 2^26
// elements (256 MiB) from 63 to 68 us.
constexpr uint64_t kMallBytes = 256ull << 20;
constexpr uint32_t kPartWG = 1024;           // the partition's workgroup
// The partition's persistent grid, per CU: at its register count one
// 1024-thread workgroup is resident per CU, and a second one per CU would
// start cold after the first (on 2^26 uniform elements over 2^20 bins the
// partition took 92 us with one per CU against 98 with two).
constexpr uint32_t kPartPerCU = 1;
constexpr uint32_t kScatterVPT = 4;          // vectors per thread in a scatter tile
constexpr uint32_t kScatterTile = kPartWG * kScatterVPT * 4;  // 16384 elements
constexpr uint32_t kScatterCap = kScatterTile + 8;               // staging slots per tile
// AUTO uses RANGE up to this many 16-bit ranges' worth of bins (318,464) and
// SCATTER beyond: on 2^26 uniform elements SCATTER wins from 2^19 bins on
// (141 us against 220 with 16-bit and 111 with 8-bit counters, the latter
// at 1,528 us against 912 on the half-Gaussian 512K-bin workload).
constexpr uint32_t kRangeMaxR = 4;
// SCATTER's in-place window: AUTO samples for it from this many elements on,
// and uses it when it holds at least 1 / kWindowMinShare of the sample. On
// the half-Gaussian 512K-bin workload an 8,192-bin window holds 51% of the
// input, and the owners' time halves (2^29 elements: 896 -> 794 us end to
// end). A window that is heavy because of one hot bin does not pay: the
// owners' hot slot already takes that bin in registers, while in the
// partition its adds pile onto one LDS word (the hot-bin workload's window
// holds 11%: 472 -> 576 us), hence a quarter.
constexpr uint64_t kWindowMinElems = 1ull << 22;
constexpr uint32_t kWindowMinShare = 4;
// STREAM: at most this many ranges (an owner scans them all when it moves);
// blocks of 8 tiles per range (about 8 x 16,384 elements of a range when the
// ranges are even), 16 to 256 tiles, per owner claim; and the polls a wait
// makes before it gives up (2^22: seconds).
constexpr uint32_t kStreamMaxRanges = 64;
constexpr uint32_t kStreamMinBlockTiles = 16, kStreamMaxBlockTiles = 256;
constexpr uint32_t kStreamSpinLog2 = 22;
// STREAM: threads per workgroup, set by the sub-tile a producer wave holds in
// registers; one workgroup fits a CU (the owner's slice takes 128 KiB of LDS)
constexpr uint32_t kStreamWG = pca::kStreamWG;
// STREAM: moves an owner may make to another range, over all workgroups, per
// workgroup (the stint pool holds workgroups x (1 + this) slots at most)
constexpr uint32_t kStreamMovesPerWG = 3;
constexpr uint32_t kMinElemsPerGroup = 4096;
constexpr int kMaxWavesPerCU = 32;

enum Phase { PH_SWEEP = 0, PH_MERGE = 1, PH_PART = 2, PH_SCAN = 3, PH_OWNER = 4, PH_SLOTS = 5,
             PH_STREAM = 6 };
const char *kPhaseNames[HIST_MAX_PHASES] = {"sweep", "merge", "partition", "range_scan",
                                            "owner_hist", "slot_merge", "stream"};

uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// Workspace bytes of `rows` partial rows of nblk blocks: plane 0, planes 1..7
// and the width codes, each region 256-byte aligned.
uint64_t partial_bytes(uint32_t rows, uint32_t nblk)
{
    const uint64_t cells = (uint64_t)rows * nblk;
    return align_up(cells * pca::kPlaneBytes, 256) +
           align_up(cells * pca::kPlaneBytes * pca::kUpperPlanes, 256) + align_up(cells, 256);
}
uint32_t ceil_div(uint64_t a, uint64_t b) { return (uint32_t)((a + b - 1) / b); }

// LDS bytes of a sweep workgroup: a slice of S bins in cw-bit counters (with
// 2^kshift copies of 32-bit ones), plus the carry-event count and list of
// the packed widths (ev_cap entries for 8-bit counters).
uint32_t sweep_lds_bytes(uint32_t cw, uint32_t S, uint32_t kshift, uint32_t ev_cap)
{
    if (cw == 32) return (S << kshift) * 4;
    if (cw == 16) return S * 2 + (4 + pca::kEventCap) * 4;
    return S + (4 + ev_cap) * 4;
}

struct DeviceInfo {
    int device = -1;
    int cu = 0;
    int xcd = 1;
    uint32_t lds = 0;  // bytes per workgroup
    // sweep waves a SIMD holds at once as far as registers allow: 0 = ask the
    // runtime for the kernel that will run, ~0u = no register limit
    uint32_t sweep_waves_per_simd = 0;
};

hist_status_t query_device(DeviceInfo *d)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return HIST_ERR_UNSUPPORTED;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return HIST_ERR_UNSUPPORTED;
    }
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return HIST_ERR_UNSUPPORTED;
    int lds = 0;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) {
        (void)hipGetLastError();
        return HIST_ERR_UNSUPPORTED;
    }
    d->device = dev;
    d->cu = prop.multiProcessorCount;
    d->xcd = std::max(1, d->cu / 32);  // gfx950: 32 CUs per XCD
    d->lds = (uint32_t)std::min<int>(lds, 163840);
    return HIST_OK;
}

}  // namespace

struct hist_plan_impl {
    DeviceInfo dev;
    uint32_t num_bins = 0;
    uint64_t max_n = 0;
    int path = 0;
    int agg = 0;
    uint32_t wg = 0;
    uint32_t xcd_map = 1;
    // FULL / RANGE
    uint32_t range_bins = 0, ranges = 0, groups = 0;
    uint32_t cw = 32;    // LDS counter bits
    uint32_t kshift = 0; // 2^kshift interleaved LDS copies (32-bit counters)
    uint32_t ev_cap = 0; // carry-event list entries (8-bit counters)
    uint32_t pacing = 1; // RANGE: 1 own pace, 2 own pace with a pacer wave, >= 3 paced (window - 2)
    uint64_t off_progress = 0;  // RANGE paced: [G][R][16] progress words
    uint64_t off_spill = 0;     // 8-bit counters: [G R][kEvSpill8] carry events past the LDS list
    uint64_t max_elems_wg = 1ull << 40;  // elements one sweep workgroup may count
    uint32_t nblk = 0;       // 256-bin blocks per partial row
    uint32_t part_rows = 0;  // partial rows the workspace holds
    // SCATTER (and STREAM: tiles, qlog)
    uint32_t tiles = 0, owners = 0, qlog = 0;
    // STREAM
    uint32_t producers = 0, bt = 0, spin = 0, uwords = 0, grid = 0, rstride = 0;
    uint32_t pool_slots = 0, move_budget = 0;
    // SCATTER's in-place window: mode (0 auto, 1 never, 2 always), width, the
    // chosen base word and the partition workgroups' rows
    uint32_t window = 1, wbins = 0, wrows = 0;
    uint64_t off_wsel = 0, off_wpart = 0;
    uint64_t off_pool = 0, off_slot_range = 0;
    uint64_t off_ctl = 0, off_trace = 0;
    // workspace
    char *ws = nullptr;
    uint64_t ws_bytes = 0, need = 0;
    uint64_t off_partials = 0, off_stage = 0, off_tcnt = 0, off_tbase = 0, off_tpre = 0,
             off_totals = 0, off_segtot = 0, off_starts = 0, off_tbase_tm = 0;
    bool tile_major = false;  // SCATTER: run tables written tile-major, then transposed
    // timing
    uint32_t tcap = 0, truns = 0;
    std::vector<hipEvent_t> ev;  // [tcap][HIST_MAX_PHASES][2]
    std::vector<uint8_t> used;   // [tcap][HIST_MAX_PHASES]
};

namespace {

hist_status_t check_opts(const hist_plan_opts_t *o)
{
    if (!o) return HIST_OK;
    if (o->path < 0 || o->path > 4) return HIST_ERR_INVALID_ARG;
    if (o->spin_log2 < 0 || o->spin_log2 > 30) return HIST_ERR_INVALID_ARG;
    if (o->window < 0 || o->window > 2) return HIST_ERR_INVALID_ARG;
    if (o->groups < 0 || o->groups > 65536) return HIST_ERR_INVALID_ARG;
    if (o->range_bins < 0 || (o->range_bins % 256) != 0 || o->range_bins > (int)kMaxLdsBins8)
        return HIST_ERR_INVALID_ARG;
    if (o->counter_bits != 0 && o->counter_bits != 8 && o->counter_bits != 16 &&
        o->counter_bits != 32)
        return HIST_ERR_INVALID_ARG;
    if (o->aggregation < -1 || o->aggregation > 4 || o->aggregation == 3) return HIST_ERR_INVALID_ARG;
    if (o->wg_size != 0 && o->wg_size != 256 && o->wg_size != 512 && o->wg_size != 1024)
        return HIST_ERR_INVALID_ARG;
    if (o->xcd_map < 0 || o->xcd_map > 2) return HIST_ERR_INVALID_ARG;
    if (o->lds_copies < 0 || o->lds_copies > 16 || (o->lds_copies & (o->lds_copies - 1)) != 0)
        return HIST_ERR_INVALID_ARG;
    if (o->pacing < 0 || o->pacing > 18) return HIST_ERR_INVALID_ARG;
    return HIST_OK;
}

// Sweep workgroups of this configuration one CU holds at once (0 if the
// runtime cannot tell); defined with the launch code below.
uint32_t sweep_resident(uint32_t cw, uint32_t wg, int agg, uint32_t lds_bytes);

// Fill every plan field that depends only on (num_bins, max_n, opts, device).
hist_status_t design(hist_plan_impl *p, uint32_t num_bins, uint64_t max_n, const hist_plan_opts_t *o)
{
    hist_plan_opts_t opts{};
    opts.aggregation = -1;
    if (o) opts = *o;
    const DeviceInfo &d = p->dev;
    const uint32_t lds_dyn = d.lds;
    const uint32_t lds_bins = std::min<uint32_t>(kMaxLdsBins, lds_dyn / 4) & ~3u;
    p->num_bins = num_bins;
    p->max_n = max_n;
    p->xcd_map = opts.xcd_map == 0 ? 1 : (uint32_t)opts.xcd_map;

    const uint32_t lds_bins16 = std::min<uint32_t>(kMaxLdsBins16,
                                                   (lds_dyn - (4 + pca::kEventCap) * 4) / 2) & ~255u;
    const uint32_t lds_bins8 = std::min<uint32_t>(kMaxLdsBins8,
                                                  lds_dyn - (4 + pca::kMinEventCap8) * 4) & ~255u;
    const uint32_t cap32 = lds_bins & ~255u;
    int path = opts.path;
    if (path == HIST_PATH_AUTO) {
        if (num_bins <= lds_bins8) path = HIST_PATH_FULL;
        else if (num_bins <= kRangeMaxR * lds_bins16) path = HIST_PATH_RANGE;  // see kRangeMaxR
        else path = HIST_PATH_SCATTER;
    }
    p->path = path;
    // AUTO aggregation: the hot slot for the two-phase path only. There it cost
    // 3% on uniform and Gaussian input and cut the owner phase 2-4x on Zipf and
    // hot-bin input; on the single-pass sweeps it cost 5% on uniform input and
    // did not help Zipf.
    p->agg = opts.aggregation >= 0 ? opts.aggregation : (path == HIST_PATH_SCATTER ? 1 : 0);

    if (path == HIST_PATH_FULL || path == HIST_PATH_RANGE) {
        // Counter width: 32-bit while a workgroup's slice fits, else 16-bit.
        uint32_t cw = (uint32_t)opts.counter_bits;
        if (cw == 0) {
            // Measured on 2^26 uniform elements: 16-bit counters (1024-thread
            // workgroups, two per CU) take 50-52 us from 2^10 to 2^14 bins and at
            // 2^16, against 52-55 us for 32-bit ones. 32-bit counters win only
            // where their slice leaves one workgroup per CU (24,576 bins: 48.8
            // vs 52.1 us; 32,768: 49.7 vs 52.7 us). 8-bit counters hold the most
            // bins per workgroup, which saves input passes: 2^17 bins in one
            // pass (53.0 us against 65.1 for two 16-bit ranges), 2^18 in two
            // (64.7 against 118.2 for four), and they stay ahead on Zipf s = 1.1
            // input there (85.3 vs 105.9, 118.2 vs 167.2 us). Up to 2^16 bins
            // they gain at most 3.7% on uniform input (2^11-2^12 bins; 1.4% or
            // less elsewhere) and lose 1.2-1.3x on Zipf input, whose hot bytes
            // wrap every 256 counts (2^14 bins: 74.1 vs 56.3 us).
            if (path == HIST_PATH_FULL)
                cw = num_bins > lds_bins16 ? 8 : num_bins > kMaxLdsBins / 2 && num_bins <= cap32 ? 32 : 16;
            else if (opts.range_bins > 0)
                cw = (uint32_t)opts.range_bins <= cap32 ? 32 : (uint32_t)opts.range_bins <= lds_bins16 ? 16 : 8;
            else cw = 8;
        }
        const uint32_t cap = cw == 32 ? cap32 : cw == 16 ? lds_bins16 : lds_bins8;
        uint32_t S, R;
        if (path == HIST_PATH_FULL) {
            R = 1;
            S = (num_bins + 255) & ~255u;
        } else if (opts.range_bins > 0) {
            S = (uint32_t)opts.range_bins;
            R = ceil_div(num_bins, S);
        } else {
            // Smallest R that fits LDS, then the one among R..2R that keeps the
            // most CUs busy per element read (R owners read every element).
            const uint32_t rmin = std::max<uint32_t>(2, ceil_div(num_bins, cap));
            double best = 1e30;
            R = rmin;
            for (uint32_t r = rmin; r <= 2 * rmin; ++r) {
                uint32_t g = (uint32_t)d.cu / r;
                if (g >= (uint32_t)d.xcd) g = g / d.xcd * d.xcd;
                if (g == 0) g = 1;
                const double cost = (double)r / ((double)g * r / d.cu);
                if (cost < best - 1e-9) { best = cost; R = r; }
            }
            S = (ceil_div(num_bins, R) + 255) & ~255u;
            R = ceil_div(num_bins, S);
        }
        if (S > cap || S == 0) return HIST_ERR_UNSUPPORTED;
        auto chunks_for = [&](uint32_t lds_bytes, uint64_t max_elems_wg, uint32_t *wg_out) {
            const uint32_t occ_lds = std::max<uint32_t>(1, d.lds / lds_bytes);
            uint32_t wg = (uint32_t)opts.wg_size;
            // Measured: 1024 threads, except a 32-bit slice that leaves one
            // workgroup per CU, which runs best with 512 (32,768 bins: 49.7 vs
            // 52.6 us; 16-bit at 65,536 bins: 50.8 with 1024 vs 56.4 us).
            if (wg == 0) wg = cw == 32 && occ_lds == 1 ? 512 : 1024;
            uint32_t occ = std::min<uint32_t>(occ_lds, kMaxWavesPerCU / (wg / 64));
            // Registers can bound residency below what LDS allows (a 1024-thread
            // sweep with more than 64 VGPRs fits once per CU): chunks beyond the
            // resident ones would run as a second round.
            // (4 SIMDs per CU)
            const uint32_t res = d.sweep_waves_per_simd == 0
                                     ? sweep_resident(cw, wg, p->agg, lds_bytes)
                                     : d.sweep_waves_per_simd == ~0u ? ~0u
                                                                     : d.sweep_waves_per_simd * 4u / (wg / 64u);
            if (res > 0) occ = std::max<uint32_t>(1, std::min(occ, res));
            uint32_t G = (uint32_t)opts.groups, slots = 0;
            if (G == 0) {
                G = (uint32_t)d.cu * occ / R;
                if (G >= (uint32_t)d.xcd) G = G / d.xcd * d.xcd;
                slots = std::max<uint32_t>(1, G);  // chunks whose owners are resident at once
                // Keep the merge traffic (G rows of num_bins counts, ~4 bits each for
                // the counts a chunk of n/G elements produces) a small fraction of the
                // input (4n bytes), and every chunk a useful size.
                const uint64_t by_merge = std::max<uint64_t>(1, max_n / num_bins);
                const uint64_t by_size = std::max<uint64_t>(1, max_n / kMinElemsPerGroup);
                G = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>({G, by_merge, by_size}));
            }
            // Enough chunks that no workgroup's carry-event list can overflow;
            // when that takes more chunks than run at once, whole rounds of them.
            const uint32_t gmin = ceil_div(max_n, max_elems_wg);
            if (G < gmin) G = slots ? ceil_div(gmin, slots) * slots : gmin;
            *wg_out = wg;
            return G;
        };
        // Interleaved LDS copies only when asked for: on uniform input every
        // copy count above 1 measured slower (2^10 bins: 52.6 us with one copy,
        // 59.9 with 8, 67.4 with 16), as clearing and summing the copies costs
        // more than the bank conflicts they spread.
        uint32_t kshift = 0, wg = 0, G = 0, ev_cap = 0;
        uint64_t max_elems_wg = 1ull << 40;  // no list: any n < 2^32
        if (cw == 32) {
            if (opts.lds_copies > 0)
                while ((1u << (kshift + 1)) <= (uint32_t)opts.lds_copies) ++kshift;
            if ((S << kshift) * 4 > lds_dyn) return HIST_ERR_UNSUPPORTED;
        } else if (cw == 16) {
            max_elems_wg = kMaxElemsPerWG16;
        } else {
            // The event list takes what LDS the workgroups of a CU leave, so a
            // large slice (one workgroup per CU) lets a workgroup count more.
            const uint32_t occ = std::max<uint32_t>(1, lds_dyn / sweep_lds_bytes(8, S, 0, pca::kMinEventCap8));
            ev_cap = (lds_dyn / occ - S) / 4 - 4;
            // the list goes on in the workspace for kEvSpill8 entries, so
            // that the Zipf 2^18-bin workload's 2^21-element chunks (one
            // round of 128 chunks, R = 2) fit: measured 353 against 371 us
            // with 256 chunks at 266,000,000 elements
            max_elems_wg = 255ull * (ev_cap + pca::kEvSpill8 - 16);
        }
        G = chunks_for(sweep_lds_bytes(cw, S, kshift, ev_cap), max_elems_wg, &wg);
        p->range_bins = S;
        p->ranges = R;
        p->groups = G;
        p->wg = wg;
        p->cw = cw;
        p->kshift = kshift;
        p->ev_cap = ev_cap;
        p->max_elems_wg = max_elems_wg;
        p->nblk = ceil_div(num_bins, pca::kBlockBins);
        uint64_t off = 0;
        p->part_rows = G > 1 ? G : 0;
        p->off_partials = off;
        off += partial_bytes(p->part_rows, p->nblk);
        // How the R owners of a chunk read it (1024-thread workgroups with packed
        // counters only: the pacer's LDS words sit in the carry-event block).
        p->pacing = 1;
        if (R > 1 && wg == 1024 && cw != 32) p->pacing = opts.pacing > 0 ? (uint32_t)opts.pacing : 1u;
        if (p->pacing >= 3) {
            p->off_progress = off;
            off += align_up((uint64_t)G * R * 4, 256);
        }
        if (cw == 8) {
            p->off_spill = off;
            off += align_up((uint64_t)G * R * pca::kEvSpill8 * 4, 256);
        }
        p->need = off;
    } else if (path == HIST_PATH_STREAM) {
        const uint32_t S = 1u << kScatterShift;
        const uint32_t R = ceil_div(num_bins, S);
        if (R > kStreamMaxRanges) return HIST_ERR_UNSUPPORTED;
        const uint32_t T = std::max<uint32_t>(1, ceil_div(max_n / 4, pca::kStreamTileVecs));
        // one workgroup per CU (each holds a 128 KiB slice), and at least one
        // per range, so that every range has an owner from the first tickets
        // on; by default 5/8 of them start as producers
        const uint32_t W = std::max<uint32_t>((uint32_t)d.cu, R);
        const uint32_t P = opts.groups > 0 ? std::min<uint32_t>((uint32_t)opts.groups, W)
                                           : std::max<uint32_t>(1, W * 5 / 8);
        p->range_bins = S;
        p->ranges = R;
        p->tiles = T;
        p->qlog = 0;
        p->grid = W;
        p->producers = P;
        p->groups = P;
        p->bt = std::min(kStreamMaxBlockTiles,
                         std::max(kStreamMinBlockTiles, (8u * R + 15u) & ~15u));
        p->spin = 1u << (opts.spin_log2 > 0 ? (uint32_t)opts.spin_log2 : kStreamSpinLog2);
        // the owner's slice and a trash word per lane; the producers' waves
        p->uwords = std::max<uint32_t>(S + 64, (kStreamWG / 64) * pca::kStreamWaveWords);
        p->wg = kStreamWG;
        p->nblk = S / pca::kBlockBins;
        if ((p->uwords + pca::kStreamShWords) * 4 > d.lds) return HIST_ERR_UNSUPPORTED;
        uint64_t off = 0;
        p->off_ctl = off;
        off += align_up((uint64_t)(pca::kCtlWords + R + T) * 4, 256);
        // run-table rows of whole 128-byte lines, one per sub-tile
        p->rstride = (R + 31u) & ~31u;
        const uint64_t subs = (uint64_t)T * pca::kStreamSubsPerTile;
        p->off_tcnt = off;
        off += subs * p->rstride * 4;
        p->off_stage = off;
        off += subs * pca::kStreamSubCap * 2;
        p->off_trace = off;
        off += align_up((uint64_t)W * pca::kStreamTraceWords * 4, 256);
        // the stint pool: a stint holds at least one block, and there are at
        // most W + the move budget of them
        p->move_budget = kStreamMovesPerWG * W;
        const uint64_t blocks = (uint64_t)R * ceil_div(T, p->bt);
        p->pool_slots = (uint32_t)std::min<uint64_t>(W + p->move_budget, blocks);
        p->off_pool = off;
        off += (uint64_t)p->pool_slots * S * 4;
        p->off_slot_range = off;
        off += align_up((uint64_t)p->pool_slots * 4, 256);
        p->need = off;
    } else {
        const uint32_t S = 1u << kScatterShift;
        const uint32_t R = ceil_div(num_bins, S);
        const uint64_t nvec_max = max_n / 4;
        const uint32_t T = std::max<uint32_t>(1, ceil_div(nvec_max, kPartWG * kScatterVPT));
        uint32_t W = (uint32_t)opts.groups;
        if (W == 0) W = (uint32_t)d.cu;
        // Sub-counters per range in the partition's rank atomics: up to 16,
        // within two counters per partition thread.
        uint32_t qlog = 4;
        while (qlog > 0 && (R << qlog) > 2 * kPartWG) --qlog;
        p->range_bins = S;
        p->ranges = R;
        p->tiles = T;
        p->owners = W;
        p->groups = W;
        p->qlog = qlog;
        p->nblk = S / pca::kBlockBins;
        p->wg = kScatterWG;
        uint64_t off = 0;
        p->off_stage = off;
        off += align_up((uint64_t)T * kScatterCap * 2, 256);
        p->off_tcnt = off;
        off += align_up((uint64_t)R * T * 4, 256);
        p->off_tbase = off;
        off += align_up((uint64_t)R * T * 4, 256);
        p->off_tpre = off;
        off += align_up((uint64_t)R * T * 4, 256);
        p->off_totals = off;
        off += align_up((uint64_t)R * 4, 256);
        p->off_segtot = off;
        off += align_up((uint64_t)R * ceil_div(T, pca::kScanSeg) * 4, 256);
        p->off_starts = off;  // uint64 start of every range in the concatenation, and the total
        off += align_up((uint64_t)(R + 1) * 8, 256);
        p->tile_major = R >= kTileMajorRanges;
        if (p->tile_major) {
            // tile-major run starts; the tile-major run counts go to the tpre
            // region, which the range scan overwrites after the transpose
            p->off_tbase_tm = off;
            off += align_up((uint64_t)R * T * 4, 256);
        }
        p->part_rows = W + R;
        p->off_partials = off;
        off += partial_bytes(p->part_rows, p->nblk);
        // the in-place window, sized for the partition's largest grid
        p->window = opts.window == 1 ? 1u : opts.window == 2 ? 2u : 0u;
        if (p->window != 1) {
            p->wbins = HIST_WINDOW_BINS;
            p->wrows = std::min<uint32_t>(T, kPartPerCU * (uint32_t)d.cu);
            p->off_wsel = off;
            off += 256;
            p->off_wpart = off;
            off += align_up((uint64_t)p->wrows * (p->wbins + pca::kWindowRowPad) * 4, 256);
        }
        p->need = off;
    }
    return HIST_OK;
}

bool overlaps(const void *a, uint64_t an, const void *b, uint64_t bn)
{
    if (!a || !b || an == 0 || bn == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

template <typename K>
hipError_t allow_lds(K kernel, uint32_t bytes)
{
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// Start and stop events to attach to a kernel's own dispatch (null when timing
// is off). Attached events take the kernel's start and end timestamps, which
// is what a profiler's kernel trace reports; no marker packet is queued
// between kernels.
struct KEv {
    hipEvent_t a = nullptr, b = nullptr;
};

template <typename F, typename... Args>
void launch(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, const KEv &ev,
            Args... args)
{
    if (ev.a || ev.b)
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, ev.a, ev.b, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
}

struct SweepArgs {
    pca::InputView in;
    uint32_t G, xcds;
    pca::Partials out;
    uint32_t *direct;
    uint32_t accumulate;
};

// Epoch of the paced sweeps' progress words: a new one per run, so that words
// an earlier run left read as "not started".
std::atomic<uint32_t> g_pace_epoch{0};

template <int WG, int AGG, int CW>
hipError_t launch_sweep_t(const hist_plan_impl *p, const SweepArgs &a, hipStream_t s, const KEv &ev)
{
    // Packed counters: 2 vectors (8 returning LDS atomics) per thread per
    // iteration stay within the LDS wait counter; measured 12% faster than 4.
    constexpr int U = CW == 32 ? 4 : 2;
    const uint32_t bytes = sweep_lds_bytes(CW, p->range_bins, CW == 32 ? p->kshift : 0u, p->ev_cap);
    pca::Pacing pc{nullptr, 0u, 0u};
    auto k = pca::k_sweep<WG, U, AGG, CW, false>;
    if constexpr (WG == 1024 && CW != 32) {
        // R > 1 owners at their own pace: plain loads. Measured against
        // non-temporal ones: the Zipf 262,144-bin workload 373 against
        // 380-395 us, 2^18 uniform bins at 2^26 elements 59.0 against 62-69 us
        // (with one owner the two time alike: 48.8 us on the headline).
        if (p->pacing == 1 && p->ranges > 1 && a.in.nvec * 16 > kMallBytes)
            k = pca::k_sweep<WG, U, AGG, CW, false, false>;
        if (p->pacing >= 2) {
            k = pca::k_sweep<WG, U, AGG, CW, true>;
            if (p->pacing >= 3) {
                pc.prog = reinterpret_cast<uint32_t *>(p->ws + p->off_progress);
                pc.epoch = g_pace_epoch.fetch_add(1, std::memory_order_relaxed) & 0xFFFu;
                pc.window = p->pacing - 2;
            }
        }
    }
    hipError_t e = allow_lds(k, bytes);
    if (e != hipSuccess) return e;
    launch(k, dim3(a.G * p->ranges), dim3(WG), bytes, s, ev, a.in, p->num_bins, p->range_bins,
           p->ranges, a.G, a.xcds, CW == 32 ? p->kshift : 0u, p->ev_cap,
           CW == 8 ? reinterpret_cast<uint32_t *>(p->ws + p->off_spill) : nullptr, a.out, a.direct,
           a.accumulate, pc);
    return hipGetLastError();
}

template <int WG, int CW>
hipError_t launch_sweep_agg(const hist_plan_impl *p, const SweepArgs &a, hipStream_t s, const KEv &ev)
{
    switch (p->agg) {
    case 0: return launch_sweep_t<WG, 0, CW>(p, a, s, ev);
    case 1: return launch_sweep_t<WG, 1, CW>(p, a, s, ev);
    case 2: return launch_sweep_t<WG, 2, CW>(p, a, s, ev);
    default: return launch_sweep_t<WG, 4, CW>(p, a, s, ev);
    }
}

template <int CW>
hipError_t launch_sweep_wg(const hist_plan_impl *p, const SweepArgs &a, hipStream_t s, const KEv &ev)
{
    switch (p->wg) {
    case 256: return launch_sweep_agg<256, CW>(p, a, s, ev);
    case 512: return launch_sweep_agg<512, CW>(p, a, s, ev);
    default: return launch_sweep_agg<1024, CW>(p, a, s, ev);
    }
}

template <int WG, int AGG, int CW>
uint32_t sweep_resident_t(uint32_t lds_bytes)
{
    auto k = pca::k_sweep<WG, CW == 32 ? 4 : 2, AGG, CW>;
    int blocks = 0;
    if (allow_lds(k, lds_bytes) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, reinterpret_cast<const void *>(k), WG,
                                                     lds_bytes) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return blocks > 0 ? (uint32_t)blocks : 0u;
}

template <int WG, int CW>
uint32_t sweep_resident_agg(int agg, uint32_t lds_bytes)
{
    switch (agg) {
    case 0: return sweep_resident_t<WG, 0, CW>(lds_bytes);
    case 1: return sweep_resident_t<WG, 1, CW>(lds_bytes);
    case 2: return sweep_resident_t<WG, 2, CW>(lds_bytes);
    default: return sweep_resident_t<WG, 4, CW>(lds_bytes);
    }
}

template <int CW>
uint32_t sweep_resident_wg(uint32_t wg, int agg, uint32_t lds_bytes)
{
    switch (wg) {
    case 256: return sweep_resident_agg<256, CW>(agg, lds_bytes);
    case 512: return sweep_resident_agg<512, CW>(agg, lds_bytes);
    default: return sweep_resident_agg<1024, CW>(agg, lds_bytes);
    }
}

uint32_t sweep_resident(uint32_t cw, uint32_t wg, int agg, uint32_t lds_bytes)
{
    return cw == 32   ? sweep_resident_wg<32>(wg, agg, lds_bytes)
           : cw == 16 ? sweep_resident_wg<16>(wg, agg, lds_bytes)
                      : sweep_resident_wg<8>(wg, agg, lds_bytes);
}

hipError_t launch_partition(const hist_plan_impl *p, pca::InputView in, uint32_t T, hipStream_t s,
                            const KEv &ev, bool window)
{
    // staged slots: 2 bytes per element
    auto k = 2 * ((uint64_t)in.nvec * 4 + in.head + in.tail) > kMallBytes
                 ? pca::k_partition<kPartWG, kScatterVPT, true>
                 : pca::k_partition<kPartWG, kScatterVPT, false>;
    const uint32_t npad = ((p->ranges << p->qlog) + 3u) & ~3u;
    const uint32_t bytes = (3 * npad + 64) * 4 + 2 * kScatterCap * 2 + (window ? p->wbins * 4 + 16 : 0u);
    hipError_t e = allow_lds(k, bytes);
    if (e != hipSuccess) return e;
    // persistent: kPartPerCU workgroups per CU, each walking tiles
    const uint32_t grid = std::min<uint32_t>(T, kPartPerCU * (uint32_t)p->dev.cu);
    uint32_t *tcnt = reinterpret_cast<uint32_t *>(p->ws + (p->tile_major ? p->off_tpre : p->off_tcnt));
    uint32_t *tbase =
        reinterpret_cast<uint32_t *>(p->ws + (p->tile_major ? p->off_tbase_tm : p->off_tbase));
    const uint32_t rstride = p->tile_major ? 1u : T, tstride = p->tile_major ? p->ranges : 1u;
    launch(k, dim3(grid), dim3(kPartWG), bytes, s, ev, in, p->num_bins, kScatterShift, p->ranges,
           p->qlog, T, reinterpret_cast<uint16_t *>(p->ws + p->off_stage), kScatterCap, tcnt, tbase,
           rstride, tstride,
           window ? reinterpret_cast<const uint32_t *>(p->ws + p->off_wsel) : (const uint32_t *)nullptr,
           p->wbins, reinterpret_cast<uint32_t *>(p->ws + p->off_wpart));
    return hipGetLastError();
}

pca::Partials plan_partials(const hist_plan_impl *p)
{
    const uint64_t cells = (uint64_t)p->part_rows * p->nblk;
    pca::Partials P;
    P.plane0 = reinterpret_cast<uint8_t *>(p->ws + p->off_partials);
    P.upper = P.plane0 + align_up(cells * pca::kPlaneBytes, 256);
    P.width = P.upper + align_up(cells * pca::kPlaneBytes * pca::kUpperPlanes, 256);
    P.nblk = p->nblk;
    return P;
}

template <int AGG>
hipError_t launch_owner_t(const hist_plan_impl *p, uint32_t T, uint32_t *counts, uint32_t accumulate,
                          hipStream_t s, const KEv &ev, const uint32_t *hot_seen)
{
    // the staged slots of T tiles, as the partition chose to store them
    auto k = 2 * (uint64_t)T * kScatterTile > kMallBytes ? pca::k_bucket_hist<kScatterWG, 8, AGG, true>
                                                          : pca::k_bucket_hist<kScatterWG, 8, AGG, false>;
    const uint32_t bytes = p->range_bins * 4 + (p->ranges + 1) * 8 + 4 * 4;
    hipError_t e = allow_lds(k, bytes);
    if (e != hipSuccess) return e;
    launch(k, dim3(p->owners), dim3(kScatterWG), bytes, s, ev,
           reinterpret_cast<const uint16_t *>(p->ws + p->off_stage), kScatterCap,
           reinterpret_cast<const uint32_t *>(p->ws + p->off_tcnt),
           reinterpret_cast<const uint32_t *>(p->ws + p->off_tbase),
           reinterpret_cast<const uint32_t *>(p->ws + p->off_tpre),
           reinterpret_cast<const uint32_t *>(p->ws + p->off_totals), p->ranges, T, p->range_bins,
           p->num_bins, p->owners, plan_partials(p),
           reinterpret_cast<uint64_t *>(p->ws + p->off_starts), counts, accumulate, hot_seen);
    return hipGetLastError();
}

struct PhaseTimer {
    hist_plan_impl *p;
    hipStream_t s;
    uint32_t slot;
    bool on;
    PhaseTimer(hist_plan_impl *p_, hipStream_t s_) : p(p_), s(s_)
    {
        on = p->tcap > 0 && p->truns < p->tcap;
        slot = p->truns;
        if (on) {
            std::fill(p->used.begin() + (size_t)slot * HIST_MAX_PHASES,
                      p->used.begin() + (size_t)(slot + 1) * HIST_MAX_PHASES, 0);
            p->truns++;
        }
    }
    hipEvent_t &event(int ph, int which)
    {
        return p->ev[((size_t)slot * HIST_MAX_PHASES + ph) * 2 + which];
    }
    // Events to attach to a kernel of phase ph: the phase's first kernel
    // carries the start event and its last kernel the stop event (a phase of
    // one kernel carries both).
    KEv ev(int ph, bool first = true, bool last = true)
    {
        KEv e;
        if (!on) return e;
        if (first) e.a = event(ph, 0);
        if (last) {
            e.b = event(ph, 1);
            p->used[(size_t)slot * HIST_MAX_PHASES + ph] = 1;
        }
        return e;
    }
};

}  // namespace

namespace {

template <bool ACC>
hipError_t launch_merge(const pca::Partials &P, uint32_t G, uint32_t num_bins, uint32_t *counts,
                        uint32_t nblk, hipStream_t s, const KEv &ev)
{
    if (G <= 256)
        launch(pca::k_merge<4, ACC>, dim3(nblk), dim3(256), 0, s, ev, P, G, num_bins, counts);
    else if (G <= 512)
        launch(pca::k_merge<8, ACC>, dim3(nblk), dim3(512), 0, s, ev, P, G, num_bins, counts);
    else
        launch(pca::k_merge<16, ACC>, dim3(nblk), dim3(1024), 0, s, ev, P, G, num_bins, counts);
    return hipGetLastError();
}

// A range's slots are the rows of its overlapping owners, about W / R + 1 of
// them: one wave per block (64 rows per round trip) once ranges are many,
// four (256 rows) when each range has many owners.
template <bool ACC>
hipError_t launch_merge_slots(const hist_plan_impl *p, uint32_t num_bins, uint32_t *counts,
                              hipStream_t s, const KEv &ev)
{
    const pca::Partials P = plan_partials(p);
    const uint64_t *starts = reinterpret_cast<const uint64_t *>(p->ws + p->off_starts);
    // With many ranges a range has few owner rows, and one round per batch (78
    // VGPRs, 6 waves per SIMD) beats eight (154 VGPRs, 3 waves): 2^22 uniform
    // bins 31.0 -> 20.3 us. A range holding a hot bin has many rows, which one
    // round per batch walks slowly: on the 2^20-bin hot-bin input (32 ranges,
    // 256 owners) it took 24.0 us against 13.9, hence the switch at
    // ranges * 4 >= owners.
    // From ranges >= 4 * owners most ranges have one owner, which wrote its
    // counts itself; a workgroup then takes 8 blocks, so that such a range
    // costs one check per 2,048 bins (2^26 bins: 114 -> 56 us). Where most
    // ranges are shared the 8 blocks run one after another and it loses
    // (2^22 bins: 20.3 -> 27.5 us).
    constexpr uint32_t kManyBPW = 8;
    if (p->ranges >= 4u * p->owners)
        launch(pca::k_merge_slots<1, ACC, 1, kManyBPW>, dim3(ceil_div(num_bins, 256 * kManyBPW)),
               dim3(64), 0, s, ev, P, starts, p->ranges, p->range_bins, num_bins, p->owners, counts);
    else if (p->ranges * 4u >= p->owners)
        launch(pca::k_merge_slots<1, ACC, 1, 1>, dim3(ceil_div(num_bins, 256)), dim3(64), 0, s, ev,
               P, starts, p->ranges, p->range_bins, num_bins, p->owners, counts);
    else if (p->ranges >= 16)
        launch(pca::k_merge_slots<1, ACC, pca::kMergeRounds, 1>, dim3(ceil_div(num_bins, 256)),
               dim3(64), 0, s, ev, P, starts, p->ranges, p->range_bins, num_bins, p->owners, counts);
    else
        launch(pca::k_merge_slots<4, ACC, pca::kMergeRounds, 1>, dim3(ceil_div(num_bins, 256)),
               dim3(256), 0, s, ev, P, starts, p->ranges, p->range_bins, num_bins, p->owners,
               counts);
    return hipGetLastError();
}

hist_status_t run_impl(hist_plan_t *p, uint32_t *counts, const int32_t *input, uint64_t n,
                       uint32_t num_bins, hipStream_t stream, uint32_t accumulate)
{
    if (!p || !counts) return HIST_ERR_INVALID_ARG;
    if (n > 0 && !input) return HIST_ERR_INVALID_ARG;
    if (num_bins != p->num_bins || n > p->max_n) return HIST_ERR_INVALID_ARG;
    if (((uintptr_t)counts & 3u) != 0 || ((uintptr_t)input & 3u) != 0) return HIST_ERR_INVALID_ARG;
    const uint64_t cbytes = (uint64_t)num_bins * 4, ibytes = n * 4;
    if (overlaps(counts, cbytes, input, ibytes) || overlaps(counts, cbytes, p->ws, p->need) ||
        overlaps(input, ibytes, p->ws, p->need))
        return HIST_ERR_INVALID_ARG;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return HIST_ERR_HIP;
    if (dev != p->dev.device) return HIST_ERR_INVALID_ARG;

    PhaseTimer tm(p, stream);
    hipError_t e = hipSuccess;
    if (n == 0) {
        if (accumulate) return HIST_OK;  // nothing to add
        launch(pca::k_fill_zero, dim3(std::max<uint32_t>(1, std::min<uint32_t>(1024, ceil_div(num_bins, 256)))),
               dim3(256), 0, stream, tm.ev(PH_SWEEP), counts, (uint64_t)num_bins);
        return hipGetLastError() == hipSuccess ? HIST_OK : HIST_ERR_HIP;
    }

    pca::InputView in;
    in.ptr = input;
    const uint64_t mis = ((uintptr_t)input & 15u) / 4;
    in.head = (uint32_t)std::min<uint64_t>(n, mis ? 4 - mis : 0);
    in.nvec = (n - in.head) / 4;
    in.tail = (uint32_t)(n - in.head - 4 * in.nvec);

    if (p->path == HIST_PATH_FULL || p->path == HIST_PATH_RANGE) {
        // Fewer chunks for a small call: keep the merge a small fraction of the work.
        uint32_t G = p->groups;
        const uint64_t by_merge = std::max<uint64_t>(1, n / num_bins);
        const uint64_t by_size = std::max<uint64_t>(1, n / kMinElemsPerGroup);
        G = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>({G, by_merge, by_size}));
        G = std::max<uint32_t>(G, ceil_div(n, p->max_elems_wg));  // bounds the carry events
        SweepArgs a;
        a.in = in;
        a.G = G;
        a.xcds = (p->xcd_map == 1 && p->ranges > 1 && G % p->dev.xcd == 0) ? p->dev.xcd : 1;
        a.out = plan_partials(p);
        a.direct = G > 1 ? nullptr : counts;
        a.accumulate = accumulate;
        // The co-owners of a chunk (R > 1) do not always find its lines in the
        // XCD's L2: on the Zipf 262,144-bin workload (R = 2, 8-bit counters)
        // the sweep's scaled FETCH_SIZE is 1.8x the input.
        const KEv sev = tm.ev(PH_SWEEP);
        e = p->cw == 32   ? launch_sweep_wg<32>(p, a, stream, sev)
            : p->cw == 16 ? launch_sweep_wg<16>(p, a, stream, sev)
                          : launch_sweep_wg<8>(p, a, stream, sev);
        if (e != hipSuccess) return HIST_ERR_HIP;
        if (G > 1) {
            // one batch of loads per lane covers 8 rows x 8 rounds per wave
            const KEv mev = tm.ev(PH_MERGE);
            e = accumulate ? launch_merge<true>(a.out, G, num_bins, counts, p->nblk, stream, mev)
                           : launch_merge<false>(a.out, G, num_bins, counts, p->nblk, stream, mev);
            if (e != hipSuccess) return HIST_ERR_HIP;
        }
        return HIST_OK;
    }

    if (p->path == HIST_PATH_STREAM) {
        const uint32_t T = std::max<uint32_t>(1, ceil_div(in.nvec, pca::kStreamTileVecs));
        if (T > p->tiles) return HIST_ERR_INVALID_ARG;  // cannot happen for n <= max_n
        uint32_t *ctl = reinterpret_cast<uint32_t *>(p->ws + p->off_ctl);
        const uint32_t words = pca::kCtlWords + p->ranges + T;
        launch(pca::k_stream_prepare, dim3(std::min<uint32_t>(1024, ceil_div(words, 256))), dim3(256),
               0, stream, tm.ev(PH_STREAM, true, false), ctl, words);
        pca::StreamArgs sa;
        sa.in = in;
        sa.num_bins = num_bins;
        sa.ranges = p->ranges;
        sa.tiles = T;
        sa.bt = p->bt;
        sa.nblocks = ceil_div(T, p->bt);
        sa.producers = p->producers;
        sa.spin = p->spin;
        sa.uwords = p->uwords;
        sa.ctl = ctl;
        sa.rows = reinterpret_cast<uint32_t *>(p->ws + p->off_tcnt);
        sa.stage = reinterpret_cast<uint16_t *>(p->ws + p->off_stage);
        sa.trace = reinterpret_cast<uint32_t *>(p->ws + p->off_trace);
        sa.rstride = p->rstride;
        sa.counts = counts;
        sa.accumulate = accumulate;
        sa.pool = reinterpret_cast<uint32_t *>(p->ws + p->off_pool);
        sa.slot_range = reinterpret_cast<uint32_t *>(p->ws + p->off_slot_range);
        sa.pool_slots = p->pool_slots;
        sa.move_budget = p->move_budget;
        auto k = pca::k_stream<kStreamWG>;
        const uint32_t bytes = (p->uwords + pca::kStreamShWords) * 4;
        e = allow_lds(k, bytes);
        if (e != hipSuccess) return HIST_ERR_HIP;
        launch(k, dim3(p->grid), dim3(kStreamWG), bytes, stream, tm.ev(PH_STREAM, false, false), sa);
        launch(pca::k_stream_merge<256>, dim3(p->ranges * (S_STREAM / pca::kStreamMergeBins)), dim3(256), 0,
               stream, tm.ev(PH_STREAM, false, true), (const uint32_t *)ctl, (const uint32_t *)sa.pool,
               (const uint32_t *)sa.slot_range, p->pool_slots, num_bins, counts, accumulate);
        return hipGetLastError() == hipSuccess ? HIST_OK : HIST_ERR_HIP;
    }

    // SCATTER
    const uint32_t T = std::max<uint32_t>(1, ceil_div(in.nvec, kPartWG * kScatterVPT));
    if (T > p->tiles) return HIST_ERR_INVALID_ARG;  // cannot happen for n <= max_n
    // the in-place window: chosen on the device from a sample of this input
    // (AUTO leaves it out below 2^22 elements, where the pick's few
    // microseconds would not pay)
    const bool window = p->window == 2 || (p->window == 0 && n >= kWindowMinElems);
    uint32_t *wsel = reinterpret_cast<uint32_t *>(p->ws + p->off_wsel);
    if (window)
        launch(pca::k_window_pick<1024>, dim3(1), dim3(1024), 0, stream, tm.ev(PH_PART, true, false),
               in.ptr, n, num_bins, p->wbins, p->window == 2 ? 0u : kWindowMinShare, wsel);
    e = launch_partition(p, in, T, stream, tm.ev(PH_PART, !window, true), window);
    if (e != hipSuccess) return HIST_ERR_HIP;
    {
        const uint32_t nseg = ceil_div(T, pca::kScanSeg);
        uint32_t *tpre = reinterpret_cast<uint32_t *>(p->ws + p->off_tpre);
        uint32_t *segtot = reinterpret_cast<uint32_t *>(p->ws + p->off_segtot);
        // the phase's first kernel carries its start event, the last its stop
        if (p->tile_major)
            launch(pca::k_transpose, dim3(ceil_div(p->ranges, 64), ceil_div(T, 64), 2), dim3(256), 0,
                   stream, tm.ev(PH_SCAN, true, false), tpre,
                   reinterpret_cast<uint32_t *>(p->ws + p->off_tcnt),
                   reinterpret_cast<const uint32_t *>(p->ws + p->off_tbase_tm),
                   reinterpret_cast<uint32_t *>(p->ws + p->off_tbase), T, p->ranges);
        const uint32_t *tcnt = reinterpret_cast<const uint32_t *>(p->ws + p->off_tcnt);
        uint32_t *totals = reinterpret_cast<uint32_t *>(p->ws + p->off_totals);
        if (p->ranges <= kRangeScanMaxRanges && T <= 1024u * 32u) {
            // every range's lengths in one load, rows of 1,024 tiles (2^26
            // elements over 2^20 bins: 4.2 us against 9.2 for the two passes;
            // 2^28 over 2^20: 7.3 against 12.2)
            const KEv sev = tm.ev(PH_SCAN, !p->tile_major, true);
            if (T <= 1024u * 4u)
                launch(pca::k_range_scan<1024, 4>, dim3(p->ranges), dim3(1024), 0, stream, sev, tcnt, T, tpre,
                       totals);
            else if (T <= 1024u * 16u)
                launch(pca::k_range_scan<1024, 16>, dim3(p->ranges), dim3(1024), 0, stream, sev, tcnt, T, tpre,
                       totals);
            else
                launch(pca::k_range_scan<1024, 32>, dim3(p->ranges), dim3(1024), 0, stream, sev, tcnt, T, tpre,
                       totals);
        } else {
            launch(pca::k_seg_scan<1024>, dim3(p->ranges * nseg), dim3(1024), 0, stream,
                   tm.ev(PH_SCAN, !p->tile_major, false), tcnt, T, nseg, tpre, segtot);
            launch(pca::k_seg_fix<256>, dim3(p->ranges * nseg), dim3(256), 0, stream,
                   tm.ev(PH_SCAN, false, true), T, nseg, tpre, segtot, totals);
        }
    }
    if (hipGetLastError() != hipSuccess) return HIST_ERR_HIP;
    {
        const KEv oev = tm.ev(PH_OWNER);
        // the pick's verdict on a hot value, when it ran
        const uint32_t *hot = window ? wsel + pca::kSelOwnersHot : nullptr;
        switch (p->agg) {
        case 0: e = launch_owner_t<0>(p, T, counts, accumulate, stream, oev, hot); break;
        case 1: e = launch_owner_t<1>(p, T, counts, accumulate, stream, oev, hot); break;
        case 2: e = launch_owner_t<2>(p, T, counts, accumulate, stream, oev, hot); break;
        default: e = launch_owner_t<4>(p, T, counts, accumulate, stream, oev, hot); break;
        }
    }
    if (e != hipSuccess) return HIST_ERR_HIP;
    {
        const KEv sev = tm.ev(PH_SLOTS, true, !window);
        e = accumulate ? launch_merge_slots<true>(p, num_bins, counts, stream, sev)
                       : launch_merge_slots<false>(p, num_bins, counts, stream, sev);
    }
    if (e != hipSuccess) return HIST_ERR_HIP;
    if (window) {
        // after the owners and the slot merge: the window's bins hold the
        // staged elements' counts (none), to which the rows are added
        launch(pca::k_window_merge<1024>, dim3(ceil_div(p->wbins, pca::kWindowMergeBins)), dim3(1024), 0, stream,
               tm.ev(PH_SLOTS, false, true), (const uint32_t *)wsel,
               reinterpret_cast<const uint32_t *>(p->ws + p->off_wpart),
               std::min<uint32_t>(T, kPartPerCU * (uint32_t)p->dev.cu), p->wbins, num_bins, counts);
        if (hipGetLastError() != hipSuccess) return HIST_ERR_HIP;
    }
    return HIST_OK;
}

void fill_info(const hist_plan_impl *p, hist_plan_info_t *info);

// Device numbers for run_in_workspace, taken once per device: the runtime's
// property query costs far more than the planning arithmetic.
constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
DeviceInfo g_dev_info[kMaxDevices];
hist_status_t g_dev_status[kMaxDevices];

hist_status_t device_info_cached(int dev, DeviceInfo *d)
{
    if (dev < 0 || dev >= kMaxDevices) return HIST_ERR_UNSUPPORTED;
    std::call_once(g_dev_once[dev], [dev] { g_dev_status[dev] = query_device(&g_dev_info[dev]); });
    if (g_dev_status[dev] != HIST_OK) return g_dev_status[dev];
    *d = g_dev_info[dev];
    return HIST_OK;
}

}  // namespace

namespace pca_host {

hist_status_t device_supported(int dev)
{
    DeviceInfo d;
    return device_info_cached(dev, &d);
}

hist_status_t run_in_workspace(uint32_t *counts, const int32_t *input, uint64_t n,
                               uint32_t num_bins, hipStream_t stream, void *ws, uint64_t ws_bytes,
                               int dev)
{
    if (!counts || (n > 0 && !input) || num_bins == 0 || n > (uint64_t)UINT32_MAX)
        return HIST_ERR_INVALID_ARG;
    if (num_bins > HIST_MAX_BINS) return HIST_ERR_UNSUPPORTED;
    if (!ws || ((uintptr_t)ws & 255u) != 0) return HIST_ERR_WORKSPACE;
    hist_plan_impl p;  // on the stack: its vectors stay empty, nothing is allocated
    hist_status_t st = device_info_cached(dev, &p.dev);
    if (st != HIST_OK) return st;
    const uint64_t max_n = std::max<uint64_t>(n, 1);
    st = design(&p, num_bins, max_n, nullptr);
    if (st != HIST_OK) return st;
    if (p.need > ws_bytes && p.path != HIST_PATH_SCATTER && p.groups > 1) {
        // The one-pass paths' workspace is their partial rows, one per input
        // chunk: take fewer, larger chunks (same kernels, same result).
        uint32_t g = p.groups;
        while (g > 1 && partial_bytes(g, p.nblk) > ws_bytes) g = g > 64 ? g - g / 16 : g - 1;
        if (g >= (uint32_t)p.dev.xcd) g = g / p.dev.xcd * p.dev.xcd;
        hist_plan_opts_t o{};
        o.aggregation = -1;
        o.groups = (int32_t)g;
        hist_plan_impl q;
        q.dev = p.dev;
        st = design(&q, num_bins, max_n, &o);
        if (st != HIST_OK) return st;
        p = q;
    }
    if (p.need > ws_bytes) return HIST_ERR_WORKSPACE;
    p.ws = static_cast<char *>(ws);
    p.ws_bytes = ws_bytes;
    return run_impl(&p, counts, input, n, num_bins, stream, 0u);
}

}  // namespace pca_host

extern "C" {

const char *hist_status_str(hist_status_t s)
{
    switch (s) {
    case HIST_OK: return "ok";
    case HIST_ERR_INVALID_ARG: return "invalid argument";
    case HIST_ERR_UNSUPPORTED: return "unsupported (no gfx950 device current, or size too large)";
    case HIST_ERR_WORKSPACE: return "workspace missing or too small";
    case HIST_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

hist_status_t hist_workspace_size(uint32_t num_bins, uint64_t max_n, const hist_plan_opts_t *opts,
                                  uint64_t *bytes)
{
    if (!bytes || num_bins == 0 || max_n > (uint64_t)UINT32_MAX) return HIST_ERR_INVALID_ARG;
    hist_status_t st = check_opts(opts);
    if (st != HIST_OK) return st;
    if (num_bins > HIST_MAX_BINS) return HIST_ERR_UNSUPPORTED;
    hist_plan_impl p;
    st = query_device(&p.dev);
    if (st != HIST_OK) return st;
    st = design(&p, num_bins, max_n, opts);
    if (st != HIST_OK) return st;
    *bytes = p.need;
    return HIST_OK;
}

hist_status_t hist_plan(hist_plan_t **plan, uint32_t num_bins, uint64_t max_n,
                        const hist_plan_opts_t *opts, void *workspace, uint64_t workspace_bytes)
{
    if (!plan) return HIST_ERR_INVALID_ARG;
    *plan = nullptr;
    if (num_bins == 0 || max_n > (uint64_t)UINT32_MAX) return HIST_ERR_INVALID_ARG;
    hist_status_t st = check_opts(opts);
    if (st != HIST_OK) return st;
    if (num_bins > HIST_MAX_BINS) return HIST_ERR_UNSUPPORTED;
    if (((uintptr_t)workspace & 255u) != 0) return HIST_ERR_INVALID_ARG;
    hist_plan_impl *p = new (std::nothrow) hist_plan_impl();
    if (!p) return HIST_ERR_INVALID_ARG;
    st = query_device(&p->dev);
    if (st == HIST_OK) st = design(p, num_bins, max_n, opts);
    if (st == HIST_OK && p->need > 0 && (!workspace || workspace_bytes < p->need))
        st = HIST_ERR_WORKSPACE;
    if (st != HIST_OK) {
        delete p;
        return st;
    }
    p->ws = static_cast<char *>(workspace);
    p->ws_bytes = workspace_bytes;
    *plan = p;
    return HIST_OK;
}

hist_status_t hist_plan_create(hist_plan_t **plan, uint32_t num_bins, uint64_t max_n,
                               const hist_plan_opts_t *opts, void *workspace,
                               uint64_t workspace_bytes)
{
    return hist_plan(plan, num_bins, max_n, opts, workspace, workspace_bytes);
}

hist_status_t hist_run(hist_plan_t *p, uint32_t *counts, const int32_t *input, uint64_t n,
                       uint32_t num_bins, hipStream_t stream)
{
    return run_impl(p, counts, input, n, num_bins, stream, 0u);
}

hist_status_t hist_run_accumulate(hist_plan_t *p, uint32_t *counts, const int32_t *input,
                                  uint64_t n, uint32_t num_bins, hipStream_t stream)
{
    return run_impl(p, counts, input, n, num_bins, stream, 1u);
}

hist_status_t hist_plan_info(const hist_plan_t *p, hist_plan_info_t *info)
{
    if (!p || !info) return HIST_ERR_INVALID_ARG;
    fill_info(p, info);
    return HIST_OK;
}

hist_status_t hist_plan_preview(const hist_device_desc_t *dev, uint32_t num_bins, uint64_t max_n,
                                const hist_plan_opts_t *opts, hist_plan_info_t *info)
{
    if (!dev || !info || num_bins == 0 || max_n > (uint64_t)UINT32_MAX) return HIST_ERR_INVALID_ARG;
    if (dev->cu_count <= 0 || dev->xcd_count <= 0 || dev->cu_count % dev->xcd_count != 0 ||
        dev->lds_bytes < 65536 || dev->lds_bytes > 163840)
        return HIST_ERR_INVALID_ARG;
    hist_status_t st = check_opts(opts);
    if (st != HIST_OK) return st;
    if (num_bins > HIST_MAX_BINS) return HIST_ERR_UNSUPPORTED;
    hist_plan_impl p;
    p.dev.cu = dev->cu_count;
    p.dev.xcd = dev->xcd_count;
    p.dev.lds = dev->lds_bytes;
    p.dev.sweep_waves_per_simd = dev->sweep_waves_per_simd == 0 ? ~0u : dev->sweep_waves_per_simd;
    st = design(&p, num_bins, max_n, opts);
    if (st != HIST_OK) return st;
    fill_info(&p, info);
    return HIST_OK;
}

}  // extern "C"

namespace {

// " pace=..." for a RANGE plan whose owners do not each read at their own
// pace with all waves counting (empty otherwise, so that the descriptions of
// plans that do not pace stay as they were).
const char *pace_tag(const hist_plan_impl *p)
{
    static thread_local char buf[32];
    if (p->path != HIST_PATH_RANGE || p->pacing <= 1) return "";
    if (p->pacing == 2) return " pace=idle-wave";
    std::snprintf(buf, sizeof buf, " pace=%u", p->pacing - 2);
    return buf;
}

void fill_info(const hist_plan_impl *p, hist_plan_info_t *info)
{
    std::memset(info, 0, sizeof(*info));
    info->path = p->path;
    info->device = p->dev.device;
    info->cu_count = p->dev.cu;
    info->xcd_count = p->dev.xcd;
    info->num_bins = p->num_bins;
    info->range_bins = p->range_bins;
    info->ranges = p->ranges;
    info->groups = p->groups;
    info->wg_size = p->wg;
    info->aggregation = p->agg;
    const bool routed = p->path == HIST_PATH_SCATTER || p->path == HIST_PATH_STREAM;
    info->tile_elems = routed ? kScatterTile : 0;
    info->counter_bits = routed ? 32 : p->cw;
    info->max_n = p->max_n;
    info->workspace_bytes = p->need;
    info->max_group_elems = routed ? 0 : p->max_elems_wg;
    info->event_cap = routed ? 0 : p->cw == 8 ? p->ev_cap + pca::kEvSpill8 : p->ev_cap;
}

}  // namespace

extern "C" {

hist_status_t hist_plan_describe(const hist_plan_t *p, char *buf, uint64_t len)
{
    if (!p || !buf || len == 0) return HIST_ERR_INVALID_ARG;
    static const char *names[] = {"auto", "full", "range", "scatter", "stream"};
    std::snprintf(buf, len,
                  "path=%s bins=%u S=%u R=%u %s=%u cw=%u copies=%u wg=%u agg=%d tile=%u cu=%d xcd=%d "
                  "lds=%u ws=%llu%s%s",
                  names[p->path], p->num_bins, p->range_bins, p->ranges,
                  p->path == HIST_PATH_SCATTER ? "W" : p->path == HIST_PATH_STREAM ? "P" : "G",
                  p->groups, p->path >= HIST_PATH_SCATTER ? 32u : p->cw, 1u << p->kshift, p->wg,
                  p->agg, p->path >= HIST_PATH_SCATTER ? kScatterTile : 0u, p->dev.cu, p->dev.xcd,
                  p->dev.lds, (unsigned long long)p->need, pace_tag(p),
                  p->path != HIST_PATH_SCATTER ? "" : p->window == 1 ? " win=off" : p->window == 2 ? " win=on" : " win=auto");
    return HIST_OK;
}

hist_status_t hist_plan_timing_enable(hist_plan_t *p, uint32_t capacity)
{
    if (!p || capacity > (1u << 16)) return HIST_ERR_INVALID_ARG;
    for (hipEvent_t e : p->ev) (void)hipEventDestroy(e);
    p->ev.clear();
    p->used.clear();
    p->tcap = 0;
    p->truns = 0;
    if (capacity == 0) return HIST_OK;
    p->ev.resize((size_t)capacity * HIST_MAX_PHASES * 2);
    for (auto &e : p->ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            (void)hipGetLastError();
            return HIST_ERR_HIP;
        }
    }
    p->used.assign((size_t)capacity * HIST_MAX_PHASES, 0);
    p->tcap = capacity;
    return HIST_OK;
}

hist_status_t hist_plan_timing_read(hist_plan_t *p, double *ms, uint32_t *launches)
{
    if (!p || !ms || !launches) return HIST_ERR_INVALID_ARG;
    for (int k = 0; k < HIST_MAX_PHASES; ++k) {
        ms[k] = 0.0;
        launches[k] = 0;
    }
    for (uint32_t r = 0; r < p->truns; ++r) {
        for (int k = 0; k < HIST_MAX_PHASES; ++k) {
            if (!p->used[(size_t)r * HIST_MAX_PHASES + k]) continue;
            hipEvent_t a = p->ev[((size_t)r * HIST_MAX_PHASES + k) * 2];
            hipEvent_t b = p->ev[((size_t)r * HIST_MAX_PHASES + k) * 2 + 1];
            float t = 0.f;
            if (hipEventSynchronize(b) != hipSuccess || hipEventElapsedTime(&t, a, b) != hipSuccess)
                return HIST_ERR_HIP;
            ms[k] += t;
            launches[k] += 1;
        }
    }
    p->truns = 0;
    return HIST_OK;
}

const char *hist_plan_phase_name(const hist_plan_t *p, uint32_t phase)
{
    (void)p;
    return phase < HIST_MAX_PHASES ? kPhaseNames[phase] : "";
}

hist_status_t hist_plan_check(hist_plan_t *p, hipStream_t stream, uint32_t *gave_up)
{
    if (!p || !gave_up) return HIST_ERR_INVALID_ARG;
    *gave_up = 0;
    if (p->path != HIST_PATH_STREAM) return HIST_OK;
    const uint32_t *err = reinterpret_cast<const uint32_t *>(p->ws + p->off_ctl) + pca::kCtlError;
    if (hipMemcpyAsync(gave_up, err, 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess) {
        (void)hipGetLastError();
        return HIST_ERR_HIP;
    }
    return HIST_OK;
}

hist_status_t hist_plan_stream_trace(hist_plan_t *p, hipStream_t stream, uint32_t *out,
                                     uint32_t capacity, uint32_t *workgroups)
{
    if (!p || !workgroups || (capacity && !out)) return HIST_ERR_INVALID_ARG;
    *workgroups = 0;
    if (p->path != HIST_PATH_STREAM) return HIST_OK;
    const uint32_t words = p->grid * pca::kStreamTraceWords;
    if (capacity < words) return HIST_ERR_INVALID_ARG;
    if (hipMemcpyAsync(out, p->ws + p->off_trace, (size_t)words * 4, hipMemcpyDeviceToHost, stream) !=
            hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess) {
        (void)hipGetLastError();
        return HIST_ERR_HIP;
    }
    *workgroups = p->grid;
    return HIST_OK;
}

void hist_plan_destroy(hist_plan_t *p)
{
    if (!p) return;
    for (hipEvent_t e : p->ev) (void)hipEventDestroy(e);
    delete p;
}

}  // extern "C"
