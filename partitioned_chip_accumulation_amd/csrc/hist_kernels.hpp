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
// Slices are merged by exclusive owners (k_merge, k_merge_slots; on the
// two-phase path an owner that holds a whole range writes it itself): one
// thread writes (or, when accumulating, reads and writes) each output bin
// once, so no global atomics and no memset of the output are needed.
//
// Conventions: wave64 (gfx950), 16-byte (dwordx4) global loads on the input
// body; LDS counters are uint32 (ds_add_u32), or two 16-bit halves or four
// bytes of a word kept exact by carry events (ds_add_rtn_u32).
//
// The kernels live in one header per stage:
//   hist_common.hpp      input view, wave and LDS helpers, the hot slot
//   hist_counters16.hpp  16-bit LDS counters with carry events
//   hist_counters8.hpp   8-bit LDS counters with carry events
//   hist_partials.hpp    partial-slice layout, flush and exclusive-owner merge
//   hist_sweep.hpp       the single-pass sweep (FULL, RANGE)
//   hist_scatter.hpp     the two-phase path (SCATTER)
//   hist_stream.hpp      the streaming owner-queue path (STREAM)
#pragma once

#include "hist_common.hpp"
#include "hist_counters16.hpp"
#include "hist_counters8.hpp"
#include "hist_partials.hpp"
#include "hist_sweep.hpp"
#include "hist_scatter.hpp"
#include "hist_stream.hpp"
