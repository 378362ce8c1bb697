"""Host-side planning rules, through hist_plan_preview (no GPU): the path,
counter width, ranges, chunk count and workspace that hist_plan_create would
choose, for an MI355X and for other described devices."""
from __future__ import annotations

import pytest

from partitioned_chip_accumulation_amd import hist

N = 1 << 26  # the path-selection sweep's length


def align(v, a=256):
    return (v + a - 1) // a * a


def partial_bytes(rows, num_bins):
    # plane 0, planes 1..7 and one width byte per 256-bin block, each region
    # 256-byte aligned (the workspace layout include/hist.h documents)
    cells = rows * ((num_bins + 255) // 256)
    return align(cells * 128) + align(cells * 128 * 7) + align(cells)


@pytest.mark.parametrize("num_bins,want", [
    (8192, ("full", 16, 1)), (20480, ("full", 16, 1)), (20481, ("full", 32, 1)),
    (40960, ("full", 32, 1)), (40961, ("full", 16, 1)), (79616, ("full", 16, 1)),
    (79617, ("full", 8, 1)), (155392, ("full", 8, 1)), (155393, ("range", 8, 2)),
    (262144, ("range", 8, 2)), (318464, ("range", 8, 3)), (318465, ("scatter", 32, 10)),
    (1 << 20, ("scatter", 32, 32)), (hist.MAX_BINS, ("scatter", 32, 2048)),
])
def test_auto_thresholds_on_mi355x(num_bins, want):
    i = hist.preview(num_bins, N)
    assert (i.path, i.counter_bits, i.ranges) == want
    assert i.device == -1 and i.cu_count == 256 and i.xcd_count == 8


@pytest.mark.parametrize("num_bins", [1024, 8192, 65536, 100_000, 155_392, 262_144, 300_000])
def test_sweep_plans_fill_the_chip_once(num_bins):
    i = hist.preview(num_bins, N)
    assert i.path in ("full", "range")
    # one resident 1024-thread workgroup per CU (registers), XCD-aligned chunks
    assert i.wg_size == 1024 and i.groups * i.ranges <= 256 and i.groups % 8 == 0
    # the partial rows, and with 8-bit counters each workgroup's 512 spilled
    # carry-event entries
    spill = align(i.groups * i.ranges * 512 * 4) if i.counter_bits == 8 else 0
    assert i.workspace_bytes == partial_bytes(i.groups, num_bins) + spill
    assert i.range_bins % 256 == 0 and i.range_bins * i.ranges >= num_bins


def test_small_inputs_take_few_chunks():
    # the merge of G rows of B counts stays small next to the input: G <= n / B
    i = hist.preview(65536, 1 << 20)
    assert i.groups == 16
    assert hist.preview(8192, 1 << 20).groups == 128
    # one chunk: no partial rows at all, the slice goes straight to the output
    one = hist.preview(65536, 4096)
    assert one.groups == 1 and one.workspace_bytes == 0


@pytest.mark.parametrize("num_bins,max_n", [(100_000, 1 << 26), (155_392, 1 << 30),
                                            (262_144, 1 << 28), (262_144, 2**32 - 1),
                                            (150_000, 2**32 - 1)])
def test_8bit_event_bound(num_bins, max_n):
    i = hist.preview(num_bins, max_n)
    assert i.counter_bits == 8
    # the list takes the LDS the slice leaves, then 512 entries in the
    # workspace; each chunk may log at most cap - 16 events, one per 255
    # counted elements
    assert i.event_cap == (163840 - i.range_bins) // 4 - 4 + 512
    assert i.max_group_elems == 255 * (i.event_cap - 16)
    assert i.groups * i.max_group_elems >= max_n
    slots = 256 // i.ranges // 8 * 8
    if i.groups > slots:
        assert i.groups % slots == 0  # whole rounds of resident chunks


def test_16bit_chunk_limit():
    i = hist.preview(65536, 2**32 - 1)
    assert i.counter_bits == 16 and i.max_group_elems == 1 << 24
    assert i.groups * (1 << 24) >= 2**32 - 1 and i.groups % 256 == 0


def test_scatter_sizes():
    i = hist.preview(1 << 20, 1 << 28)
    tiles = (1 << 28) // 4 // 4096
    assert (i.range_bins, i.ranges, i.groups, i.tile_elems) == (32768, 32, 256, 16384)
    assert i.aggregation == 1
    assert i.workspace_bytes > partial_bytes(256 + 32, 32768) + tiles * 16392 * 2


def scatter_workspace(num_bins, max_n, owners=256, window=True):
    """The SCATTER workspace, region by region, each 256-byte aligned, in the
    plan's order: staged slots, run tables (counts, starts, prefix), range totals,
    segment totals, range starts, from 1,024 ranges a tile-major copy of the
    run starts, W + R partial rows of 32,768-bin slices, then (unless the
    in-place window is off) the pick's words and, per partition workgroup
    (min(tiles, CUs) of them), a row of the window's 8,192 bins and 64
    words more, the first of which holds the hot value's total."""
    R = -(-num_bins // 32768)
    T = max(1, -(-(max_n // 4) // 4096))
    b = align(T * 16392 * 2) + 3 * align(R * T * 4) + align(R * 4)
    b += align(R * -(-T // 4096) * 4) + align((R + 1) * 8)
    if R >= 1024:
        b += align(R * T * 4)
    b += partial_bytes(owners + R, 32768)
    if window:
        b += 256 + align(min(T, 256) * (hist.WINDOW_BINS + 64) * 4)
    return b


@pytest.mark.parametrize("num_bins,max_n", [
    (318_465, N), (1 << 20, 1 << 28), (524_288, 1 << 29), ((1 << 24) - 5, 2_000_000),
    (1023 * 32768, N), (1024 * 32768, N), (1024 * 32768 + 1, 1 << 20), (hist.MAX_BINS, N),
    (hist.MAX_BINS, 5), (1 << 21, 2**32 - 1),
])
def test_scatter_workspace_layout(num_bins, max_n):
    i = hist.preview(num_bins, max_n, path="scatter")
    assert i.ranges == -(-num_bins // 32768)
    assert i.workspace_bytes == scatter_workspace(num_bins, max_n)
    for w, on in ((1, False), (2, True)):
        assert hist.preview(num_bins, max_n, path="scatter", window=w).workspace_bytes == \
            scatter_workspace(num_bins, max_n, window=on)


def test_window_option_is_checked():
    for bad in (-1, 3):
        with pytest.raises(hist.HistError) as e:
            hist.preview(1 << 20, N, path="scatter", window=bad)
        assert e.value.status == hist.HIST_ERR_INVALID_ARG


def test_forced_options():
    assert hist.preview(8192, N, path="scatter").path == "scatter"
    r = hist.preview(100_000, N, path="range", range_bins=4096)
    assert (r.range_bins, r.ranges, r.counter_bits) == (4096, 25, 32)
    assert hist.preview(65536, N, counter_bits=8).counter_bits == 8
    assert hist.preview(8192, N, wg_size=512).wg_size == 512
    with pytest.raises(hist.HistError) as e:
        hist.preview(200_000, N, path="full")  # more bins than one workgroup holds
    assert e.value.status == hist.HIST_ERR_UNSUPPORTED


def test_smaller_device():
    # half the CUs and 64 KiB of LDS: every capacity threshold moves down
    d = hist.DeviceDesc(128, 4, 65536, 6)
    assert hist.preview(30000, N, device=d).path == "full"
    assert hist.preview(30000, N, device=d).counter_bits == 16
    assert hist.preview(40000, N, device=d).counter_bits == 8
    assert hist.preview(61000, N, device=d).path == "range"
    i = hist.preview(8192, N, device=d)
    assert i.cu_count == 128 and i.groups * i.ranges <= 128


def test_no_register_limit_means_lds_bound_residency():
    # with registers unlimited, small slices run two 1024-thread workgroups per CU
    free = hist.DeviceDesc(256, 8, 163840, 0)
    assert hist.preview(8192, N, device=free).groups == 512
    assert hist.preview(8192, N).groups == 256


@pytest.mark.parametrize("desc", [(0, 8, 163840, 6), (256, 0, 163840, 6), (256, 3, 163840, 6),
                                  (256, 8, 32768, 6), (256, 8, 200000, 6)])
def test_bad_device_descriptions(desc):
    with pytest.raises(hist.HistError) as e:
        hist.preview(8192, N, device=hist.DeviceDesc(*desc))
    assert e.value.status == hist.HIST_ERR_INVALID_ARG


def test_bad_arguments():
    lib = hist.library()
    i = hist.PlanInfo()
    import ctypes
    d = hist.mi355x()
    assert lib.hist_plan_preview(None, 8, 8, None, ctypes.byref(i)) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_plan_preview(ctypes.byref(d), 8, 8, None, None) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_plan_preview(ctypes.byref(d), 0, 8, None, ctypes.byref(i)) == \
        hist.HIST_ERR_INVALID_ARG
    assert lib.hist_plan_preview(ctypes.byref(d), 8, 2**32, None, ctypes.byref(i)) == \
        hist.HIST_ERR_INVALID_ARG
    assert lib.hist_plan_preview(ctypes.byref(d), hist.MAX_BINS + 1, 8, None,
                                 ctypes.byref(i)) == hist.HIST_ERR_UNSUPPORTED
