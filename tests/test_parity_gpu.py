"""GPU parity: the HIP path against the CPU oracle, bit for bit.

Histogram counts are integers and every schedule reaches the same counts
(page "Distributed Shared Memory", section "The cluster histogram": each
element adds exactly one to its bin, slices are summed), so the bar is exact
equality for every bin, with no tolerance. All calls go through the C ABI via
the binding; the oracle runs on the host over the same bytes.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from partitioned_chip_accumulation_amd import hist, inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(DEV)
    yield


def check(x: np.ndarray, num_bins: int, label: str, offset: int = 0, **opts):
    """Run one plan over x (placed `offset` elements into a device buffer, to
    exercise misaligned starts) and compare with the oracle."""
    ref, dropped = oracle.hist(x, num_bins)
    say(f"case {label}: n={x.size} bins={num_bins} offset={offset} opts={opts}")
    buf = torch.empty(x.size + offset + 4, dtype=torch.int32, device=DEV)
    buf.fill_(-1)
    xt = buf[offset:offset + x.size]
    xt.copy_(torch.from_numpy(x))
    plan = hist.Plan(num_bins, max(1, x.size), device=DEV, **opts)
    got = plan.run(xt).cpu().numpy()
    torch.cuda.synchronize(DEV)
    if not np.array_equal(got, ref):
        bad = np.flatnonzero(got != ref)
        raise AssertionError(f"{label} ({plan.describe()}): {bad.size} bins differ, first "
                             f"{bad[:5].tolist()} got {got[bad[:5]].tolist()} "
                             f"want {ref[bad[:5]].tolist()}")
    assert int(got.astype(np.int64).sum()) + dropped == x.size
    plan.close()


def rnd(seed, n, lo, hi):
    return np.random.default_rng(seed).integers(lo, hi, size=n, dtype=np.int64).astype(np.int32)


# --- small and ragged ------------------------------------------------------

PATH_CASES = [
    ("full", {}),
    ("full-agg2", {"aggregation": 2}),
    ("range", {"path": "range", "range_bins": 2048}),
    ("range-agg4", {"path": "range", "range_bins": 1024, "aggregation": 4}),
    ("full-cw16", {"counter_bits": 16}),
    ("full-cw16-agg2", {"counter_bits": 16, "aggregation": 2}),
    ("full-cw16-hot", {"counter_bits": 16, "aggregation": 1}),
    ("full-hot", {"aggregation": 1}),
    ("scatter-hot", {"path": "scatter", "aggregation": 1}),
    ("full-copies1", {"lds_copies": 1}),
    ("full-copies2", {"lds_copies": 2}),
    ("full-copies4-hot", {"lds_copies": 4, "aggregation": 1}),
    ("full-copies4-agg2", {"lds_copies": 4, "aggregation": 2}),
    ("range-copies8", {"path": "range", "range_bins": 2048, "lds_copies": 8}),
    ("range-cw16", {"path": "range", "range_bins": 2048, "counter_bits": 16}),
    ("full-cw8", {"counter_bits": 8}),
    ("full-cw8-agg2", {"counter_bits": 8, "aggregation": 2}),
    ("full-cw8-hot", {"counter_bits": 8, "aggregation": 1}),
    ("range-cw8", {"path": "range", "range_bins": 2048, "counter_bits": 8}),
    ("range-cw8-wg256", {"path": "range", "range_bins": 1024, "counter_bits": 8, "wg_size": 256}),
    ("scatter", {"path": "scatter"}),
    ("scatter-agg1", {"path": "scatter", "aggregation": 1}),
]


@pytest.mark.parametrize("label,opts", PATH_CASES, ids=[c[0] for c in PATH_CASES])
def test_small_uniform_every_path(label, opts):
    x = inputs.generate(1, n=1_000_003)  # several tiles and chunks, ragged tail
    check(x, 8192, label, **opts)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("path", ["auto", "range", "scatter"])
def test_small_workloads(cfg, path):
    w = inputs.WORKLOADS[cfg]
    x = inputs.generate(cfg, n=(1 << 20) + 12345)
    opts = {"path": path}
    if path == "range" and w.num_bins <= 40960:
        opts["range_bins"] = 4096
    check(x, w.num_bins, f"wl{cfg}-{path}", **opts)


@pytest.mark.parametrize("n", [0, 1, 2, 3, 4, 5, 7, 63, 64, 65, 1023, 16383, 16384, 16385,
                               16384 * 3 + 5, 262_147])
@pytest.mark.parametrize("offset", [0, 1, 3])
def test_lengths_and_alignment(n, offset):
    x = rnd(n + offset, n, -2, 70_000)
    for opts in ({}, {"path": "range"}, {"path": "scatter"}):
        check(x, 65536, f"len{n}", offset=offset, **opts)


@pytest.mark.parametrize("num_bins", [1, 2, 3, 5, 255, 4095, 8191, 8193, 32767, 32768, 32769,
                                      40703, 40704, 40705, 40960, 65535, 65537, 79616, 79617,
                                      100_003, 155_391, 155_392, 155_393, 262_145])
def test_bin_counts(num_bins):
    x = rnd(num_bins, 300_007, -3, num_bins + 5)
    paths = ["auto", "scatter"]
    if num_bins <= 155_392:
        paths.append("full")
    if num_bins > 8:
        paths.append("range")
    for p in paths:
        check(x, num_bins, f"bins{num_bins}-{p}", path=p)


@pytest.mark.parametrize("num_bins", [hist.MAX_BINS, hist.MAX_BINS - 1])
def test_maximum_bin_count(num_bins):
    """The largest supported bin count: 2,048 two-phase ranges (the partition's
    rank counters and the owners' range table at their LDS limits), a ragged
    last range, and the RANGE path with one chunk per range."""
    x = rnd(77, 1_000_003, -3, num_bins + 5)
    x[:1000] = num_bins - 1  # the last bin, in the last (ragged) range
    for p in ["auto", "scatter", "range"]:
        check(x, num_bins, f"maxbins{num_bins}-{p}", path=p)


def test_out_of_range_and_negative_values():
    x = rnd(5, 500_000, -(2**31), 2**31 - 1)
    x[::2] = rnd(6, x[::2].size, 0, 70_000)
    for p in ["auto", "range", "scatter"]:
        check(x, 70_000, f"oor-{p}", path=p)


@pytest.mark.parametrize("b", [0, 32767, 32768, 65535])
def test_all_one_bin(b):
    x = np.full(1 << 22, b, np.int32)
    for p, agg in [("range", 0), ("range", 1), ("range", 2), ("scatter", 0), ("scatter", 1),
                   ("scatter", 4), ("full", 1), ("full", 2)]:
        check(x, 65536, f"one{b}-{p}-agg{agg}", path=p, aggregation=agg)


@pytest.mark.parametrize("path,bins,groups", [("full", 150_000, 1), ("full", 150_000, 3),
                                              ("range", 262_144, 2)])
def test_counter8_identical_events_in_a_window(path, bins, groups):
    """8-bit counters with the input piled onto one bin (and a second bin in
    the same word): every window of the event list holds up to 64 copies of
    the same entry, which the flush applies together (+256 m, -m), and the
    neighbouring byte takes the cascades."""
    n = 3_000_000
    b = bins - 6  # byte 2 of its word: its carries cascade into byte 3 (bin b + 1)
    x = np.full(n, b, np.int32)
    x[::7] = b + 1
    x[::1001] = 5
    check(x, bins, f"identical-events-{path}-g{groups}", path=path, counter_bits=8, groups=groups)


@pytest.mark.parametrize("agg", [0, 1])
@pytest.mark.parametrize("path,bins", [("full", 150_000), ("range", 262_144)])
def test_counter8_carry_chains(agg, path, bins):
    """8-bit counters, one chunk: words whose bytes above the first one end
    one short of a wrap (255 adds each) while the first byte wraps once
    (256 adds). Whichever add comes last decides where the carries start:
    when the first byte's wrap comes after the others' adds it carries
    through every byte above it, out of the word's top byte, in one add. The
    chains start at byte 0, 1 and 2 in different words."""
    words = np.arange(37, 37 + 3 * 1400, 3, dtype=np.int64) % (bins // 4)
    adds = {0: [256, 255, 255, 255], 1: [0, 256, 255, 255], 2: [0, 0, 256, 255]}
    parts = []
    for k, w in enumerate(words):
        for q, c in enumerate(adds[k % 3]):
            parts.append(np.full(c, 4 * w + q, np.int64))
    parts.append(rnd(12, 100_000, 0, bins).astype(np.int64))
    x = np.concatenate(parts)
    x = x[np.random.default_rng(13 + agg).permutation(x.size)].astype(np.int32)
    check(x, bins, f"cw8-chains-{path}-agg{agg}", path=path, counter_bits=8, groups=1,
          aggregation=agg, **({"range_bins": 131_072} if path == "range" else {}))


@pytest.mark.parametrize("agg", [0, 1, 4])
@pytest.mark.parametrize("path,bins", [("full", 65536), ("range", 200_000)])
def test_counter16_carry_events(agg, path, bins):
    # Few chunks and many copies of a few bins: every chunk's 16-bit counters
    # wrap several times, in the low half (even bins) and the high half (odd
    # bins) of a word, and both halves of one word together.
    rng = np.random.default_rng(agg)
    hot = np.array([4, 5, 7, 65534, 65535, bins - 1], np.int32)
    x = np.concatenate([np.repeat(hot, [400_003, 300_007, 150_001, 350_000, 199_999, 70_000]),
                        rnd(9, 500_000, 0, bins)])
    x = x[rng.permutation(x.size)].astype(np.int32)
    check(x, bins, f"cw16-{path}-agg{agg}", path=path, counter_bits=16, groups=3,
          aggregation=agg)


@pytest.mark.parametrize("agg", [0, 1, 2, 4])
@pytest.mark.parametrize("path,bins,groups", [("full", 150_000, 3), ("full", 155_392, 1),
                                              ("range", 400_000, 2), ("full", 4099, 1)])
def test_counter8_carry_events(agg, path, bins, groups):
    # Few chunks and many copies of a few bins: every chunk's 8-bit counters
    # carry many times, out of every byte of a word (4..7 share a word, so
    # their carries cascade), out of the word's top byte (11), and in the
    # last, ragged word of the slice. groups=1 takes the direct write.
    rng = np.random.default_rng(agg)
    hot = np.array([4, 5, 6, 7, 8, 11, bins - 1], np.int32)
    reps = [40_001, 30_007, 25_000, 20_003, 1_000, 9_999, 7_000]
    x = np.concatenate([np.repeat(hot, reps), rnd(9, 300_000, 0, bins)])
    x = x[rng.permutation(x.size)].astype(np.int32)
    check(x, bins, f"cw8-{path}-agg{agg}-g{groups}", path=path, counter_bits=8, groups=groups,
          aggregation=agg, **({"range_bins": 131_072} if path == "range" else {}))


@pytest.mark.parametrize("wg", [256, 512])
@pytest.mark.parametrize("path,bins,groups", [("full", 150_000, 3), ("full", 4099, 1),
                                              ("range", 300_000, 2)])
def test_counter8_carry_events_smaller_workgroups(wg, path, bins, groups):
    # The flush gives each wave four pairs of blocks spaced by the wave count
    # (4 or 8 here), so events in adjacent pairs go to different waves; hot
    # bins in adjacent blocks (0-7, 256-263, 512-515) and a run of 3,000 bins
    # with a few hundred copies each put events in many adjacent pairs.
    rng = np.random.default_rng(wg)
    hot = np.array([0, 1, 2, 3, 4, 5, 6, 7, 256, 263, 512, 515, bins - 1], np.int32)
    run = np.repeat(np.arange(1000, 4000, dtype=np.int32) % bins, 300)
    x = np.concatenate([np.repeat(hot, 20_000), run, rnd(10, 200_000, 0, bins)])
    x = x[rng.permutation(x.size)].astype(np.int32)
    check(x, bins, f"cw8-wg{wg}-{path}-g{groups}", path=path, counter_bits=8, groups=groups,
          wg_size=wg, **({"range_bins": 150_016} if path == "range" else {}))


@pytest.mark.parametrize("wg,groups", [(1024, 2), (512, 3), (256, 2), (1024, 1), (256, 1)])
def test_counter8_every_leaf_of_the_event_application(wg, groups):
    """8-bit counters: carries out of every count a lane holds at the flush.
    A wave's flush takes four pairs of 256-bin blocks spaced by the wave count
    (pairs w, w + NW, w + 2 NW, w + 3 NW for wave w), and a lane holds 8
    counts (two words) of each: 32 counts, each reached by its own leaf of the
    event application. Here every one of those counts, for one lane of every
    wave, gets at least 256 copies in every chunk, so every leaf applies
    events, with carries out of byte 3 and cascades into the next byte. One
    chunk takes the direct write, whose application covers one pair (8
    leaves) at a time."""
    nw = wg // 64
    bins = 512 * 4 * nw
    hot = []
    for w in range(nw):
        lane = (7 * w + 3) % 64
        for j in range(4):
            for i in range(8):
                hot.append(512 * (w + j * nw) + 8 * lane + i)
    copies = 300 * groups + 100  # >= 256 in every chunk of the shuffled input
    x = np.concatenate([np.repeat(np.array(hot, np.int32), copies), rnd(11, 50_000, 0, bins)])
    x = x[np.random.default_rng(wg + groups).permutation(x.size)].astype(np.int32)
    check(x, bins, f"cw8-leaves-wg{wg}-g{groups}", path="full", counter_bits=8, groups=groups,
          wg_size=wg)


@pytest.mark.parametrize("agg", [0, 1])
@pytest.mark.parametrize("groups", [2, 16])
def test_zipf_workload_shape_on_8bit_ranges(agg, groups):
    """The Zipf 262,144-bin workload's recipe at 2^22 elements on its AUTO
    schedule's kind (8-bit counters, two ranges): hot bytes wrap every 256
    counts, so the carry events and their application run at scale, in well
    under the full size's time."""
    x = inputs.generate(3, n=1 << 22)
    check(x, 262_144, f"zipf-2^22-range8-agg{agg}-g{groups}", path="range", counter_bits=8,
          groups=groups, aggregation=agg)


@pytest.mark.parametrize("pacing", [1, 2, 3, 4, 10])
@pytest.mark.parametrize("shape", ["zipf-2^22", "uniform-2-ranges", "many-chunks-3-ranges"])
def test_range_owner_pacing(pacing, shape):
    """RANGE with the owners of a chunk reading non-temporally (1), with plain
    loads (2), or paced against each other within 1, 2 or 8 batches (3, 4,
    10). The counts must not depend on it: every owner counts what it loads.
    Three ranges pace in a ring; 1,024 chunks put co-owners in different
    rounds of resident workgroups, so some waits give up. Values outside the
    bins (negative ones here) are skipped as always."""
    if shape == "zipf-2^22":
        x, bins, opts = inputs.generate(3, n=1 << 22), 262_144, {"counter_bits": 8, "groups": 16}
    elif shape == "uniform-2-ranges":
        x, bins, opts = rnd(31, (1 << 22) + 5, -3, 300_000), 300_000, {"counter_bits": 8,
                                                                        "groups": 8}
    else:
        x, bins, opts = rnd(32, 1 << 23, 0, 200_000), 200_000, {"counter_bits": 16,
                                                                 "groups": 1024}
    check(x, bins, f"pacing{pacing}-{shape}", path="range", pacing=pacing, **opts)


@pytest.mark.parametrize("case,bins", [("one-bin-at-the-limit", 155_392),
                                       ("one-bin-at-the-limit", 100_000),
                                       ("one-bin-past-the-limit", 155_392),
                                       ("every-bin-near-255", 2048)])
def test_counter8_event_list_bound(case, bins):
    """The carry-event list at its bound: one workgroup (groups=1) counting
    the most elements the plan lets one chunk hold, all in one bin, logs about
    n / 255 events, close to the list's capacity (the LDS its slice leaves:
    the minimum at 155,392 bins, much more at 100,000); one element more and
    the plan splits the input. With every bin near 255 copies the events
    spread over the whole slice."""
    probe = hist.Plan(bins, 1, device=DEV, path="full", counter_bits=8, groups=1)
    info = probe.info()
    probe.close()
    limit = info.max_group_elems
    assert limit == 255 * (info.event_cap - 16) and info.event_cap >= 2048
    if case == "every-bin-near-255":
        x = np.repeat(np.arange(bins, dtype=np.int32), limit // bins)
        x = x[np.random.default_rng(5).permutation(x.size)]
    else:
        x = np.full(limit + (case == "one-bin-past-the-limit"), bins - 2, np.int32)
    for agg in (0, 1):
        check(x, bins, f"cw8-bound-{case}-agg{agg}", path="full", counter_bits=8, groups=1,
              aggregation=agg)


@pytest.mark.parametrize("bins", [100_000, 155_392])
def test_counter8_event_spill_in_partial_rows(bins):
    """Two chunks, each at the list's bound and all in one bin: each
    workgroup logs past its LDS list into its spill area in the workspace,
    and the partial-row flush applies both parts (the bound test above covers
    the direct write of one chunk)."""
    probe = hist.Plan(bins, 1, device=DEV, path="full", counter_bits=8, groups=2)
    info = probe.info()
    probe.close()
    limit = info.max_group_elems
    assert limit == 255 * (info.event_cap - 16) and info.event_cap > 512
    x = np.full(2 * limit, bins - 3, np.int32)
    x[::97] = 7
    for agg in (0, 1):
        check(x, bins, f"cw8-spill-{bins}-agg{agg}", path="full", counter_bits=8, groups=2,
              aggregation=agg)


AUTO_CASES = [  # bin count -> (path, counter bits, ranges) the measured thresholds give
    (8192, ("full", 16, 1)), (20480, ("full", 16, 1)), (20481, ("full", 32, 1)),
    (40960, ("full", 32, 1)), (40961, ("full", 16, 1)), (79616, ("full", 16, 1)),
    (79617, ("full", 8, 1)), (155392, ("full", 8, 1)), (155393, ("range", 8, 2)),
    (262144, ("range", 8, 2)), (318464, ("range", 8, 3)), (318465, ("scatter", 32, 10)),
    (1 << 20, ("scatter", 32, 32)),
]


@pytest.mark.parametrize("num_bins,want", AUTO_CASES, ids=[str(c[0]) for c in AUTO_CASES])
def test_auto_plan_follows_the_measured_thresholds(num_bins, want):
    """AUTO's path, counter width and range count at each threshold of the
    path-selection sweep, for 2^26 elements (the sweep's n)."""
    info = hist.Plan(num_bins, 1 << 26, device=DEV).info()
    assert (info.path, info.counter_bits, info.ranges) == want, info
    if info.path != "scatter":
        # one round of resident sweep workgroups
        assert info.groups * info.ranges <= info.cu_count * 2


@pytest.mark.parametrize("num_bins,max_n", [(1024, 1 << 26), (8192, 1 << 20), (65536, 1 << 26),
                                            (100_000, 1 << 26), (262_144, 1 << 28),
                                            (1 << 20, 1 << 28), (524_288, 1 << 29),
                                            (262_144, 2**32 - 1)])
def test_preview_matches_the_device_plan(num_bins, max_n):
    """hist_plan_preview with the MI355X description gives the plan that
    hist_plan_create makes on the device (the runtime's occupancy for the
    1024-thread sweeps is one workgroup per CU, as 6 waves per SIMD say)."""
    dev = hist.Plan(num_bins, max_n, device=DEV).info()
    pre = hist.preview(num_bins, max_n)
    assert dev.cu_count == 256 and dev.xcd_count == 8
    assert {**pre.__dict__, "device": dev.device} == dev.__dict__


@pytest.mark.parametrize("num_bins,opts", [(155_392, {}), (262_144, {}), (65_536, {}),
                                           (100_000, {"counter_bits": 8, "path": "full"})])
def test_plan_at_the_largest_n(num_bins, opts):
    """At n = 2^32 - 1 the carry-event bound sets the chunk count: whole rounds
    of resident workgroups, each chunk within the per-chunk limit, and a
    workspace that holds every chunk's partial row."""
    n = 2**32 - 1
    info = hist.Plan(num_bins, 1 << 20, device=DEV, **opts).info()  # small: rounds for n
    big = hist.Plan(num_bins, n, device=DEV, **opts).info()
    assert big.path == info.path and big.counter_bits == info.counter_bits
    assert big.groups * big.max_group_elems >= n
    if big.groups > info.groups:  # rounded up to whole rounds of the resident chunks
        resident = info.cu_count // big.ranges
        assert big.groups % (resident // info.xcd_count * info.xcd_count) == 0
    assert big.workspace_bytes >= big.groups * ((num_bins + 255) // 256) * 128


def test_groups_and_wg_sizes():
    x = inputs.generate(2, n=(1 << 21) + 7)
    for opts in [{"groups": 1}, {"groups": 3}, {"groups": 8}, {"groups": 256},
                 {"counter_bits": 32, "path": "range"}, {"counter_bits": 16, "groups": 1},
                 {"counter_bits": 16, "groups": 5, "wg_size": 256},
                 {"wg_size": 256}, {"wg_size": 512}, {"xcd_map": 2},
                 {"path": "scatter", "groups": 1}, {"path": "scatter", "groups": 7},
                 {"path": "scatter", "groups": 1000}]:
        check(x, 65536, f"opts{opts}", **opts)


def test_misaligned_output_buffer():
    x = inputs.generate(2, n=1 << 20)
    ref, _ = oracle.hist(x, 65536)
    plan = hist.Plan(65536, x.size, device=DEV)
    out = torch.empty(65536 + 1, dtype=torch.int32, device=DEV)
    got = plan.run(torch.from_numpy(x).to(DEV), out[1:]).cpu().numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("offset", [0, 1, 3])
def test_owner_written_ranges_at_any_output_alignment(offset):
    """With more ranges than owners the owners write most ranges' counts
    themselves, 16 bytes at a time when the range starts 16-byte aligned and
    word by word otherwise; run and accumulate, on outputs 0, 4 and 12 bytes
    past an aligned base."""
    bins = (1 << 24) + 1000
    x = rnd(41, 1_500_001, -2, bins + 2)
    ref, _ = oracle.hist(x, bins)
    xt = torch.from_numpy(x).to(DEV)
    plan = hist.Plan(bins, x.size, device=DEV, path="scatter")
    base = torch.zeros(bins + 3, dtype=torch.int32, device=DEV)
    out = base[offset:offset + bins]
    got = plan.run(xt, out).cpu().numpy()
    assert np.array_equal(got, ref)
    plan.run(xt, out, accumulate=True)
    got2 = out.cpu().numpy().view(np.uint32)
    torch.cuda.synchronize(DEV)
    assert np.array_equal(got2, (2 * ref.astype(np.uint64)).astype(np.uint32))
    plan.close()


def test_argument_errors_on_device():
    plan = hist.Plan(1000, 100, device=DEV)
    # every buffer is large enough for any call below, so a missed check
    # could not write out of bounds
    x = torch.zeros(2000, dtype=torch.int32, device=DEV)[:101]
    with pytest.raises(hist.HistError) as e:
        plan.run(x)  # n > max_n
    assert e.value.status == hist.HIST_ERR_INVALID_ARG
    lib = hist.library()
    out = torch.empty(1000, dtype=torch.int32, device=DEV)
    s = torch.cuda.current_stream(DEV).cuda_stream
    assert lib.hist_run(plan._plan, out.data_ptr(), x.data_ptr(), 10, 999, s) == \
        hist.HIST_ERR_INVALID_ARG  # num_bins differs from the plan
    assert lib.hist_run(plan._plan, out.data_ptr(), x.data_ptr() + 2, 10, 1000, s) == \
        hist.HIST_ERR_INVALID_ARG  # misaligned input
    assert lib.hist_run(plan._plan, x.data_ptr(), x.data_ptr(), 10, 1000, s) == \
        hist.HIST_ERR_INVALID_ARG  # output overlaps input
    small = hist.PlanOpts()
    small.aggregation = -1
    p = __import__("ctypes").c_void_p()
    big = hist.workspace_size(65536, 1 << 24)
    assert big > 0
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    assert lib.hist_plan_create(__import__("ctypes").byref(p), 65536, 1 << 24, None,
                                ws.data_ptr(), 16) == hist.HIST_ERR_WORKSPACE


def test_repeat_is_idempotent():
    x = torch.from_numpy(inputs.generate(3, n=1 << 22)).to(DEV)
    plan = hist.Plan(262_144, x.numel(), device=DEV)
    first = plan.run(x).clone()
    for _ in range(20):
        assert torch.equal(plan.run(x), first)


ACC_CASES = [
    ("direct-one-chunk", 4096, 6000, {"path": "full"}),
    ("full-cw32", 8192, 400_000, {}),
    ("full-cw16", 65536, 1_000_000, {}),
    ("full-cw8", 150_000, 1_000_000, {"path": "full"}),
    ("direct-cw8", 150_000, 400_000, {"path": "full", "groups": 1}),
    ("range", 200_000, 2_000_000, {"path": "range"}),
    ("scatter-hot", 300_000, 1_000_000, {"path": "scatter", "aggregation": 1}),
    # 512 ranges over 256 owners: most ranges have one owner, which adds its
    # counts itself; the ranges between owners go through the slot merge
    ("scatter-whole-ranges", (1 << 24) - 5, 2_000_000, {"path": "scatter"}),
]


@pytest.mark.parametrize("label,num_bins,n,opts", ACC_CASES, ids=[c[0] for c in ACC_CASES])
def test_accumulate_over_chunks(label, num_bins, n, opts):
    """hist_run_accumulate over ragged pieces (one of them empty) adds the
    whole input's histogram to what counts held, modulo 2^32."""
    x = rnd(31, n, -5, num_bins + 5)
    ref, _ = oracle.hist(x, num_bins)
    prefill = np.random.default_rng(32).integers(0, 2**32, size=num_bins,
                                                 dtype=np.uint64).astype(np.uint32)
    prefill[:3] = [0xFFFFFFFF, 0xFFFFFFF0, 0]  # wraps
    want = ((prefill.astype(np.uint64) + ref.astype(np.uint64)) % 2**32).astype(np.uint32)
    say(f"case accumulate {label}: n={n} bins={num_bins} opts={opts}")
    xt = torch.from_numpy(x).to(DEV)
    out = torch.from_numpy(prefill.view(np.int32).copy()).to(DEV)
    plan = hist.Plan(num_bins, n, device=DEV, **opts)
    cuts = [0, n // 3, n // 3, n // 3 + 1, 2 * n // 3 + 5, n]
    for a, b in zip(cuts[:-1], cuts[1:]):
        plan.run(xt[a:b], out=out, accumulate=True)
    got = out.cpu().numpy().view(np.uint32)
    torch.cuda.synchronize(DEV)
    assert np.array_equal(got, want), f"{label} ({plan.describe()}): {np.sum(got != want)} bins differ"
    plan.close()


@pytest.mark.parametrize("path", ["full", "range", "scatter"])
def test_run_then_accumulate(path):
    """An overwrite of the first piece followed by accumulation of the rest
    gives the histogram of the whole input, whatever counts held before."""
    num_bins, n = (60_000 if path == "full" else 100_000), 700_001
    x = rnd(33, n, 0, num_bins)
    ref, _ = oracle.hist(x, num_bins)
    say(f"case run-then-accumulate: path={path}")
    xt = torch.from_numpy(x).to(DEV)
    out = torch.full((num_bins,), 12345, dtype=torch.int32, device=DEV)
    plan = hist.Plan(num_bins, n, device=DEV, path=path,
                     range_bins=32768 if path == "range" else 0)
    plan.run(xt[:250_000], out=out)
    plan.run(xt[250_000:], out=out, accumulate=True)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref)
    plan.close()


def test_accumulate_needs_an_output():
    plan = hist.Plan(1024, 100, device=DEV)
    with pytest.raises(ValueError):
        plan.run(torch.zeros(10, dtype=torch.int32, device=DEV), accumulate=True)
    plan.close()


@pytest.mark.parametrize("rtn", [False, True])
def test_lds_atomic_calibration_kernel(rtn):
    """The calibration kernel does its adds: word 0 is hit by lane 0 of each
    of the 16 waves per iteration when the lanes' words are distinct, and by
    all 1024 threads when every lane adds to one word."""
    cu = torch.cuda.get_device_properties(DEV).multi_processor_count
    sink = torch.zeros(cu, dtype=torch.int32, device=DEV)
    iters = 7
    hist.lds_atomic("distinct", rtn, iters, sink)
    got = sink.cpu().numpy()
    if not rtn:
        assert (got == 16 * iters).all()
    hist.lds_atomic("same", False, iters, sink)
    assert (sink.cpu().numpy() == 1024 * iters).all()
    with pytest.raises(hist.HistError):
        hist.lds_atomic("same", False, iters, sink[:cu - 1])


@pytest.mark.parametrize("path,num_bins", [("full", 65536), ("range", 200_000),
                                           ("scatter", 300_000)])
def test_graph_capture_and_replay(path, num_bins):
    """hist_run queues kernels only (no memset, no synchronisation), so a
    caller can capture it in a graph. Each replay histograms whatever the
    captured input buffer holds then; between replays the test does eager
    work of its own (refilling the buffer) and synchronises."""
    n = 1_000_003
    say(f"case graph: path={path} bins={num_bins}")
    plan = hist.Plan(num_bins, n, device=DEV, path=path)
    xt = torch.empty(n, dtype=torch.int32, device=DEV)
    out = torch.empty(num_bins, dtype=torch.int32, device=DEV)
    xt.copy_(torch.from_numpy(rnd(40, n, 0, num_bins)))
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        plan.run(xt, out)  # warm-up on the capture stream (sets kernel attributes)
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize(DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.run(xt, out)
    for k in range(4):
        x = rnd(41 + k, n, -2, num_bins + 2)
        xt.copy_(torch.from_numpy(x))
        out.fill_(-1)
        torch.cuda.synchronize(DEV)
        graph.replay()
        torch.cuda.synchronize(DEV)
        ref, _ = oracle.hist(x, num_bins)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref), f"replay {k}"
    del graph
    plan.close()


def test_timing_records_phases():
    x = torch.from_numpy(inputs.generate(2, n=1 << 22)).to(DEV)
    plan = hist.Plan(65536, x.numel(), device=DEV)
    plan.timing_enable(8)
    for _ in range(5):
        plan.run(x)
    ph = plan.timing_read()
    assert ph["sweep"][1] == 5 and ph["sweep"][0] > 0
    plan = hist.Plan(1 << 20, x.numel(), device=DEV, path="scatter")
    plan.timing_enable(8)
    plan.run(x)
    assert set(plan.timing_read()) == {"partition", "range_scan", "owner_hist", "slot_merge"}


def test_global_atomic_comparator():
    x = inputs.generate(4, n=1 << 21)
    ref, _ = oracle.hist(x, 1 << 20)
    got = hist.global_atomic(torch.from_numpy(x).to(DEV), 1 << 20).cpu().numpy()
    assert np.array_equal(got, ref)


# --- the published sizes ---------------------------------------------------

_full_cache = {}


def full(cfg):
    if cfg not in _full_cache:
        _full_cache.clear()
        w = inputs.WORKLOADS[cfg]
        say(f"generating workload {cfg} ({w.n} elements)")
        x = inputs.generate(cfg)
        ref, dropped = oracle.hist(x, w.num_bins)
        _full_cache[cfg] = (x, ref, dropped, torch.from_numpy(x).to(DEV))
    return _full_cache[cfg]


FULL_CASES = [
    (1, {}), (1, {"aggregation": 2}), (1, {"path": "scatter"}),
    (2, {}), (2, {"aggregation": 1}), (2, {"path": "scatter"}),
    (3, {}), (3, {"aggregation": 4}), (3, {"path": "scatter", "aggregation": 2}),
    (4, {}), (4, {"aggregation": 4}), (4, {"aggregation": 1}), (4, {"path": "range"}),
    (3, {"path": "scatter", "aggregation": 1}), (3, {"aggregation": 1}),
    (2, {"aggregation": 1}), (2, {"path": "range", "counter_bits": 32, "aggregation": 1}),
    (5, {}), (5, {"aggregation": 2}), (5, {"path": "range"}),
    (2, {"counter_bits": 8}), (3, {"path": "range", "counter_bits": 8}),
    (3, {"path": "range", "counter_bits": 8, "aggregation": 1}),
    (5, {"path": "range", "counter_bits": 8}),
]


@pytest.mark.parametrize("cfg,opts", FULL_CASES,
                         ids=[f"wl{c}-{'-'.join(f'{k}{v}' for k, v in o.items()) or 'auto'}"
                              for c, o in FULL_CASES])
def test_full_size_workloads(cfg, opts):
    x, ref, dropped, xt = full(cfg)
    w = inputs.WORKLOADS[cfg]
    plan = hist.Plan(w.num_bins, w.n, device=DEV, **opts)
    say(f"full workload {cfg}: {plan.describe()}")
    got = plan.run(xt).cpu().numpy()
    torch.cuda.synchronize(DEV)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{bad.size} bins differ, first {bad[:5].tolist()}"
    assert int(got.astype(np.int64).sum()) + dropped == w.n
    plan.close()


# --- beyond 32-bit element indices, stress, streams -------------------------

def test_more_than_2_pow_31_elements():
    # 8 GiB of input: element offsets and tile/chunk arithmetic exceed 32 bits.
    n = (1 << 31) + 7
    say(f"generating {n} elements")
    x = inputs.uniform(11, n, 1 << 20)
    xt = torch.from_numpy(x).to(DEV)
    for bins, opts in [(65536, {}), (200_000, {"path": "range"}), (1 << 20, {})]:
        ref, dropped = oracle.hist(x, bins)
        plan = hist.Plan(bins, n, device=DEV, **opts)
        say(f"case n=2^31+7 bins={bins}: {plan.describe()}")
        got = plan.run(xt).cpu().numpy()
        torch.cuda.synchronize(DEV)
        assert np.array_equal(got, ref), f"bins={bins}: {np.flatnonzero(got != ref)[:5]}"
        assert int(got.astype(np.int64).sum()) + dropped == n
        plan.close()
    del xt


def test_stress_repeated_runs_stay_exact():
    # Integer counts leave no room for noise: any lost update or race shows as
    # a mismatch. Alternate plans over the same input many times.
    x = inputs.generate(4, n=(1 << 22) + 3)
    ref, _ = oracle.hist(x, 1 << 20)
    xt = torch.from_numpy(x).to(DEV)
    plans = [hist.Plan(1 << 20, x.size, device=DEV, **o) for o in
             ({}, {"aggregation": 0}, {"groups": 37}, {"path": "range"},
              {"path": "range", "aggregation": 1})]
    outs = []
    for k in range(100):
        outs.append(plans[k % len(plans)].run(xt).clone())
    torch.cuda.synchronize(DEV)
    for k, o in enumerate(outs):
        assert np.array_equal(o.cpu().numpy(), ref), f"run {k} ({plans[k % len(plans)].describe()})"


def test_runs_on_a_side_stream():
    x = inputs.generate(2, n=1 << 22)
    ref, _ = oracle.hist(x, 65536)
    xt = torch.from_numpy(x).to(DEV)
    plan = hist.Plan(65536, x.size, device=DEV)
    s = torch.cuda.Stream(DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):
        out = torch.empty(65536, dtype=torch.int32, device=DEV)
        plan.run(xt, out)
    s.synchronize()
    assert np.array_equal(out.view(torch.uint32).cpu().numpy(), ref)


def test_two_plans_on_two_streams_in_flight():
    """Independent histograms on two streams, each with its own plan and
    output, passed as Plan.run(stream=...): alternating runs overlap on the
    device and every output is exact."""
    x = inputs.generate(2, n=(1 << 22) + 5)
    ref, _ = oracle.hist(x, 65536)
    xt = torch.from_numpy(x).to(DEV)
    streams = [torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream(DEV))
    plans = [hist.Plan(65536, x.size, device=DEV) for _ in streams]
    outs = [torch.empty(65536, dtype=torch.int32, device=DEV) for _ in streams]
    for k in range(20):
        plans[k % 2].run(xt, outs[k % 2], stream=streams[k % 2])
    torch.cuda.synchronize(DEV)
    for o in outs:
        assert np.array_equal(o.view(torch.uint32).cpu().numpy(), ref)
    with pytest.raises(ValueError):
        plans[0].run(xt, outs[0], stream=_OtherDeviceStream())
    for p in plans:
        p.close()


class _OtherDeviceStream:
    """Stands in for a stream of another device, which a one-GPU machine lacks."""
    device = torch.device("cuda", 99)
    cuda_stream = 0


@pytest.mark.parametrize("case", ["one-range", "all-invalid", "sparse-ranges", "tiny-last-range",
                                  "tile-edges", "short-runs", "mixed-runs", "sorted-block"])
def test_scatter_edge_cases(case):
    bins = 1 << 20
    if case == "short-runs":       # 512 ranges, about 32 elements per (tile, range): one run per lane
        bins = 1 << 24
        x = rnd(8, 3_000_001, -3, bins + 5)
    elif case == "mixed-runs":     # long runs in range 100 (shared by many owners), short elsewhere
        bins = (1 << 24) - 77
        x = np.concatenate([rnd(9, 2_000_000, 0, bins), rnd(10, 900_000, 100 * 32768, 101 * 32768),
                            np.full(50_000, bins - 1, np.int32)])
        x = x[np.random.default_rng(11).permutation(x.size)].astype(np.int32)
    elif case == "sorted-block":   # short runs on average, but each range has one run of ~3,000
        bins = 1 << 24
        x = np.concatenate([np.sort(rnd(12, 1_500_000, 0, bins)), rnd(13, 1_500_007, -3, bins + 5)])
    elif case == "one-range":        # every element in range 5: all owners share one range
        x = rnd(1, 700_001, 5 * 32768, 6 * 32768)
    elif case == "all-invalid":    # nothing to count: every range empty
        x = rnd(2, 300_000, bins, bins + 1000)
    elif case == "sparse-ranges":  # only ranges 0, 7 and 31 hold elements
        x = np.concatenate([rnd(3, 100_000, 0, 100), rnd(4, 200_000, 7 * 32768, 8 * 32768),
                            rnd(5, 50_000, bins - 10, bins)])
        x = x[np.random.default_rng(6).permutation(x.size)].astype(np.int32)
    elif case == "tiny-last-range":
        bins = 32768 * 3 + 1       # the last range holds a single bin
        x = rnd(7, 400_003, 0, bins)
        x[::97] = bins - 1
    else:                          # lengths around whole tiles of 16,384 elements
        for n in (16384 * 5 - 1, 16384 * 5, 16384 * 5 + 1, 16384 * 5 + 7):
            check(rnd(n, n, 0, bins), bins, f"scatter-{case}-{n}", path="scatter")
        return
    for agg in (0, 1):
        check(x, bins, f"scatter-{case}-agg{agg}", path="scatter", aggregation=agg)


# --- seeded fuzz over sizes, paths and options -------------------------------

def _fuzz_case(seed, large=False):
    g = np.random.default_rng(1000 + seed + {False: 0, True: 50_000, "huge": 90_000}[large])
    num_bins = int(min(2**20, max(1, round(2 ** g.uniform(0, 20)))))
    n = int(g.choice([0, 1, 7, int(g.integers(1, 5000)), int(g.integers(5000, 300_000))]))
    if large is True:
        num_bins = int(round(2 ** g.uniform(10, 21)))
        n = int(g.integers(4_000_000, 20_000_000))
    elif large == "huge":  # far past LDS: hundreds to 2,048 ranges, short runs
        num_bins = int(min(2**26, round(2 ** g.uniform(21, 26))))
        n = int(g.integers(500_000, 12_000_000))
    kind = g.choice(["uniform", "skew", "onebin", "wild"])
    if kind == "uniform":
        x = g.integers(0, num_bins, size=n)
    elif kind == "skew":
        x = np.minimum(g.zipf(1.3, size=n) - 1, num_bins - 1)
        x = (x * 2654435761) % num_bins  # spread the hot values over the bins
    elif kind == "onebin":
        x = np.full(n, int(g.integers(0, num_bins)))
    else:
        x = g.integers(-(2**31), 2**31 - 1, size=n)
        x[::3] = g.integers(0, num_bins, size=x[::3].size)
    x = x.astype(np.int64).astype(np.int32)
    paths = ["auto", "scatter"] + (["full"] if num_bins <= 155_392 else []) + \
        (["range", "range"] if num_bins > 1 else [])
    if large == "huge":
        paths = ["auto", "auto", "scatter", "scatter", "scatter", "range"]
    path = str(g.choice(paths))
    opts = {"path": path, "aggregation": int(g.choice([-1, 0, 1, 2, 4]))}
    if path in ("full", "range"):
        opts["wg_size"] = int(g.choice([0, 256, 512, 1024]))
        opts["counter_bits"] = int(g.choice([0, 8, 16, 32]))
        if opts["counter_bits"] == 32 and g.random() < 0.5:
            opts["lds_copies"] = int(g.choice([1, 2, 4]))
        if path == "range":
            cap = {32: 40960, 16: 79616}.get(opts["counter_bits"], 155_392)
            opts["range_bins"] = int(g.integers(1, cap // 256 + 1)) * 256
            opts["xcd_map"] = int(g.choice([0, 1, 2]))
        if g.random() < 0.3:
            opts["groups"] = int(g.integers(1, 300))
    elif path == "scatter" and g.random() < 0.3:
        opts["groups"] = int(g.integers(1, 600))
    accumulate = bool(g.random() < 0.25)
    return x, num_bins, opts, accumulate


@pytest.mark.parametrize("seed,large", [(k, False) for k in range(96)] + [(k, True) for k in range(12)]
                         + [(k, "huge") for k in range(12)])
def test_fuzz_sizes_paths_options(seed, large):
    """Random (seeded) bin counts, lengths, input shapes, paths and plan options,
    each checked bit for bit against the oracle; a quarter of the cases
    accumulate onto random counts. Combinations a plan does not support must
    be refused with HIST_ERR_UNSUPPORTED, never run. The large cases (4-20
    million elements, up to 2^21 bins) span many chunks and tiles; the huge ones
    (2^21-2^26 bins) reach the two-phase path's short-run regime."""
    x, num_bins, opts, accumulate = _fuzz_case(seed, large)
    say(f"case fuzz{seed}: n={x.size} bins={num_bins} opts={opts} accumulate={accumulate}")
    try:
        plan = hist.Plan(num_bins, max(1, x.size), device=DEV, **opts)
    except hist.HistError as e:
        assert e.status == hist.HIST_ERR_UNSUPPORTED, e
        return
    ref, _ = oracle.hist(x, num_bins)
    xt = torch.from_numpy(x).to(DEV)
    if accumulate:
        base = np.random.default_rng(seed).integers(0, 2**32, size=num_bins, dtype=np.uint64)
        base = base.astype(np.uint32)
        out = torch.from_numpy(base.view(np.int32).copy()).to(DEV)
        plan.run(xt, out=out, accumulate=True)
        want = ((base.astype(np.uint64) + ref) % 2**32).astype(np.uint32)
    else:
        out = plan.run(xt)
        want = ref
    got = out.cpu().numpy().view(np.uint32)
    torch.cuda.synchronize(DEV)
    assert np.array_equal(got, want), f"{plan.describe()}: {int(np.sum(got != want))} bins differ"
    plan.close()


# --- measured schedule choice (hist_tune) ------------------------------------

@pytest.mark.parametrize("num_bins,kind", [(8192, "uniform"), (262_144, "zipf"), (1 << 20, "zipf")])
def test_tune_measures_every_allowed_schedule_and_picks_the_fastest(num_bins, kind):
    n = 1 << 22
    x = inputs.zipf(21, n, num_bins, 1.1) if kind == "zipf" else rnd(22, n, 0, num_bins)
    say(f"case tune bins={num_bins} {kind}")
    xt = torch.from_numpy(x).to(DEV)
    best, rows = hist.tune(xt, num_bins, reps=2)
    assert len(rows) == hist.TUNE_MAX_ENTRIES
    for r in rows:
        o = r["opts"]
        if o["path"] == "full":  # allowed exactly when the counter width's slice holds all bins
            cap = {32: 40960, 16: 79616, 8: 155_392}[o["counter_bits"]]
            assert (r["status"] == hist.HIST_OK) == (num_bins <= cap), r
        else:
            assert r["status"] == hist.HIST_OK, r
    measured = [r for r in rows if r["status"] == hist.HIST_OK]
    assert all(r["ms"] > 0 for r in measured)
    assert best == min(measured, key=lambda r: r["ms"])["opts"]
    ref, _ = oracle.hist(x, num_bins)
    plan = hist.Plan(num_bins, n, device=DEV, **best)
    got = plan.run(xt).cpu().numpy()
    torch.cuda.synchronize(DEV)
    assert np.array_equal(got, ref), plan.describe()
    plan.close()


def test_tune_on_a_sample_shorter_than_max_n_and_its_errors():
    """Tuning on a sample for plans of a larger max_n: the options it returns
    make a plan for that max_n which is exact on a full-size input. counts
    receives the sample's histogram. An output that overlaps the input is
    refused before anything runs."""
    import ctypes
    num_bins, n = 300_000, 1 << 21
    x = inputs.zipf(24, 4 * n, num_bins, 1.1)
    xt = torch.from_numpy(x).to(DEV)
    best, rows = hist.tune(xt[:n], num_bins, max_n=4 * n, reps=1)
    assert any(r["status"] == hist.HIST_OK for r in rows)
    plan = hist.Plan(num_bins, 4 * n, device=DEV, **best)
    ref, _ = oracle.hist(x, num_bins)
    assert np.array_equal(plan.run(xt).cpu().numpy(), ref)
    plan.close()
    lib = hist.library()
    need = ctypes.c_uint64(0)
    assert lib.hist_tune_workspace_size(num_bins, 4 * n, ctypes.byref(need)) == hist.HIST_OK
    ws = torch.empty(int(need.value), dtype=torch.uint8, device=DEV)
    counts = torch.empty(num_bins, dtype=torch.int32, device=DEV)
    opts, cnt = hist.PlanOpts(), ctypes.c_uint32(0)
    entries = (hist.TuneEntry * hist.TUNE_MAX_ENTRIES)()
    stream = torch.cuda.current_stream(DEV).cuda_stream
    assert lib.hist_tune(num_bins, 4 * n, xt.data_ptr(), n, counts.data_ptr(), ws.data_ptr(),
                         ws.numel(), 1, stream, ctypes.byref(opts), entries,
                         hist.TUNE_MAX_ENTRIES, ctypes.byref(cnt)) == hist.HIST_OK
    assert cnt.value == hist.TUNE_MAX_ENTRIES
    sample_ref, _ = oracle.hist(x[:n], num_bins)
    assert np.array_equal(counts.view(torch.uint32).cpu().numpy(), sample_ref)
    # counts overlapping the input: refused with INVALID_ARG, nothing queued
    assert lib.hist_tune(num_bins, 4 * n, xt.data_ptr(), n, xt.data_ptr() + 4 * 16,
                         ws.data_ptr(), ws.numel(), 1, stream, ctypes.byref(opts), entries,
                         hist.TUNE_MAX_ENTRIES, ctypes.byref(cnt)) == hist.HIST_ERR_INVALID_ARG


def test_tune_skips_schedules_the_workspace_cannot_hold():
    num_bins, n = 262_144, 1 << 21
    x = rnd(23, n, 0, num_bins)
    xt = torch.from_numpy(x).to(DEV)
    cands = [("range", 32, 0), ("range", 16, 0), ("range", 16, 1), ("range", 8, 0),
             ("range", 8, 1), ("scatter", 0, 0), ("scatter", 0, 1)]
    need = {c: hist.workspace_size(num_bins, n, path=c[0], counter_bits=c[1], aggregation=c[2])
            for c in cands}
    small = min(need.values())
    ws = torch.empty(small, dtype=torch.uint8, device=DEV)
    best, rows = hist.tune(xt, num_bins, reps=1, workspace=ws)
    for r in rows:
        o = r["opts"]
        key = (o["path"], o["counter_bits"], o["aggregation"])
        if key in need:
            want = hist.HIST_OK if need[key] <= small else hist.HIST_ERR_WORKSPACE
            assert r["status"] == want, r
    assert need[(best["path"], best["counter_bits"], best["aggregation"])] <= small
    tiny = torch.empty(256, dtype=torch.uint8, device=DEV)
    with pytest.raises(hist.HistError) as e:
        hist.tune(xt, num_bins, reps=1, workspace=tiny)
    assert e.value.status == hist.HIST_ERR_WORKSPACE


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_select_predicts_a_schedule_that_is_exact(cfg):
    """hist_select samples the device input, times one stream read of it and
    predicts every schedule without running any; the schedule it names is
    then run, and must be exact like any other."""
    x = inputs.generate(cfg, n=1 << 21)
    B = inputs.WORKLOADS[cfg].num_bins
    xt = torch.from_numpy(x).to(DEV)
    best, rows = hist.select(xt, B)
    assert rows and all(r["status"] in (hist.HIST_OK, hist.HIST_ERR_UNSUPPORTED) for r in rows)
    ok = [r for r in rows if r["status"] == hist.HIST_OK]
    assert ok and min(ok, key=lambda r: r["predicted_us"])["opts"] == best
    say(f"select cfg {cfg}: {best} " + " ".join(f"{r['schedule']}:{r['predicted_us']:.1f}"
                                                  for r in ok))
    check(x, B, f"selected-cfg{cfg}", **best)


STREAM_CASES = [  # (label, input, bins, producers)
    ("hot-bin shape 2^22", lambda: inputs.generate(4, n=1 << 22), 1 << 20, 0),
    ("half-Gaussian shape 2^22", lambda: inputs.generate(5, n=1 << 22), 1 << 19, 0),
    ("uniform 2^21 bins, ragged", lambda: rnd(41, 3_000_001, -7, (1 << 21) + 9), 1 << 21, 0),
    ("one range, one tile", lambda: rnd(42, 10_000, 0, 5000), 5000, 0),
    ("partial last range", lambda: rnd(43, 500_003, 0, 100_003), 100_003, 0),
    ("every range empty but one", lambda: np.full(700_001, 65_537, np.int32), 1 << 20, 0),
    ("one producer", lambda: inputs.generate(4, n=1 << 21), 1 << 20, 1),
    ("all producers", lambda: inputs.generate(5, n=1 << 21), 1 << 19, 256),
    ("eight producers", lambda: rnd(44, 1 << 22, 0, 1 << 20), 1 << 20, 8),
]


@pytest.mark.parametrize("case", STREAM_CASES, ids=[c[0] for c in STREAM_CASES])
def test_stream_path(case):
    """The streaming owner-queue path (STREAM) against the oracle: producers
    route tiles and publish them, owners count each range as its tiles arrive
    and move to the ranges with the most work left, adding their counts under
    the range's lock. Every bounded wait must have ended on its own."""
    label, make, bins, producers = case
    x = make()
    for offset in (0, 1):
        ref, dropped = oracle.hist(x, bins)
        say(f"case stream {label}: n={x.size} bins={bins} offset={offset} P={producers}")
        buf = torch.full((x.size + offset + 4,), -1, dtype=torch.int32, device=DEV)
        xt = buf[offset:offset + x.size]
        xt.copy_(torch.from_numpy(x))
        plan = hist.Plan(bins, max(1, x.size), device=DEV, path="stream", groups=producers)
        got = plan.run(xt).cpu().numpy()
        assert not plan.check(), f"{label}: a wait gave up"
        assert np.array_equal(got, ref), f"{label} ({plan.describe()})"
        # a second run on the same workspace, accumulating onto the first
        acc = torch.from_numpy(got.view(np.int32).copy()).to(DEV)
        plan.run(xt, out=acc, accumulate=True)
        assert not plan.check()
        got2 = acc.cpu().numpy().view(np.uint32).astype(np.int64)
        assert np.array_equal(got2, 2 * ref.astype(np.int64)), label
        plan.close()


def test_stream_accumulates_and_repeats():
    x = inputs.generate(4, n=1 << 21)
    bins = 1 << 20
    ref, _ = oracle.hist(x, bins)
    plan = hist.Plan(bins, x.size, device=DEV, path="stream")
    xt = torch.from_numpy(x).to(DEV)
    out = torch.full((bins,), 3, dtype=torch.int32, device=DEV)
    for _ in range(3):
        plan.run(xt, out, accumulate=True)
    got = out.cpu().numpy().view(np.uint32).astype(np.int64)
    assert np.array_equal(got, 3 + 3 * ref.astype(np.int64))
    for _ in range(3):  # overwriting runs in a row reuse the workspace
        assert np.array_equal(plan.run(xt).cpu().numpy(), ref)
    assert not plan.check()
    plan.close()


def test_stream_waits_that_give_up_are_reported():
    """A poll bound of 2 makes owners give up on tiles not yet published (a
    forced failure of the bounded wait, from the host): the kernel still ends,
    and the plan reports the give-up."""
    x = inputs.generate(4, n=1 << 22)
    bins = 1 << 20
    plan = hist.Plan(bins, x.size, device=DEV, path="stream", spin_log2=1, groups=8)
    xt = torch.from_numpy(x).to(DEV)
    gave_up = False
    for _ in range(3):
        plan.run(xt)
        gave_up = gave_up or plan.check()
    say(f"stream spin 2: gave up {gave_up}")
    assert gave_up
    plan.close()


def top_cluster(seed, n, num_bins):
    """Half the elements in the last 3,000 bins and 100 values past them, the
    rest uniform over the bins, some negative: the heaviest window runs past
    num_bins and must be cut there."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-50, num_bins, size=n, dtype=np.int64)
    hot = rng.random(n) < 0.5
    x[hot] = rng.integers(num_bins - 3000, num_bins + 100, size=int(hot.sum()))
    return x.astype(np.int32)


def hot_values(seed, n, num_bins, hot, cluster=None):
    """Uniform over the bins, some negative and some past the last bin, with
    each (value, share) of hot holding that share of the elements and, when
    cluster is (first bin, bins, share), that share spread over those bins."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-50, num_bins + 50, size=n, dtype=np.int64)
    u = rng.random(n)
    lo = 0.0
    for value, share in hot:
        x[(u >= lo) & (u < lo + share)] = value
        lo += share
    if cluster:
        first, width, share = cluster
        m = (u >= lo) & (u < lo + share)
        x[m] = first + rng.integers(0, width, size=int(m.sum()))
    return x.astype(np.int32)


WINDOW_CASES = [  # (label, input, bins)
    ("half-Gaussian shape 2^22", lambda: inputs.generate(5, n=1 << 22), 1 << 19),
    ("hot-bin shape 2^22", lambda: inputs.generate(4, n=1 << 22), 1 << 20),
    ("cluster at the last bins", lambda: top_cluster(51, (1 << 22) + 5, 700_001), 700_001),
    ("uniform 2^21 bins", lambda: rnd(52, 1 << 22, 0, 1 << 21), 1 << 21),
    ("below the sampling size", lambda: top_cluster(53, 100_003, 300_000), 300_000),
    ("two hot values, no window", lambda: hot_values(54, (1 << 22) + 3, 1 << 22, [(777, 0.12), (3_000_001, 0.09)]),
     1 << 22),
    ("hot value beside a window",
     lambda: hot_values(55, 1 << 22, 1 << 20, [(900_000, 0.08)], cluster=(1000, 4000, 0.4)), 1 << 20),
    ("hot value at the last bin", lambda: hot_values(56, (1 << 22) + 1, 500_000, [(499_999, 0.2)]), 500_000),
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=[c[0] for c in WINDOW_CASES])
def test_scatter_in_place_window(case):
    """SCATTER with its in-place window: the partition workgroups count the
    heaviest 8,192 bins a sample shows in LDS, and a value that holds a
    thirty-second of the sample in registers, and never stage either; their
    rows are added after the owners. Auto, off and forced must all be exact,
    at an aligned and a misaligned start, overwriting and accumulating."""
    label, make, bins = case
    x = make()
    ref, _ = oracle.hist(x, bins)
    for window in (0, 1, 2):
        for offset in (0, 1):
            say(f"case window {label}: n={x.size} bins={bins} window={window} offset={offset}")
            buf = torch.full((x.size + offset + 4,), -1, dtype=torch.int32, device=DEV)
            xt = buf[offset:offset + x.size]
            xt.copy_(torch.from_numpy(x))
            plan = hist.Plan(bins, x.size, device=DEV, path="scatter", window=window)
            assert ("win=auto", "win=off", "win=on")[window] in plan.describe()
            got = plan.run(xt).cpu().numpy()
            assert np.array_equal(got, ref), f"{label} window={window} offset={offset}"
            acc = torch.from_numpy(got.view(np.int32).copy()).to(DEV)
            plan.run(xt, out=acc, accumulate=True)
            got2 = acc.cpu().numpy().view(np.uint32).astype(np.int64)
            assert np.array_equal(got2, 2 * ref.astype(np.int64)), f"{label} accumulate"
            plan.close()
