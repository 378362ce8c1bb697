"""Benchmark of the partitioned LDS histogram on one MI355X.

A step is one hist_run (every kernel of the path) over one batch of the
65,536-bin uniform workload: n = 67,108,864 int32 indices uniform in
[0, 65536) from seed 1, 65,536 uint32 bins. The inputs are resident in HBM
before timing starts. Four device copies of the input are used in rotation,
so that consecutive steps cannot serve a 256 MiB input from the 256 MB
Infinity Cache that the previous step filled.

The steps run on one stream. `--two-streams` adds, from the same run, the
same K steps alternating over two streams, each stream with its own plan,
workspace and output: two independent histograms are then in flight, and
one's merge and launch ramp overlap the other's sweep, as for a caller who
histograms a series of batches with a plan per stream. (`--streams 2` makes
that the timed mode; the roofline's per-launch durations then include the
overlap.)

Before the W warm-up steps of each timed region, 0.3 s of untimed runs of
the same plan let the clocks settle: with K = 20 a region lasts about a
millisecond, and a fresh box's first milliseconds run below the settled clock
(20-step runs measured 52.3-53.0 us per step without this, 500-step runs
50.2).

Prints one JSON line (rank 0). Throughput `value` is Gelem/s over the K timed
steps (wall clock between two device synchronisations, no instrumentation in
between). `roofline` is for the dominant kernel, timed live over a second run
of K steps with HIP events attached to the kernels' own dispatches (the
kernel's start and end, as a profiler's kernel trace reports them);
`roofline.rocprof` gives the same kernel's average from the committed
rocprofv3 trace of this command, when the kernel sources still match it.
`workloads` repeats the measurement (W warm-up and K timed steps, AUTO's
plan) on the four other workloads at full size, each checked bit for bit.
`cpu_baseline` is the CPU oracle (a sequential loop, one core) timed on a
bounded sample of the same input; that is the only use of the oracle here.
The result checks (`parity_vs_bincount`, `workloads[*].parity`, the sweeps'
`parity`) compare with numpy's bincount.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
# The sources a stored profile entry was taken from, when the entry does not
# list its own (entries written before they did).
KERNEL_SOURCES = [f"partitioned_chip_accumulation_amd/csrc/{f}" for f in (
    "hist_common.hpp", "hist_counters16.hpp", "hist_partials.hpp", "hist_sweep.hpp",
    "hist_scatter.hpp", "hist_kernels.hpp", "hist_api.hip", "hist_counters8.hpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_TIMES_FILE = os.path.join(ROOT, "profiles", "kernel_times.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--config", type=int, default=2, help="workload 1..5 (2 = the headline)")
    ap.add_argument("--n", type=int, default=None, help="override the workload length")
    ap.add_argument("--uniform-bins", type=int, default=0,
                    help="instead of a workload, uniform int32 over this many bins (sweeps)")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also run one plain copy of this many MiB (for counter scaling)")
    ap.add_argument("--path", default="auto", choices=["auto", "full", "range", "scatter", "stream"])
    ap.add_argument("--groups", type=int, default=0)
    ap.add_argument("--range-bins", type=int, default=0)
    ap.add_argument("--agg", type=int, default=-1)
    ap.add_argument("--wg", type=int, default=0)
    ap.add_argument("--xcd-map", type=int, default=0)
    ap.add_argument("--counter-bits", type=int, default=0)
    ap.add_argument("--lds-copies", type=int, default=0,
                    help="interleaved LDS copies for 32-bit counters (0 = the plan's choice)")
    ap.add_argument("--pacing", type=int, default=0,
                    help="RANGE owners' reads: 1 non-temporal, 2 plain, 3.. plain and paced "
                         "within (pacing - 2) batches (0 = the plan's choice)")
    ap.add_argument("--window", type=int, default=0,
                    help="SCATTER's in-place window: 0 auto, 1 off, 2 always")
    ap.add_argument("--copies", type=int, default=4, help="input copies used in rotation")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="bound on the CPU-baseline work (0 = skip)")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--streams", type=int, default=1,
                    help="histograms in flight: consecutive steps alternate over this many "
                         "streams, each with its own plan, workspace and output")
    ap.add_argument("--two-streams", action="store_true",
                    help="also time the K steps alternating over two streams (two histograms in "
                         "flight); off by default, so that every launch of a kernel in a trace "
                         "of the default command is timed alike")
    ap.add_argument("--no-two-streams", action="store_true",
                    help="the default (kept so that older profiling commands still run)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the `workloads` record (the four other workloads at full size)")
    ap.add_argument("--tune", action="store_true",
                    help="time every schedule on the input first (hist_tune) and bench the fastest")
    ap.add_argument("--select", action="store_true",
                    help="predict every schedule on the input with the cost model (hist_select: a "
                         "sample and one stream read, no schedule run) and bench the predicted "
                         "fastest")
    ap.add_argument("--comparators", action="store_true",
                    help="also time the global-atomic fallback and the stream-read ceiling")
    ap.add_argument("--path-sweep", action="store_true",
                    help="time every applicable path over bin counts 2^10..2^22 on uniform "
                         "input of --n (default 2^26) elements; one JSON line per cell")
    ap.add_argument("--sweep-log2", default="10,22",
                    help="first,last log2 bin count of --path-sweep")
    ap.add_argument("--sweep-zipf", type=float, default=0.0,
                    help="--path-sweep on finite Zipf input with this exponent (ranks permuted "
                         "to bins) instead of uniform input")
    ap.add_argument("--calibrate", action="store_true",
                    help="measure the machine's ceilings the kernels meet (HBM stream read and "
                         "copy, LDS atomic rates by address pattern, shared-L2 placement of "
                         "range owners); one JSON line per measurement")
    ap.add_argument("--workload-matrix", action="store_true",
                    help="time every applicable path on each of the five workloads; one JSON "
                         "line per cell")
    return ap.parse_args()


def time_cells(plan, xs, out, warm: int, steps: int) -> float:
    """Seconds per run: wall clock over back-to-back runs on rotated inputs."""
    import torch
    for k in range(warm):
        plan.run(xs[k % len(xs)], out)
    torch.cuda.synchronize(out.device)
    t0 = time.perf_counter()
    for k in range(steps):
        plan.run(xs[k % len(xs)], out)
    torch.cuda.synchronize(out.device)
    return (time.perf_counter() - t0) / steps


def reference_counts(x, num_bins: int):
    """Bit-exact reference for the measurement modes' checks: numpy's bincount
    over the in-range values, an independent library routine (the CPU oracle
    is reserved for the CPU baseline timing)."""
    import numpy as np
    v = x[(x >= 0) & (x < num_bins)]
    return np.bincount(v, minlength=num_bins).astype(np.uint32)


def settle(run, seconds: float = 0.3):
    """Call run(k) untimed for about `seconds` (in groups of 8, synchronised),
    so that the timed steps after it meet settled clocks."""
    import torch
    t0 = time.perf_counter()
    k = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            run(k)
            k += 1
        torch.cuda.synchronize()


def settle_clocks(B, n, xs, out, seconds: float = 0.3):
    """Run the plan's own choice untimed for a while before a row's cells are
    timed: the first cells after an input upload otherwise run at unsettled
    clocks (as the second cell of a row, a plan measured 6% slower than the
    same plan as the last)."""
    import torch
    from partitioned_chip_accumulation_amd import hist
    plan = hist.Plan(B, n, device=out.device)
    t0 = time.perf_counter()
    k = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            plan.run(xs[k % len(xs)], out)
            k += 1
        torch.cuda.synchronize(out.device)
    plan.close()


def calibrate(args):
    """On-chip and HBM ceilings on this GPU, each a JSON line."""
    import torch

    from partitioned_chip_accumulation_amd import hist, inputs

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cu = torch.cuda.get_device_properties(dev).multi_processor_count
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize(dev)
        ev0.record()
        for _ in range(reps):
            fn()
        ev1.record()
        torch.cuda.synchronize(dev)
        return ev0.elapsed_time(ev1) / 1e3 / reps

    # HBM: 1 GiB read once, and a 512 MiB copy (rotating buffers defeat the 256 MB MALL).
    src = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    t = timed(lambda: hist.stream_read(src, sink), 20)
    print(json.dumps({"what": "hbm_stream_read", "GBps": round(4 * src.numel() / t / 1e9, 1),
                      "bytes": 4 * src.numel()}), flush=True)
    half = 1 << 27
    t = timed(lambda: hist.copy(dst[:half], src[:half]), 20)
    print(json.dumps({"what": "hbm_copy", "GBps": round(8 * half / t / 1e9, 1),
                      "bytes_moved": 8 * half}), flush=True)
    del src, dst
    # LDS atomics: time per wave instruction per CU, and cycles at the 2.4 GHz peak clock.
    iters = 2048
    lsink = torch.zeros(cu, dtype=torch.int32, device=dev)
    for pattern in ("distinct", "random", "same", "groups8"):
        for rtn in (False, True):
            t = timed(lambda: hist.lds_atomic(pattern, rtn, iters, lsink), 5)
            per_instr = t / (16 * iters * 16)
            print(json.dumps({"what": "lds_atomic", "pattern": pattern, "with_return": rtn,
                              "ns_per_wave_instr_per_cu": round(per_instr * 1e9, 3),
                              "cycles_at_2p4GHz": round(per_instr * 2.4e9, 2)}), flush=True)
    # LDS latency: dependent chains of one wave (each address waits for the
    # previous return).
    for pattern in hist.LDS_LATENCY_PATTERNS:
        r = hist.lds_latency(pattern, 1 << 16, dev)
        print(json.dumps({"what": "lds_latency", "pattern": pattern,
                          "cycles_per_op": round(r["cycles_per_op"], 2),
                          "ns_per_op": round(r["ns_per_op"], 3),
                          "clock_ghz": round(r["clock_ghz"], 3) if r["clock_ghz"] else None}),
              flush=True)
    # Handoff between two workgroups through global memory, on one XCD (partner
    # 8: workgroups are dealt to the 8 XCDs in turn) and across XCDs (partner 1).
    for mode in (0, 1):
        for partner in (8, 1):
            hist.handoff(partner, mode, 64, dev)  # warm-up
            r = hist.handoff(partner, mode, 4096, dev)
            print(json.dumps({"what": "handoff", "mode": ["token", "payload+release/acquire"][mode],
                              "partner": partner, "same_xcd": r["xcd_wg0"] == r["xcd_partner"],
                              "round_trip_cycles": round(r["round_trip_cycles"], 1),
                              "round_trip_ns": round(r["round_trip_ns"], 1),
                              "timed_out": r["timed_out"], "payload_errors": r["payload_errors"],
                              "xcds": r["xcds"]}), flush=True)
    # Primitives of the cost model (hist_predict): a launch, a sweep's fixed cost,
    # one 8-bit carry event, the two-phase path's fixed cost. Each comes from the
    # library's own kernels on synthetic input that isolates one cost, timed on
    # the device with the events the plan attaches to its kernels (the host's
    # per-call overhead would hide short kernels).
    import numpy as np

    def kernel_us(plan, xt, out, reps, phase=None):
        """Average device time per call: one phase, or all phases summed."""
        for _ in range(3):
            plan.run(xt, out)
        torch.cuda.synchronize(dev)
        plan.timing_enable(reps)
        for _ in range(reps):
            plan.run(xt, out)
        ph = plan.timing_read()
        plan.timing_enable(0)
        if phase is not None:
            ms, cnt = ph[phase]
            return ms / cnt * 1e3
        return sum(ms / cnt for ms, cnt in ph.values()) * 1e3

    empty = torch.empty(0, dtype=torch.int32, device=dev)
    o256 = torch.empty(256, dtype=torch.int32, device=dev)
    plan = hist.Plan(256, 1, device=dev)
    t = kernel_us(plan, empty, o256, 200, "sweep")
    plan.close()
    print(json.dumps({"what": "model_primitive", "name": "launch_us", "value": round(t, 3),
                      "how": "device time of the one kernel of a hist_run with n = 0"}), flush=True)
    # a sweep's fixed cost: the intercept of one plan's sweep time at n and 2n
    o64k = torch.empty(65536, dtype=torch.int32, device=dev)
    plan = hist.Plan(65536, 1 << 25, device=dev, path="full", counter_bits=16)
    x1 = torch.from_numpy(inputs.uniform(7, 1 << 25, 65536)).to(dev)
    t1 = kernel_us(plan, x1[:1 << 24], o64k, 50, "sweep")
    t2 = kernel_us(plan, x1, o64k, 50, "sweep")
    print(json.dumps({"what": "model_primitive", "name": "sweep_fixed_us",
                      "value": round(2 * t1 - t2, 3), "t_2p24_us": round(t1, 2),
                      "t_2p25_us": round(t2, 2), "plan": plan.describe(),
                      "how": "FULL 16-bit sweep of 2^24 and 2^25 uniform elements over 65,536 "
                             "bins, 256 chunks: 2 T(n) - T(2n)"}), flush=True)
    plan.close()
    del x1
    # carry events: uniform over 2,048 bins, 2^28 elements in 512 chunks (the
    # 8-bit event list's bound allows at most 560,490 elements a chunk here), so
    # a bin takes about 256 adds a chunk and half the bins wrap their byte once;
    # the 16-bit plan with the same chunks has no events
    ne, be, ge = 1 << 28, 2048, 512
    xe_host = inputs.uniform(8, ne, be)
    xe = torch.from_numpy(xe_host).to(dev)
    oe = torch.empty(be, dtype=torch.int32, device=dev)
    p8 = hist.Plan(be, ne, device=dev, path="full", counter_bits=8, groups=ge)
    p16 = hist.Plan(be, ne, device=dev, path="full", counter_bits=16, groups=ge)
    assert p8.info().groups == ge and p16.info().groups == ge
    t8, t16 = kernel_us(p8, xe, oe, 10, "sweep"), kernel_us(p16, xe, oe, 10, "sweep")
    nvec = ne // 4
    events = 0
    for g in range(ge):  # chunk g holds body vectors [g nvec / G, (g + 1) nvec / G)
        lo, hi = (g * nvec // ge) * 4, ((g + 1) * nvec // ge) * 4
        events += int((np.bincount(xe_host[lo:hi], minlength=be) // 256).sum())
    print(json.dumps({"what": "model_primitive", "name": "event_cycles",
                      "value": round((t8 - t16) * 1e-6 * cu * 2.4e9 / events, 2),
                      "t8_us": round(t8, 2), "t16_us": round(t16, 2), "events": events,
                      "plan8": p8.describe(), "plan16": p16.describe(),
                      "how": "sweep time of FULL 8-bit minus FULL 16-bit on 2^28 uniform elements "
                             "over 2,048 bins in 512 chunks, per carry event, in cycles of every "
                             "CU at 2.4 GHz"}), flush=True)
    p8.close()
    p16.close()
    del xe, xe_host
    # the two-phase path's fixed cost: the intercept of its summed phases at n and 2n
    o1m = torch.empty(1 << 20, dtype=torch.int32, device=dev)
    x3 = torch.from_numpy(inputs.uniform(9, 1 << 23, 1 << 20)).to(dev)
    plan = hist.Plan(1 << 20, 1 << 23, device=dev, path="scatter", aggregation=0)
    t1 = kernel_us(plan, x3[:1 << 22], o1m, 50)
    t2 = kernel_us(plan, x3, o1m, 50)
    print(json.dumps({"what": "model_primitive", "name": "scatter_fixed_us",
                      "value": round(2 * t1 - t2, 3), "t_2p22_us": round(t1, 2),
                      "t_2p23_us": round(t2, 2), "plan": plan.describe(),
                      "how": "two-phase path on 2^22 and 2^23 uniform elements over 2^20 bins, "
                             "its phases summed: 2 T(n) - T(2n)"}), flush=True)
    plan.close()
    del x3, o1m
    torch.cuda.empty_cache()
    # Shared L2: RANGE with the R owners of a chunk on one XCD vs in plain order.
    n, B = 1 << 26, 1 << 17
    x = torch.from_numpy(inputs.uniform(1, n, B)).to(dev)
    xs = [x] + [x.clone() for _ in range(3)]
    out = torch.empty(B, dtype=torch.int32, device=dev)
    for xcd_map in (1, 2):
        plan = hist.Plan(B, n, device=dev, path="range", counter_bits=16, xcd_map=xcd_map)
        dt = time_cells(plan, xs, out, 20, 200)
        print(json.dumps({"what": "range_owner_placement",
                          "placement": "one XCD per chunk" if xcd_map == 1 else "plain order",
                          "bins": B, "n": n, "us_per_run": round(dt * 1e6, 2),
                          "plan": plan.describe()}), flush=True)
        plan.close()


def workload_matrix(args):
    """Every applicable schedule forced on every workload, each checked bit
    for bit against numpy's bincount: which path the data itself favours,
    beside the plan's choice from the bin count alone."""
    import numpy as np
    import torch

    from partitioned_chip_accumulation_amd import hist, inputs

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    for cfg in range(1, 6):
        w = inputs.WORKLOADS[cfg]
        x = inputs.generate(cfg, n=w.n)
        ref = reference_counts(x, w.num_bins)
        xs = [torch.from_numpy(x).to(dev)]
        for _ in range(3):
            xs.append(xs[0].clone())
        out = torch.empty(w.num_bins, dtype=torch.int32, device=dev)
        B = w.num_bins
        cells = []
        if B <= 40960:
            cells.append(("full32", {"path": "full", "counter_bits": 32}))
        if B <= 79616:
            cells.append(("full16", {"path": "full", "counter_bits": 16}))
        if B <= 155392:
            cells.append(("full8", {"path": "full", "counter_bits": 8}))
        if B >= 2048:
            cells.append(("range32", {"path": "range", "counter_bits": 32}))
            cells.append(("range16", {"path": "range", "counter_bits": 16}))
            cells.append(("range16+hot", {"path": "range", "counter_bits": 16,
                                          "aggregation": 1}))
            cells.append(("range8", {"path": "range", "counter_bits": 8}))
            cells.append(("range8+hot", {"path": "range", "counter_bits": 8, "aggregation": 1}))
        cells.append(("scatter", {"path": "scatter", "aggregation": 0}))
        cells.append(("scatter+hot", {"path": "scatter", "aggregation": 1}))
        if B <= 1 << 21:
            cells.append(("stream", {"path": "stream"}))
        cells.append(("auto", {}))  # last: the first cell after an upload runs slow
        steps = max(10, min(args.steps, int(4e9 / (4 * w.n))))
        settle_clocks(B, w.n, xs, out)
        for name, opts in cells:
            if B > 4 * 79616 and name.startswith("range32"):
                continue  # dozens of passes over the input: not a contender
            try:
                plan = hist.Plan(B, w.n, device=dev, **opts)
            except hist.HistError as e:
                print(json.dumps({"workload": w.name, "cell": name, "error": str(e)}), flush=True)
                continue
            dt = time_cells(plan, xs, out, 10, steps)
            ok = bool(np.array_equal(out.view(torch.uint32).cpu().numpy(), ref))
            print(json.dumps({"workload": w.name, "n": w.n, "bins": B, "cell": name,
                              "us_per_run": round(dt * 1e6, 1),
                              "gelem_s": round(w.n / dt / 1e9, 1), "parity": ok,
                              "plan": plan.describe()}), flush=True)
            plan.close()
        del xs, out
        torch.cuda.empty_cache()


def path_sweep(args):
    """Every schedule the library offers, on uniform (or --sweep-zipf) input,
    across bin counts.

    The cells are the evidence behind the plan's automatic choice: for each
    bin count the fastest bit-exact schedule wins. Timing is the same as the
    headline's (wall clock over back-to-back runs on rotated input copies).
    """
    import numpy as np
    import torch

    from partitioned_chip_accumulation_amd import hist, inputs

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    n = args.n or (1 << 26)
    steps = min(args.steps, 100)
    best = {}
    lb0, lb1 = (int(v) for v in args.sweep_log2.split(","))
    for lb in range(lb0, lb1 + 1):
        B = 1 << lb
        x = inputs.zipf(2, n, B, args.sweep_zipf) if args.sweep_zipf > 0 else inputs.uniform(1, n, B)
        ref = reference_counts(x, B)
        xs = [torch.from_numpy(x).to(dev)]
        for _ in range(3):
            xs.append(xs[0].clone())
        out = torch.empty(B, dtype=torch.int32, device=dev)
        cells = []
        if B <= 40960:
            cells.append(("full32", {"path": "full", "counter_bits": 32}))
        if B <= 79616:
            cells.append(("full16", {"path": "full", "counter_bits": 16}))
        if B <= 155392:
            cells.append(("full8", {"path": "full", "counter_bits": 8}))
        if B >= 2048:
            cells.append(("range32", {"path": "range", "counter_bits": 32}))
            cells.append(("range16", {"path": "range", "counter_bits": 16}))
            cells.append(("range8", {"path": "range", "counter_bits": 8}))
        cells.append(("scatter", {"path": "scatter"}))
        if args.sweep_zipf > 0:
            cells.append(("scatter+hot", {"path": "scatter", "aggregation": 1}))
        if B <= 1 << 21:
            cells.append(("stream", {"path": "stream"}))
        cells.append(("auto", {}))  # last: the first cell after an upload runs slow
        settle_clocks(B, n, xs, out)
        for name, opts in cells:
            try:
                plan = hist.Plan(B, n, device=dev, **opts)
            except hist.HistError as e:
                print(json.dumps({"bins": B, "cell": name, "error": str(e)}), flush=True)
                continue
            for k in range(20):
                plan.run(xs[k % 4], out)
            torch.cuda.synchronize(dev)
            t0 = time.perf_counter()
            for k in range(steps):
                plan.run(xs[k % 4], out)
            torch.cuda.synchronize(dev)
            dt = (time.perf_counter() - t0) / steps
            ok = bool(np.array_equal(out.view(torch.uint32).cpu().numpy(), ref))
            rec = {"bins": B, "n": n, "cell": name, "us_per_run": round(dt * 1e6, 2),
                   "input": f"zipf s={args.sweep_zipf:g}" if args.sweep_zipf > 0 else "uniform",
                   "gelem_s": round(n / dt / 1e9, 1), "parity": ok, "plan": plan.describe()}
            print(json.dumps(rec), flush=True)
            if name != "auto" and ok and (B not in best or dt < best[B][1]):
                best[B] = (name, dt)
            plan.close()
        del xs
    print("# fastest bit-exact schedule per bin count: " +
          ", ".join(f"2^{B.bit_length() - 1}:{v[0]}" for B, v in sorted(best.items())),
          file=sys.stderr, flush=True)


def kernel_source_sha(sources: list[str] | None = None) -> str:
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        try:
            with open(os.path.join(ROOT, rel), "rb") as f:
                h.update(f.read())
        except OSError:
            return "missing:" + rel
    return h.hexdigest()


def stored_entry(path: str, key: str) -> dict:
    """The entry for this kernel and workload in a committed profile summary
    (profiles/traffic.json: counter-derived HBM bytes per launch, LDS and
    occupancy counters; profiles/kernel_times.json: rocprofv3 kernel-trace
    durations), or {} when there is none or the kernel sources changed since
    it was taken."""
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return {}
    e = data.get(key)
    if not e or e.get("kernel_source_sha") != kernel_source_sha(e.get("sources")):
        return {}
    return e


def counters_for(key: str) -> dict:
    return stored_entry(TRAFFIC_FILE, key)


def dominant_kernel(phases: dict, n: int, B: int):
    """(phase name, algorithmic bytes per launch, average launch seconds,
    launches) of the kernel that reads the input (sweep, partition or
    stream), else of the phase with the most device time. On a launch-bound
    input the merge can take as long as the sweep; the roofline still
    describes the sweep. The sweep and the partition read each element once
    (4 bytes); the owner kernel reads its 2-byte routed slots; the merges
    write the 4-byte bins."""
    readers = {k: v for k, v in phases.items() if k in ("sweep", "partition", "stream")}
    name, (ms, launches) = max((readers or phases).items(), key=lambda kv: kv[1][0])
    if name in ("sweep", "partition", "stream"):
        nbytes = 4 * n
    elif name == "owner_hist":
        nbytes = 2 * n
    else:
        nbytes = 4 * B
    return name, nbytes, ms / launches / 1e3, launches


def roofline_for(phases: dict, n: int, B: int, key_tail: str) -> dict:
    name, nbytes, avg_s, launches = dominant_kernel(phases, n, B)
    achieved = nbytes / avg_s / 1e9
    key = f"{name}:{key_tail}"
    r = {"bound": "hbm", "kernel": name, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
         "traffic": counters_for(key).get("bytes_per_launch"), "traffic_key": key,
         "lds_counters": counters_for(key).get("lds_counters"), "algorithmic_bytes": nbytes,
         "avg_launch_us": round(avg_s * 1e6, 2), "launches": launches}
    t = stored_entry(KERNEL_TIMES_FILE, key)
    r["rocprof"] = None if not t else {
        "avg_launch_us": t["avg_us"], "frac": round(nbytes / (t["avg_us"] * 1e-6) / 1e9 /
                                                    HBM_PEAK_GBPS, 4),
        "calls": t["calls"], "kernel": t["kernel"], "profile": t["profile"]}
    return r


def time_workload(cfg: int, steps: int, warmup: int, dev, check: bool = True,
                  comparators: bool = False) -> dict:
    """One workload at full size with AUTO's plan: W warm-up and K timed runs
    (wall clock between device synchronisations), then K runs with kernel
    events for the dominant kernel, and a bit-exact check against numpy's
    bincount."""
    import numpy as np
    import torch

    from partitioned_chip_accumulation_amd import hist, inputs

    w = inputs.WORKLOADS[cfg]
    print(f"# workload {w.name}: generating {w.n} elements", file=sys.stderr, flush=True)
    x = inputs.generate(cfg, n=w.n)
    xs = [torch.from_numpy(x).to(dev)]
    if 4 * w.n * 4 <= 256 * 2**20:
        xs += [xs[0].clone() for _ in range(3)]  # as the headline: four copies in rotation
    out = torch.empty(w.num_bins, dtype=torch.int32, device=dev)
    plan = hist.Plan(w.num_bins, w.n, device=dev)
    settle(lambda k: plan.run(xs[k % len(xs)], out))
    for k in range(warmup):
        plan.run(xs[k % len(xs)], out)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for k in range(steps):
        plan.run(xs[k % len(xs)], out)
    torch.cuda.synchronize(dev)
    dt = (time.perf_counter() - t0) / steps
    plan.timing_enable(steps)
    for k in range(steps):
        plan.run(xs[k % len(xs)], out)
    phases = plan.timing_read()
    plan.timing_enable(0)
    rec = {"n": w.n, "num_bins": w.num_bins, "recipe": w.recipe, "plan": plan.describe(),
           "us_per_histogram": round(dt * 1e6, 2), "gelem_s": round(w.n / dt / 1e9, 2),
           "achieved_GBps": round((4 * w.n + 4 * w.num_bins) / dt / 1e9, 1),
           "hbm_frac": round((4 * w.n + 4 * w.num_bins) / dt / 1e9 / HBM_PEAK_GBPS, 4),
           "phases_us": {k: round(v[0] / v[1] * 1e3, 2) for k, v in phases.items()},
           "roofline": roofline_for(phases, w.n, w.num_bins, f"{w.name}:n={w.n}:{plan.describe()}"),
           "parity": None}
    if len(xs) > 1:
        rec["note"] = ("input copies fit the 256 MB Infinity Cache; launch- and cache-bound, so "
                       "the HBM fraction is not meaningful")
    ref = reference_counts(x, w.num_bins) if check or comparators else None
    if check:
        rec["parity"] = bool(np.array_equal(out.view(torch.uint32).cpu().numpy(), ref))
    plan.close()
    if comparators:
        rec["comparators"] = comparator_figures(xs, w.num_bins, ref)
    return rec


def comparator_figures(xs, num_bins: int, ref) -> dict:
    """The global-atomic fallback (page "Distributed Shared Memory", section
    "When it beats global atomics": every element one atomic add into global
    memory) and the stream-read ceiling on the same input, both timed with
    events around a few back-to-back runs; the fallback's counts are checked
    against the same reference."""
    import numpy as np
    import torch

    from partitioned_chip_accumulation_amd import hist

    dev = xs[0].device
    n = xs[0].numel()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    got = hist.global_atomic(xs[0], num_bins)  # untimed, and checked
    torch.cuda.synchronize(dev)
    ok = bool(np.array_equal(got.cpu().numpy(), ref)) if ref is not None else None
    reps = max(2, min(20, int(2e9 / (4 * n))))
    s.record()
    for k in range(reps):
        hist.global_atomic(xs[k % len(xs)], num_bins)
    e.record()
    torch.cuda.synchronize(dev)
    ga = s.elapsed_time(e) / 1e3 / reps
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    hist.stream_read(xs[0], sink)
    s.record()
    for k in range(reps):
        hist.stream_read(xs[k % len(xs)], sink)
    e.record()
    torch.cuda.synchronize(dev)
    rd = s.elapsed_time(e) / 1e3 / reps
    return {"global_atomic_us": round(ga * 1e6, 1), "global_atomic_gelem_s": round(n / ga / 1e9, 2),
            "global_atomic_parity": ok, "stream_read_us": round(rd * 1e6, 1),
            "stream_read_GBps": round(4 * n / rd / 1e9, 1), "reps": reps}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only; there is no multi-GPU path. Sharded, each GPU "
              "would count a contiguous chunk of the input and a reduce-scatter by bin range "
              "would make GPU k the owner of bins [kB/g, (k+1)B/g). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.calibrate:
        calibrate(args)
        return
    if args.workload_matrix:
        workload_matrix(args)
        return
    if args.path_sweep:
        path_sweep(args)
        return

    import numpy as np
    import torch

    from partitioned_chip_accumulation_amd import hist, inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = inputs.WORKLOADS[args.config]
    n = w.n if args.n is None else args.n
    B = w.num_bins
    t_gen = time.perf_counter()
    if args.uniform_bins:
        B = args.uniform_bins
        w = inputs.Workload(0, f"uniform-{B}", n, B, 1, f"int32 uniform in [0, {B}), seed 1")
        x = inputs.uniform(1, n, B)
    else:
        x = inputs.generate(args.config, n=n)
    t_gen = time.perf_counter() - t_gen
    xs = [torch.from_numpy(x).to(dev)]
    for _ in range(max(0, args.copies - 1)):
        xs.append(xs[0].clone())
    out = torch.empty(B, dtype=torch.int32, device=dev)

    tuned = None
    selected = None
    if args.select:
        # predicted schedule choice on this input, before and outside the timed region
        t0 = time.perf_counter()
        best, rows = hist.select(xs[0], B)
        selected = {"opts": best, "seconds": round(time.perf_counter() - t0, 4),
                    "predicted_us": {r["schedule"]: round(r["predicted_us"], 1)
                                     for r in rows if r["status"] == hist.HIST_OK}}
        plan_opts = best
    elif args.tune:
        # measured schedule choice on this input, before and outside the timed region
        best, rows = hist.tune(xs[0], B, max_n=n, reps=3)
        tuned = {"opts": best, "candidates_ms": {
            f"{r['opts']['path']}{r['opts']['counter_bits'] or ''}"
            f"{'+hot' if r['opts']['aggregation'] == 1 else ''}": round(r["ms"], 4)
            for r in rows if r["status"] == hist.HIST_OK}}
        plan_opts = best
    else:
        plan_opts = dict(path=args.path, groups=args.groups, range_bins=args.range_bins,
                         aggregation=args.agg, wg_size=args.wg, xcd_map=args.xcd_map,
                         counter_bits=args.counter_bits, lds_copies=args.lds_copies,
                         pacing=args.pacing, window=args.window)
    # One plan (and workspace) and one output per stream: the steps on different
    # streams are independent histograms, so they may overlap on the device.
    nstreams = max(1, args.streams)
    two = nstreams != 2 and args.two_streams
    nplans = max(2 if two else 1, nstreams)  # the two-stream figure needs a second plan
    plans = [hist.Plan(B, n, device=dev, **plan_opts) for _ in range(nplans)]
    plan = plans[0]
    streams = [torch.cuda.current_stream(dev)] + [torch.cuda.Stream(dev)
                                                 for _ in range(nplans - 1)]
    outs = [out] + [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(nplans - 1)]
    info = plan.info()
    print(f"# plan: {plan.describe()}  (input generated in {t_gen:.1f} s)", file=sys.stderr,
          flush=True)

    if args.copy_calibration:
        a = torch.empty(args.copy_calibration << 18, dtype=torch.int32, device=dev)
        bcopy = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize(dev)
        hist.copy(bcopy, a)
        torch.cuda.synchronize(dev)
        del a, bcopy

    def step(k: int, ns: int):
        if ns == 1:  # the plain call: one stream, nothing around it
            plan.run(xs[k % len(xs)], out)
        else:
            j = k % ns
            plans[j].run(xs[k % len(xs)], outs[j], stream=streams[j])

    def timed(events: bool, ns: int):
        for p in plans[:ns]:
            p.timing_enable((args.steps + args.warmup) if events else 0)
        settle(lambda k: step(k, ns))
        for k in range(args.warmup):
            step(k, ns)
        torch.cuda.synchronize(dev)
        if events:
            for p in plans[:ns]:
                p.timing_read()  # discard warm-up records
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for k in range(args.steps):
            step(k, ns)
        torch.cuda.synchronize(dev)
        dt = time.perf_counter() - t0
        if not events:
            return dt, None
        merged: dict = {}
        for p in plans[:ns]:
            for name, (ms, cnt) in p.timing_read().items():
                m0, c0 = merged.get(name, (0.0, 0))
                merged[name] = (m0 + ms, c0 + cnt)
            p.timing_enable(0)
        return dt, merged

    # The headline region runs without per-kernel events (attaching them adds
    # host work per launch); a second region of the same length attaches HIP
    # events to every kernel's dispatch, for the roofline figures. With several streams a step is still one whole histogram; the
    # steps of different streams overlap, as a caller's independent histograms
    # on separate streams would.
    elapsed, _ = timed(False, nstreams)
    elapsed_events, phases = timed(True, nstreams)
    elapsed_2 = timed(False, 2)[0] if two else (elapsed if nstreams == 2 else None)

    # Per-step distribution: a third region with one pair of events around
    # each run on the launch stream (the events sit between runs).
    plan.timing_enable(0)
    nstat = min(args.steps, 2000)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(nstat)]
    torch.cuda.synchronize(dev)
    for k in range(nstat):
        ev[k][0].record()
        plan.run(xs[k % len(xs)], out)
        ev[k][1].record()
    torch.cuda.synchronize(dev)
    per_step = np.sort(np.array([a.elapsed_time(b) * 1e3 for a, b in ev]))
    step_us = {"median": round(float(np.median(per_step)), 2), "min": round(float(per_step[0]), 2),
               "p90": round(float(per_step[int(0.9 * (nstat - 1))]), 2), "samples": nstat}

    parity = None
    if not args.no_parity:
        ref = reference_counts(x, B)
        parity = all(bool(np.array_equal(o.view(torch.uint32).cpu().numpy(), ref)) for o in outs)

    ms_per_step = elapsed / args.steps * 1e3
    gelem = n * args.steps / elapsed / 1e9
    alg_bytes = 4 * n + 4 * B
    gbps = alg_bytes * args.steps / elapsed / 1e9

    # Dominant kernel: the phase with the most device time.
    roofline = roofline_for(phases, n, B, f"{w.name}:n={n}:{plan.describe()}")
    if 4 * n * len(xs) <= 256 * 2**20:
        # all input copies fit the 256 MB Infinity Cache: the steps are served
        # from it, and kernel launches dominate
        roofline["note"] = ("input copies fit the 256 MB Infinity Cache; launch- and "
                            "cache-bound, so the HBM fraction is not meaningful")

    # The other four workloads at full size, AUTO's plan, each checked bit for
    # bit (after the headline, so that nothing runs between its regions).
    workloads = None
    if not args.no_workloads and args.config == 2 and args.n is None and not args.uniform_bins \
            and nstreams == 1 and not args.tune and not args.select:
        workloads = {}
        for cfg in (1, 3, 4, 5):
            wk = inputs.WORKLOADS[cfg]
            workloads[wk.name] = time_workload(cfg, args.steps, args.warmup, dev,
                                               check=not args.no_parity,
                                               comparators=args.comparators)
            torch.cuda.empty_cache()

    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        oracle.hist(x[:1024], B)  # build/load outside the timing
        reps, spent, t_start = 0, 0.0, time.perf_counter()
        while True:
            t1 = time.perf_counter()
            oracle.hist(x, B)
            spent += time.perf_counter() - t1
            reps += 1
            if time.perf_counter() - t_start >= args.cpu_seconds or reps >= 10000:
                break
        model = ""
        try:
            with open("/proc/cpuinfo") as f:
                model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
        except OSError:
            pass
        cpu = {"value": round(n * reps / spent / 1e9, 4), "unit": "Gelem/s", "cores": 1,
               "kind": "oracle",
               "host": {"cpu_model": model, "usable_cores": len(os.sched_getaffinity(0)),
                        "cpu_count": os.cpu_count()},
               "sample": f"{reps} full passes of the timed input ({n} elements each), "
                         f"{spent:.1f} s, sequential loop on one host core "
                         f"(host has {len(os.sched_getaffinity(0))} usable cores)"}

    comparators = None
    if args.comparators:
        comparators = comparator_figures(xs, B, reference_counts(x, B))

    line = {
        "metric": "Gelem/s and achieved HBM GB/s vs peak, 65,536-bin int32 histogram, 1 MI355X",
        "value": round(gelem, 2),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "achieved_GBps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "parity_vs_bincount": parity,
        "config": {"workload": f"{w.name}: {w.recipe}; n={n}, {B} uint32 bins",
                   "n": n, "num_bins": B, "plan": plan.describe(),
                   "input_copies": len(xs), "streams": nstreams,
                   **({"tuned": tuned} if tuned else {}),
                   **({"selected": selected} if selected else {})},
        "phases_ms_per_step": {k: round(v[0] / v[1], 5) for k, v in phases.items()},
        "ms_per_step_with_events": round(elapsed_events / args.steps * 1e3, 5),
        "step_us_event_bracketed": step_us,
        "two_streams": None if elapsed_2 is None else {
            "ms_per_step": round(elapsed_2 / args.steps * 1e3, 5),
            "value": round(n * args.steps / elapsed_2 / 1e9, 2)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if comparators is not None:
        line["comparators"] = comparators
    line["workloads"] = workloads
    print(json.dumps(line), flush=True)
    for p in plans:
        p.close()


if __name__ == "__main__":
    main()
