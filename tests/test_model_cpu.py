"""The schedule cost model (hist_predict), host only.

The model predicts each schedule's time from primitive rates, a baseline read
rate, each schedule's traffic and a sample of the input (the cost-guided
selection of "CREDIT: Cost-guided Reduction-reuse with Efficient DSMEM
Inter-CTA Tiling", its cost model section). These tests pin its mechanics on
inputs whose statistics are known, and its choices against the schedules'
measured times committed under profiles/: the measured tables are the
evidence the predictions are checked against, and nothing in the model was
fitted to them.
"""
from __future__ import annotations

import json
import os
import re

import numpy as np
import pytest

from partitioned_chip_accumulation_amd import hist, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
MS = 1 << 16  # sample elements


def by_name(rows):
    return {r["schedule"]: r for r in rows}


def test_calibration_figures_are_the_probes():
    c = hist.model_calibration()
    assert c.read_gbps > 1000 and c.copy_gbps > 1000 and c.clock_ghz == 2.4
    assert c.lds_cycles == 7.3 and abs(c.lds_dup_cycles - (30.1 - 7.3) / 56) < 1e-3
    assert 0 < c.launch_us < 20 and 0 < c.sweep_fixed_us < 20 and 0 < c.scatter_fixed_us < 100
    assert 0 < c.event_cycles < 1000


def test_terms_follow_the_schedules_traffic():
    n, B = 1 << 26, 1 << 19
    best, rows = hist.predict(B, n, inputs.uniform(1, MS, B))
    r = by_name(rows)
    one_pass = 4 * n / (hist.model_calibration().read_gbps * 1e3)
    # each owned range is one pass over the input
    for name in ("range8", "range16", "range32"):
        info = hist.preview(B, n, **r[name]["opts"])
        assert r[name]["pass_us"] == pytest.approx(info.ranges * one_pass, rel=1e-9)
    # full slices are allowed only where they fit
    assert r["full16"]["status"] == hist.HIST_ERR_UNSUPPORTED and r["full16"]["predicted_us"] == -1
    # the two-phase path: the input, 2-byte slots written and read back
    assert r["scatter"]["pass_us"] > one_pass
    assert best == min((x for x in rows if x["status"] == 0),
                       key=lambda x: x["predicted_us"])["opts"]


def test_carry_events_appear_only_where_counts_wrap():
    n = 1 << 26
    # uniform over 1,024 bins: 256 chunks of 2^18 elements put about 256 adds on
    # every bin of a chunk, so 8-bit counters wrap; 16-bit ones never do
    r = by_name(hist.predict(1024, n, inputs.uniform(1, MS, 1024))[1])
    assert r["full8"]["events_us"] > 0 and r["full16"]["events_us"] == 0
    # over 16,384 bins a chunk puts 16 adds on a bin: no wraps at all
    r = by_name(hist.predict(16384, n, inputs.uniform(1, MS, 16384))[1])
    assert r["full8"]["events_us"] == 0
    # one value holding everything wraps once every 256 adds: n / 256 events
    hot = np.full(MS, 77, np.int32)
    r = by_name(hist.predict(16384, n, hot)[1])
    c = hist.model_calibration()
    cyc_us = 1.0 / (256 * c.clock_ghz * 1e3)
    assert r["full8"]["events_us"] == pytest.approx(n / 256 * c.event_cycles * cyc_us, rel=0.01)


def test_same_word_lanes_and_the_hot_slot():
    B = 1 << 20
    x = inputs.uniform(1, MS, B)
    x[::10] = 524287  # a tenth of the input on one value
    # below 2^22 elements the two-phase path samples nothing: the hot value's
    # lanes collide on its word, and the owners' hot slot takes them out of
    # the LDS atomics again
    n = 1 << 21
    uni = by_name(hist.predict(B, n, inputs.uniform(1, MS, B))[1])
    hot = by_name(hist.predict(B, n, x)[1])
    assert hot["scatter"]["lds_us"] > uni["scatter"]["lds_us"]
    assert hot["scatter+hot"]["lds_us"] < hot["scatter"]["lds_us"]
    assert uni["scatter+hot"]["lds_us"] == pytest.approx(uni["scatter"]["lds_us"], rel=0.02)
    # from 2^22 the sample names the value, the partition counts it in
    # registers, and the owners see the other nine tenths with no contention
    n = 1 << 26
    uni = by_name(hist.predict(B, n, inputs.uniform(1, MS, B))[1])
    hot = by_name(hist.predict(B, n, x)[1])
    assert hot["scatter"]["lds_us"] == pytest.approx(0.9 * uni["scatter"]["lds_us"], rel=0.03)
    assert hot["scatter"]["pass_us"] < uni["scatter"]["pass_us"]


def test_values_outside_the_bins_cost_no_atomics():
    n, B = 1 << 24, 65536
    inside = by_name(hist.predict(B, n, inputs.uniform(2, MS, B))[1])
    half = inputs.uniform(2, MS, B)
    half[::2] = -5
    outside = by_name(hist.predict(B, n, half)[1])
    assert outside["full16"]["lds_us"] == pytest.approx(inside["full16"]["lds_us"] / 2, rel=0.05)
    assert outside["full16"]["pass_us"] == inside["full16"]["pass_us"]  # still read


def test_argument_errors():
    lib = hist.library()
    best = hist.PlanOpts()
    dev = hist.mi355x()
    import ctypes
    assert lib.hist_predict(None, None, 10, 10, None, 0, ctypes.byref(best), None, 0,
                            None) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_predict(ctypes.byref(dev), None, 0, 10, None, 0, ctypes.byref(best), None, 0,
                            None) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_predict(ctypes.byref(dev), None, 10, 0, None, 0, ctypes.byref(best), None, 0,
                            None) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_predict(ctypes.byref(dev), None, 10, 10, None, 5, ctypes.byref(best), None, 0,
                            None) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_predict(ctypes.byref(dev), None, hist.MAX_BINS + 1, 10, None, 0,
                            ctypes.byref(best), None, 0, None) == hist.HIST_ERR_UNSUPPORTED
    bad = hist.model_calibration()
    bad.read_gbps = 0
    assert lib.hist_predict(ctypes.byref(dev), ctypes.byref(bad), 10, 10, None, 0,
                            ctypes.byref(best), None, 0, None) == hist.HIST_ERR_INVALID_ARG
    # no device needed for any of this; hist_select refuses before touching one
    assert lib.hist_select(10, None, 10, None, None, 0, None, ctypes.byref(best), None, 0,
                           None) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_select(10, 16, 10, None, None, 0, None, ctypes.byref(best), None, 0,
                           None) == hist.HIST_ERR_WORKSPACE


def measured_tables():
    """The committed measurements: {row label: (input kind, bins, n, {schedule: us})}."""
    rows = {}

    def read(path, kind_of):
        hdr = None
        for line in open(os.path.join(PROFILES, path)):
            line = line.rstrip("\n")
            if line.startswith("| bins") or line.startswith("| workload"):
                hdr = [c.strip() for c in line.strip("|").split("|")]
                continue
            if hdr and line.startswith("| ") and not line.startswith("|---"):
                cells = [c.strip().replace("**", "") for c in line.strip("|").split("|")]
                kind, B, n = kind_of(cells[0])
                rows[f"{path}: {cells[0]}"] = (kind, B, n, {
                    h: float(c) for h, c in zip(hdr[1:], cells[1:])
                    if c and "FAIL" not in c and h != "auto"})
            elif not line.startswith("|"):
                hdr = None if line.startswith("AUTO") else hdr

    def pow2(label):
        return 1 << int(re.match(r"2\^(\d+)", label).group(1))

    read("path_selection_uniform_n2p26.md", lambda l: ("uniform", pow2(l), 1 << 26))
    read("path_selection_zipf1.1_n2p26.md", lambda l: ("zipf", pow2(l), 1 << 26))
    cfg = {w.name: c for c, w in inputs.WORKLOADS.items()}
    read("path_matrix_workloads.md",
         lambda l: (str(cfg[l]), inputs.WORKLOADS[cfg[l]].num_bins, inputs.WORKLOADS[cfg[l]].n))
    return rows


def sample_of(kind, B):
    if kind == "uniform":
        return inputs.uniform(1, MS, B)  # the sweeps' seed
    if kind == "zipf":
        return inputs.zipf(2, MS, B, 1.1)
    return inputs.generate(int(kind), n=MS)


def test_predicted_choice_against_the_measured_schedules():
    """On every row of the committed path-selection sweeps (uniform and Zipf
    input, 2^26 elements) and of the five-workload matrix, the schedule the
    model predicts fastest, among those the row measured, must take at most
    5% longer than the fastest measured one on at least 90% of the rows."""
    rows = measured_tables()
    assert len(rows) == 25
    misses = []
    for label, (kind, B, n, meas) in rows.items():
        _, preds = hist.predict(B, n, sample_of(kind, B))
        pred = {p["schedule"]: p["predicted_us"] for p in preds
                if p["status"] == hist.HIST_OK and p["schedule"] in meas}
        pick = min(pred, key=pred.get)
        best = min(meas, key=meas.get)
        if meas[pick] > 1.05 * meas[best]:
            misses.append(f"{label}: predicted {pick} ({meas[pick]} us), fastest {best} "
                          f"({meas[best]} us)")
    print("\n".join(misses))
    assert len(misses) <= len(rows) // 10, misses
