"""Host-side pieces of bench.py (no GPU): the stored-counter lookup and its
source guard, the measurement modes' reference, and the one-GPU guard."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_counters_are_used_only_for_the_current_kernel_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    key = "sweep:w:n=1:plan"
    f.write_text(json.dumps({key: {"kernel_source_sha": bench.kernel_source_sha(),
                                   "bytes_per_launch": 123}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.counters_for(key)["bytes_per_launch"] == 123
    assert bench.counters_for("other") == {}
    f.write_text(json.dumps({key: {"kernel_source_sha": "0" * 64, "bytes_per_launch": 123}}))
    assert bench.counters_for(key) == {}  # counters taken from other kernel sources
    f.write_text("not json")
    assert bench.counters_for(key) == {}


def test_committed_profiles_match_the_kernel_sources():
    # the counter and kernel-trace entries under profiles/ were taken from the
    # kernels as committed (each entry names the sources its hash covers)
    for path in (bench.TRAFFIC_FILE, bench.KERNEL_TIMES_FILE):
        with open(path) as fh:
            data = json.load(fh)
        stale = [k for k, e in data.items()
                 if e["kernel_source_sha"] != bench.kernel_source_sha(e.get("sources"))]
        assert data and not stale, (path, stale)
        assert any(k.startswith("sweep:uniform-64k:") for k in data)


def test_reference_counts_skip_values_outside_the_bins():
    x = np.array([0, 1, 1, -1, 5, 4, 2**31 - 1, -2**31, 3], dtype=np.int32)
    ref = bench.reference_counts(x, 5)
    assert ref.dtype == np.uint32 and ref.tolist() == [1, 2, 0, 1, 1]


def test_more_than_one_gpu_is_refused_before_any_device_call():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_the_roofline_follows_the_kernel_that_reads_the_input():
    # a launch-bound input whose merge took as long as its sweep
    name, nbytes, avg_s, launches = bench.dominant_kernel(
        {"sweep": (4.31, 1), "merge": (4.84, 1)}, n=1 << 20, B=8192)
    assert (name, nbytes, launches) == ("sweep", 4 << 20, 1)
    assert avg_s == pytest.approx(4.31e-3)
    # the two-phase path: the partition, not the longer owner phase
    name, nbytes, _, _ = bench.dominant_kernel(
        {"partition": (3.0, 10), "owner_hist": (4.0, 10), "slot_merge": (0.2, 10)}, n=1000, B=10)
    assert (name, nbytes) == ("partition", 4000)
    # no reader timed: the longest phase, priced at the bins it writes
    name, nbytes, _, _ = bench.dominant_kernel({"merge": (1.0, 2)}, n=1000, B=10)
    assert (name, nbytes) == ("merge", 40)
