"""Pins for the seeded input generator (no GPU needed).

The generator draws inputs only; parity never depends on it, since the GPU
path and the oracle read the same bytes. These tests make sure it is the
published SplitMix64, deterministic, parallel-safe, and that each workload has
the shape its recipe promises (uniform spread, Zipf head mass, the exact hot
bin count, the Gaussian mass on the range boundary).
"""
from __future__ import annotations

import hashlib
import json
import os

import numpy as np
import pytest

from partitioned_chip_accumulation_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "inputs_sha256.json")


def test_splitmix64_matches_published_sequence():
    # SplitMix64 from state 0 (Steele, Lea & Flood, OOPSLA 2014; the public
    # reference implementation): its first three outputs.
    got = [int(v) for v in inputs.stream(0, 0, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_stream_is_counter_based():
    k = inputs.key(7, inputs.TAG_UNIFORM)
    whole = inputs.stream(k, 0, 10_000)
    assert np.array_equal(whole[1234:5678], inputs.stream(k, 1234, 5678 - 1234))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_generation_is_deterministic(cfg):
    a = inputs.generate(cfg, n=100_003)
    b = inputs.generate(cfg, n=100_003)
    assert np.array_equal(a, b)
    w = inputs.WORKLOADS[cfg]
    assert a.min() >= 0 and a.max() < w.num_bins


def test_seeds_differ():
    assert not np.array_equal(inputs.uniform(0, 1000, 1 << 16), inputs.uniform(1, 1000, 1 << 16))


def test_uniform_chi_square():
    x = inputs.generate(1)
    counts = np.bincount(x, minlength=8192)
    expected = x.size / 8192
    chi2 = float(((counts - expected) ** 2 / expected).sum())
    # 8191 degrees of freedom: mean 8191, sd ~128; allow 6 sd.
    assert abs(chi2 - 8191) < 6 * 128


def test_uniform_non_power_of_two_range():
    x = inputs.uniform(3, 200_000, 1000, lo=-10)
    assert x.min() == -10 and x.max() == 989


def test_zipf_head_mass():
    n = 1 << 22
    x = inputs.generate(3, n=n)
    k = np.arange(1, 262_145, dtype=np.float64)
    p1 = 1.0 / np.sum(k ** -1.1)
    top = np.bincount(x, minlength=262_144).max() / n
    assert abs(top - p1) < 5 * np.sqrt(p1 * (1 - p1) / n)
    assert abs(p1 - 0.1297) < 0.001


def test_hot_bin_exact_count_and_spread():
    n = 1 << 22
    x, uniform_hits = inputs.generate(4, n=n, return_aux=True)
    assert int(np.sum(x == 524287)) == n // 10 + uniform_hits
    # shuffled: the hot value is spread evenly, not packed at the front
    first = np.mean(x[: n // 10] == 524287)
    assert abs(first - 0.1) < 0.01


def test_gaussian_half_shape():
    n = 1 << 22
    x, gauss_at_or_above = inputs.generate(5, n=n, return_aux=True)
    near = np.abs(x.astype(np.int64) - 262144) <= 3000
    # the Gaussian half is almost all within 3 sigma; the uniform half adds
    # 6001/2^19 of its mass there.
    expected = 0.5 * 0.9973 + 0.5 * 6001 / 2**19
    assert abs(near.mean() - expected) < 0.005
    assert abs(gauss_at_or_above / (n - n // 2) - 0.5002) < 0.002


def test_golden_hashes():
    with open(GOLDEN) as f:
        golden = json.load(f)
    for cfg, entry in golden["inputs"].items():
        x = inputs.generate(int(cfg), n=entry["n"])
        assert hashlib.sha256(x.tobytes()).hexdigest() == entry["sha256"], cfg


def test_zipf_any_size_matches_the_workload_recipe():
    # inputs.zipf is the 262,144-bin Zipf workload's generator with its size and exponent free
    n = 200_003
    assert np.array_equal(inputs.zipf(2, n, 262_144, 1.1), inputs.generate(3, n=n))
    x = inputs.zipf(7, 100_000, 1000, 1.5)
    assert x.min() >= 0 and x.max() < 1000
    # a heavier exponent concentrates more mass in the top bin
    top = lambda v: np.bincount(v).max() / v.size  # noqa: E731
    assert top(x) > top(inputs.zipf(7, 100_000, 1000, 1.1))
