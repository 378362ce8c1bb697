"""The two-phase path splits the concatenation of all ranges' elements (N
positions) over W owners: owner i takes [floor(i*N/W), floor((i+1)*N/W)).
The owner kernel decides from its own span whether it holds a range whole
(and then writes the range's counts itself); the slot merge finds a range's
owners with owner_of(p) = floor(((p+1)*W - 1)/N) and skips a range whose
first and last positions have the same owner. Exactly one side may write
each bin, so the two rules must agree: owner_of(p) is the i whose span holds
p, for every N and W. (Both formulas as the kernels use them, in
hist_scatter.hpp.)"""
from __future__ import annotations

import random


def spans(N, W):
    return [(i * N // W, (i + 1) * N // W) for i in range(W)]


def owner_of(p, N, W):
    return ((p + 1) * W - 1) // N


def test_owner_of_names_the_span_holding_the_position():
    for N in range(1, 300):
        for W in range(1, 60):
            s = spans(N, W)
            for p in range(N):
                e0, e1 = s[owner_of(p, N, W)]
                assert e0 <= p < e1, (N, W, p)


def test_whole_range_rule_matches_the_merge_skip_at_large_sizes():
    rng = random.Random(7)
    for _ in range(2000):
        N = rng.randrange(1, 2**32)
        W = rng.choice([1, 3, 100, 256, 600])
        rb = rng.randrange(0, N)
        re = rng.randrange(rb + 1, min(N, rb + 2**20) + 1)
        i = owner_of(rb, N, W)
        e0, e1 = i * N // W, (i + 1) * N // W
        whole = e0 <= rb and re <= e1                              # owner kernel
        single = owner_of(rb, N, W) == owner_of(re - 1, N, W)      # slot merge
        assert whole == single, (N, W, rb, re)
