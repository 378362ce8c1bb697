"""The streaming owner-queue path's protocol, run on the CPU (no GPU).

The page "Distributed Shared Memory", section "The cluster histogram", sends
every increment to the block that owns its bin; the page "Hopper DSMEM vs
HBM" passes data between blocks through a flag in memory (its latency test).
The STREAM path does the same with workgroups in one persistent kernel:
producers route input tiles by owning range and publish each tile with a
flag; owners claim blocks of tiles for the range they hold and wait for the
flags; an owner whose range runs out writes its counts (a stint) to the next
slot of a pool and moves, from a budget of moves, to the range with the most
blocks left; a merge step then sums each range's stints into the output.

This is a step-by-step model of that protocol, in the kernel's order of
shared-memory operations: every workgroup is a generator that yields at each
one, and a seeded scheduler picks which workgroup moves next, starts
workgroups late (as a GPU does when not all are resident) and lets some sit
idle for long stretches. The tests check that every workgroup finishes (no
wait without end: producers never wait, owners wait only on tiles that a
started producer will publish), that the stints fit the pool, that every
(tile, range) run is counted exactly once, and that the counts equal the
histogram.
"""
from __future__ import annotations

import random

import numpy as np
import pytest


class Shared:
    def __init__(self, tiles, ranges):
        self.ticket = 0
        self.tile_next = 0
        self.flag = [0] * tiles
        self.claim = [0] * ranges
        self.slots = 0  # stint counter
        self.moves = 0  # move counter
        self.pool = {}  # slot -> (range, counts)
        self.counted = {}  # (tile, range) -> times counted


def workgroup(sh, data, num_bins, S, R, T, BT, NB, P, budget, log):
    """One workgroup of the persistent kernel, yielding at each shared access."""
    ticket = sh.ticket
    sh.ticket += 1
    yield "ticket"
    if ticket < P:  # producer
        while True:
            t = sh.tile_next
            sh.tile_next += 1
            yield "claim tile"
            if t >= T:
                break
            yield "route tile"  # the tile's runs, staged and tabled
            sh.flag[t] = 1  # published
            yield "publish"
    # owner
    cur = ticket % R
    slice_ = None
    while True:
        b = sh.claim[cur]
        sh.claim[cur] += 1
        yield "claim block"
        if b < NB:
            if slice_ is None:
                slice_ = np.zeros(S, np.int64)
            for t in range(b * BT, min((b + 1) * BT, T)):  # wait for the block's tiles
                spins = 0
                while sh.flag[t] == 0:
                    spins += 1
                    assert spins < 100000, "flag wait without end"
                    yield "wait flag"
            for t in range(b * BT, min((b + 1) * BT, T)):  # count range cur's runs
                part = data[t]
                run = part[part // S == cur] % S
                np.add.at(slice_, run, 1)
                sh.counted[(t, cur)] = sh.counted.get((t, cur), 0) + 1
            yield "count block"
            continue
        if slice_ is not None:  # the stint goes to the next pool slot
            slot = sh.slots
            sh.slots += 1
            yield "take slot"
            sh.pool[slot] = (cur, slice_)
            yield "write stint"
            slice_ = None
        left = [(NB - sh.claim[q], q) for q in range(R) if sh.claim[q] < NB]
        yield "scan claims"
        if not left:
            break
        m = sh.moves
        sh.moves += 1
        yield "take move"
        if m >= budget:
            break
        cur = max(left)[1]
    log.append(ticket)


def merge(sh, num_bins, S, R, counts, accumulate):
    """The merge step: each range's stints summed into its output bins."""
    for r in range(R):
        total = np.zeros(S, np.int64)
        for rr, c in sh.pool.values():
            if rr == r:
                total += c
        lo, ln = r * S, min(S, num_bins - r * S)
        counts[lo:lo + ln] = (counts[lo:lo + ln] if accumulate else 0) + total[:ln]


def run_protocol(seed, n, num_bins, W, P, BT, tile=64, accumulate=False, start=None, budget=None):
    rng = random.Random(seed)
    x = np.random.default_rng(seed).integers(-3, num_bins + 3, size=n)
    S = 32768
    R = (num_bins + S - 1) // S
    T = max(1, (n + tile - 1) // tile)
    NB = (T + BT - 1) // BT
    budget = 3 * W if budget is None else budget
    pool_slots = min(W + budget, R * NB)
    data = [x[t * tile:(t + 1) * tile] for t in range(T)]
    data = [d[(d >= 0) & (d < num_bins)] for d in data]
    counts = np.full(num_bins, 7 if accumulate else -1, np.int64)
    base = counts.copy()
    sh = Shared(T, R)
    log = []
    gens = [workgroup(sh, data, num_bins, S, R, T, BT, NB, P, budget, log) for _ in range(W)]
    # workgroups start at random moments; a started one may sit idle for a while
    start = start or [rng.randint(0, 200) for _ in range(W)]
    live, clock, steps = [], 0, 0
    pending = sorted(range(W), key=lambda i: start[i])
    while pending or live:
        while pending and start[pending[0]] <= clock:
            live.append(pending.pop(0))
        clock += 1
        if not live:
            continue
        g = rng.choice(live) if rng.random() < 0.9 else live[0]
        try:
            next(gens[g])
        except StopIteration:
            live.remove(g)
        steps += 1
        assert steps < 5_000_000, "the protocol did not finish"
    assert sh.slots <= pool_slots, "more stints than pool slots"
    merge(sh, num_bins, S, R, counts, accumulate)
    want = np.bincount(x[(x >= 0) & (x < num_bins)], minlength=num_bins)
    if accumulate:
        want = want + base
    return counts, want, sh, T, R, log


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("num_bins,W,P,BT", [(1 << 17, 6, 3, 2), (100_000, 5, 1, 3),
                                             (40_000, 8, 7, 1), (1 << 16, 3, 3, 4)])
def test_every_workgroup_finishes_and_counts_are_exact(seed, num_bins, W, P, BT):
    counts, want, sh, T, R, log = run_protocol(seed, 3000, num_bins, W, P, BT)
    assert sorted(log) == list(range(W))  # every workgroup ended
    assert np.array_equal(counts, want)
    # every (tile, range) run counted exactly once
    assert sh.counted == {(t, r): 1 for t in range(T) for r in range(R)}


def test_accumulate_adds_every_stint():
    counts, want, *_ = run_protocol(3, 2500, 1 << 17, 5, 2, 2, accumulate=True)
    assert np.array_equal(counts, want)


def test_owners_that_start_first_wait_for_late_producers():
    # the producers start last: owners wait on flags until a producer starts
    W, P = 6, 2
    start = [500 + i if i < P else i for i in range(W)]
    # tickets follow start order, so the late workgroups take the producer tickets
    counts, want, sh, T, R, log = run_protocol(11, 2000, 1 << 17, W, P, 2,
                                               start=sorted(start))
    assert np.array_equal(counts, want) and sorted(log) == list(range(W))


def test_one_workgroup_does_everything():
    counts, want, *_ = run_protocol(5, 1000, 1 << 17, 1, 1, 3)
    assert np.array_equal(counts, want)


@pytest.mark.parametrize("seed", range(4))
def test_a_spent_move_budget_still_counts_everything(seed):
    # no moves at all: every owner stays on its first range, which it leaves
    # only when the range's last block is claimed
    counts, want, sh, T, R, log = run_protocol(seed, 3000, 1 << 17, 6, 3, 2, budget=0)
    assert np.array_equal(counts, want) and sorted(log) == list(range(6))
    assert sh.slots <= 6
