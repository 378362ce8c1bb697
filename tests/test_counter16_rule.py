"""CPU check of the decode rule behind the 16-bit LDS counters (no GPU).

Two bins share a 32-bit word; the low bin adds 1 (or k after aggregation),
the high bin adds 1 << 16 (or k << 16). From the old value an add returns,
the kernels log two kinds of event: the low half wrapping (L) and a carry out
of the word (C). The flush recovers the exact counts as
    lo = (W & 0xFFFF) + 65536 L,   hi = (W >> 16) + 65536 C - L   (mod 2^32).
This test replays random add sequences, including words that start with one
or both halves full, and checks the rule against the true counts, using the
same event tests as the kernels (the general form for any k and the k = 1
form of the unaggregated batch path).
"""
import random

import pytest

M = 0xFFFFFFFF


def events_general(old, hi, k):
    delta = (k << 16) if hi else k
    lo_wrap = (not hi) and (old & 0xFFFF) + k > 0xFFFF
    carry = old > M - delta
    return lo_wrap, carry


def events_k1(old, hi):
    half = (old >> 16) if hi else (old & 0xFFFF)
    if half != 0xFFFF:
        return False, False
    return (not hi), (hi or (old >> 16) == 0xFFFF)


@pytest.mark.parametrize("seed", range(4))
def test_decode_rule(seed):
    rnd = random.Random(seed)
    for _ in range(40):
        w, L, C, true = 0, 0, 0, [0, 0]
        if rnd.random() < 0.4:
            lo0, hi0 = rnd.choice([(65535, 65535), (65534, 65535), (65535, 0), (0, 65535)])
            true = [lo0, hi0]
            w = lo0 + (hi0 << 16)
        p_hi = rnd.random()
        for _ in range(rnd.choice([10, 5000, 70000, 140000])):
            hi = rnd.random() < p_hi
            k = rnd.choice([1, 1, 1, 1, 3, 64]) if seed % 2 else 1
            old = w
            w = (w + ((k << 16) if hi else k)) & M
            true[hi] += k
            lw, cy = events_general(old, hi, k)
            if k == 1:
                assert (lw, cy) == events_k1(old, hi)
            L += lw
            C += cy
        lo = (w & 0xFFFF) + 65536 * L
        hi_ = ((w >> 16) + 65536 * C - L) & M
        assert (lo, hi_) == (true[0], true[1])
