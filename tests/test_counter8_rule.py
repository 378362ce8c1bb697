"""CPU check of the decode rule behind the 8-bit LDS counters (no GPU).

Four bins share a 32-bit word, bin p in byte p; an add of k (1 <= k <= 255)
to bin p adds k << 8p to the word. A byte that overflows carries into the
next byte of the word, which may overflow in turn, and a carry out of byte 3
leaves the word. From the old value an add returns, the kernels log one
event per byte p that carried out: the carry into bit 8p + 8 is that bit of
old ^ delta ^ new for p < 3, and a carry out of the word shows as new < old.
With C_p the carries out of byte p, the flush recovers the exact counts as
    A_p = byte_p(W) + 256 C_p - C_(p-1)   (C_-1 = 0).
This test replays random add sequences, including words that start with
bytes at 0xFF (so that one add cascades through several bytes), checks the
rule against the true counts, checks the k = 1 screen the kernels use
(an event is possible only when the incremented byte was 0xFF), and checks
the bound of at most E / 255 events for E counted elements.
"""
import random

import pytest

M = 0xFFFFFFFF


def carries(old, p, k):
    """Bytes q >= p that carried out when k << 8p was added to old."""
    delta = (k << (8 * p)) & M
    new = (old + delta) & M
    x = old ^ delta ^ new
    out = [q for q in range(3) if (x >> (8 * q + 8)) & 1]
    if new < old:
        out.append(3)
    return out, new


def screen_k1(old, p):
    return ((old >> (8 * p)) & 0xFF) == 0xFF


@pytest.mark.parametrize("seed", range(6))
def test_decode_rule(seed):
    rnd = random.Random(seed)
    for _ in range(40):
        w, C, true, events, added = 0, [0, 0, 0, 0], [0, 0, 0, 0], 0, 0
        if rnd.random() < 0.5:
            init = [rnd.choice([0, 1, 0xFE, 0xFF]) for _ in range(4)]
            true = list(init)
            w = sum(b << (8 * q) for q, b in enumerate(init))
        weights = [rnd.random() for _ in range(4)]
        for _ in range(rnd.choice([10, 700, 5000, 70000])):
            p = rnd.choices(range(4), weights)[0]
            k = rnd.choice([1, 1, 1, 1, 3, 200, 255]) if seed % 2 else 1
            out, new = carries(w, p, k)
            if k == 1:
                assert screen_k1(w, p) == bool(out)
            for q in out:
                assert q >= p
                C[q] += 1
            events += len(out)
            added += k
            w = new
            true[p] += k
        got = [(((w >> (8 * q)) & 0xFF) + 256 * C[q] - (C[q - 1] if q else 0)) & M
               for q in range(4)]
        assert got == true
        # one add of k <= 255 carries out of each byte at most once, and every
        # carry out of byte q needs 256 units into it: events <= E / 255
        assert events <= added // 255 + 4
