"""The packed-sequence work map of the preparation kernels, modelled on the host (no GPU).

Sequence s owns slots [B_s, B_{s+1}) with B_s = floor(cu[s] / C) + s; the kernel finds the sequence
of a slot by a 64-ary search over B and skips slots past a sequence's last chunk.  These tests check
the arithmetic the kernel relies on: every chunk of every sequence is reached by exactly one slot,
a sequence has at most one empty slot, the host's slot count floor(T / C) + N covers all of them,
and the search (same steps as the device code) returns the right sequence for N up to 5000."""
import numpy as np
import pytest


def search(cu, C, slot):
    """The device search: lanes probe lo + lane * step, the highest lane with B <= slot wins."""
    lo, hi = 0, len(cu) - 1
    rounds = 0
    while True:
        rounds += 1
        step = (hi - lo + 63) // 64
        s = lo + np.arange(64) * step
        inside = s < hi
        B = np.where(inside, cu[np.minimum(s, len(cu) - 1)] // C + s, 0)
        below = inside & (B <= slot)
        assert below[0]
        L = int(np.nonzero(below)[0].max())
        lo += L * step
        hi = min(lo + step, hi)
        if step == 1:
            break
    c = slot - (cu[lo] // C + lo)
    n = (cu[lo + 1] - cu[lo] + C - 1) // C
    return lo, (c if c < n else -1), rounds


def random_cu(rng, n, lo, hi, zero_frac=0.0):
    lens = rng.integers(lo, hi + 1, size=n)
    lens[rng.random(n) < zero_frac] = 0
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


@pytest.mark.parametrize("C", [32, 64, 128])
@pytest.mark.parametrize("n,lo,hi,zero_frac", [(1, 1, 300, 0.0), (8, 300, 16384, 0.0),
                                                (64, 1, 65, 0.0), (65, 1, 200, 0.2),
                                                (1200, 1, 129, 0.05), (5000, 1, 33, 0.1)])
def test_every_chunk_once(C, n, lo, hi, zero_frac):
    rng = np.random.default_rng(n * 1000 + C)
    cu = random_cu(rng, n, lo, hi, zero_frac)
    T = int(cu[-1])
    slots = T // C + n                       # the host's slot count
    B = cu // C + np.arange(n + 1)
    assert np.all(np.diff(B) >= 1)
    nchunks = (np.diff(cu) + C - 1) // C
    surplus = np.diff(B) - nchunks
    assert surplus.min() >= 0 and surplus.max() <= 1
    assert B[n] == slots
    seen = set()
    for slot in range(slots):
        s, c, rounds = search(cu, C, slot)
        # one round trip while N <= 64, at most ceil(log64 N) in general
        assert rounds <= max(1, int(np.ceil(np.log(n) / np.log(64) - 1e-12)))
        assert n > 64 or rounds == 1
        assert B[s] <= slot < B[s + 1]
        if c >= 0:
            assert (s, c) not in seen
            seen.add((s, c))
    assert len(seen) == int(nchunks.sum())
