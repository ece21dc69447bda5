"""The tile-dealing tables of the C = 128 backward kernel (csrc/wy_backward.hip), read from the
source: every lower 16x16 tile is dealt exactly once per phase, and the work per wave is as
balanced as the comments state.  Host only (no GPU)."""
import os
import re

import pytest

SRC = os.path.join(os.path.dirname(__file__), "..", "chunkwise_gated_deltanet_amd", "csrc", "wy_backward.hip")
LOWER = {(i, j) for i in range(8) for j in range(i + 1)}


def table(name):
    text = open(SRC).read()
    m = re.search(r"__constant__ unsigned char " + name + r"\[[^\]]*\](?:\[[^\]]*\])*\s*=\s*\{(.*?)\};", text, re.S)
    assert m, name
    body = re.sub(r"//[^\n]*", "", m.group(1))
    return [int(x) for x in re.findall(r"\d+", body)]


def per_wave(flat, width):
    return [[c for c in flat[w * width:(w + 1) * width] if c != 255] for w in range(8)]


def test_y_tiles_cover_the_lower_triangle_with_equal_steps():
    waves = per_wave(table("kYTiles"), 8)
    tiles = [(c >> 3, c & 7) for w in waves for c in w]
    assert sorted(tiles) == sorted(LOWER)                  # each lower tile once
    steps = [sum((c & 7) + 1 for c in w) for w in waves]    # Y(Mt, J) costs J + 1 steps
    assert steps == [15] * 8
    assert all(steps[w] + steps[w + 4] == 30 for w in range(4))


def test_m_tiles_cover_the_lower_triangle_with_equal_steps():
    waves = per_wave(table("kMTiles"), 5)
    tiles = [(c >> 3, c & 7) for w in waves for c in w]
    assert sorted(tiles) == sorted(LOWER)
    steps = [sum(8 - (c >> 3) for c in w) for w in waves]   # M(I, J) costs 8 - I steps
    assert steps == [15] * 8
    assert sorted(len(w) for w in waves) == [4, 4, 4, 4, 5, 5, 5, 5]


def test_x_segments_cover_the_lower_triangle():
    flat = table("kXSeg")
    assert len(flat) == 6 * 2 * 3
    tiles, counts = [], []
    for w in range(6):
        n = 0
        for s in range(2):
            I, J0, J1 = flat[(w * 2 + s) * 3:(w * 2 + s) * 3 + 3]
            if I != 255:
                tiles += [(I, J) for J in range(J0, J1 + 1)]
                n += J1 - J0 + 1
        counts.append(n)
    assert sorted(tiles) == sorted(LOWER)
    assert max(counts) <= 7                                  # seven tiles or fewer per X wave


@pytest.mark.parametrize("S,TS,per", [(64, 4, 2), (32, 2, 1)])
def test_two_pass_coupling_deal(S, TS, per):
    """The dealing written in coupling8<S>: pass A tile (pr, mr, nc) costs TS - nc MFMA steps,
    pass B tile costs mr + 1; both passes cover every tile of every pair once."""
    npair = 128 // (2 * S)
    full = {(p, m, n) for p in range(npair) for m in range(TS) for n in range(TS)}
    a, b, cost_a, cost_b = [], [], [0] * 8, [0] * 8
    for w in range(8):
        for t in range(per):
            pr = 0 if S == 64 else w >> 2
            mr = w >> 1 if S == 64 else (w >> 1) & 1
            nc = (w & 1 if t == 0 else 3 - (w & 1)) if S == 64 else w & 1
            a.append((pr, mr, nc))
            cost_a[w] += TS - nc
            nc2 = w >> 1 if S == 64 else (w >> 1) & 1
            mr2 = (w & 1 if t == 0 else 3 - (w & 1)) if S == 64 else w & 1
            b.append((pr, mr2, nc2))
            cost_b[w] += mr2 + 1
    assert sorted(a) == sorted(full) and sorted(b) == sorted(full)
    if S == 64:
        assert cost_a == [5] * 8 and cost_b == [5] * 8
    # the dealing in the source is the one checked here
    text = open(SRC).read()
    assert "const int nc = S == 64 ? (t == 0 ? (wave & 1) : 3 - (wave & 1)) : wave & 1;" in text
    assert "const int mr = S == 64 ? (t == 0 ? (wave & 1) : 3 - (wave & 1)) : wave & 1;" in text
