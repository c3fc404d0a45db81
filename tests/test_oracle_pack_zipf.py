"""Pins for oracle.pack (hand-worked words) and oracle.zipf (the pages' 2.86x and closed forms)."""

import os

import numpy as np
import pytest

from oracle import pack, zipf

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLD, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_pack_golden_words():
    for b, o, m, w in _rows("pack_words.txt"):
        word = pack.pack(int(b), int(o), int(m))
        assert word == int(w, 16)
        assert pack.unpack(word) == (int(b), int(o), int(m))


def test_pack_rejects_out_of_range():
    for args in [(1 << 24, 0, 1), (-1, 0, 1), (0, 1 << 24, 1), (0, 0, 0), (0, 0, 1 << 16)]:
        with pytest.raises(ValueError):
            pack.pack(*args)


def test_pack_roundtrip_random():
    rng = np.random.default_rng(7)
    for _ in range(2000):
        b, o = (int(x) for x in rng.integers(0, 1 << 24, size=2))
        m = int(rng.integers(1, 1 << 16))
        assert pack.unpack(pack.pack(b, o, m)) == (b, o, m)


def test_request_tiles_golden():
    rows = _rows("request_tiles.txt")
    segs = []
    for spec in rows[0][1:]:
        blocks, L, p0, ctx = spec.split(";")
        segs.append({"blocks": [int(x) for x in blocks.split(",")], "len": int(L), "pos0": int(p0),
                     "ctx": ctx == "1"})
    for row in rows[1:]:
        kind, n_ctx, words = row[0], int(row[1]), [int(w, 16) for w in row[2:]]
        got, got_ctx = pack.request_tiles(segs, kind)
        assert got == words and got_ctx == n_ctx


def test_zipf_pages_value():
    """The notes print 2.86x at D = 20, C = 100 under 'moderate' Zipf: some alpha in (0.5, 1.5) gives it."""
    (C, D, gain), = [(int(a), int(b), float(c)) for a, b, c in _rows("zipf_gain.txt")]
    lo, hi = 0.5, 1.5
    assert zipf.hit_ratio_gain(C, D, lo) > gain > zipf.hit_ratio_gain(C, D, hi)
    for _ in range(60):  # bisection on a decreasing function
        mid = (lo + hi) / 2
        if zipf.hit_ratio_gain(C, D, mid) > gain:
            lo = mid
        else:
            hi = mid
    assert abs(zipf.hit_ratio_gain(C, D, lo) - gain) < 1e-9
    assert 0.84 < lo < 0.87  # "moderate" skew


def test_zipf_closed_forms():
    # alpha = 0: uniform popularity, the gain is C / floor(C/D)
    assert zipf.hit_ratio_gain(100, 20, 0.0) == pytest.approx(20.0, rel=1e-15)
    # alpha = 1: harmonic numbers H_100 / H_5
    h100 = sum(1.0 / i for i in range(1, 101))
    assert zipf.hit_ratio_gain(100, 20, 1.0) == pytest.approx(h100 / (1 + 1 / 2 + 1 / 3 + 1 / 4 + 1 / 5), rel=1e-14)
    # very skewed popularity: only the top document matters, gain -> 1
    assert zipf.hit_ratio_gain(100, 20, 40.0) == pytest.approx(1.0, abs=1e-12)
    # monotone decreasing in alpha
    vals = [zipf.hit_ratio_gain(100, 20, a) for a in np.linspace(0, 3, 31)]
    assert all(x > y for x, y in zip(vals, vals[1:]))
