"""Position-agnostic vs position-aware cache hit ratios (LazyAttention notes, papernotes.org, "Background and
motivation": the Zipf closed form and its 2.86x; "Main experiments": the VRAM hit-ratio table).

* oracle.lru (a plain list-based LRU) is pinned by hand-worked sequences, by Mattson's stack-distance
  characterisation of LRU and by the no-limit count (misses = distinct keys);
* the library's caches (paging.DocCache / paging.PositionAwareCache, driven by hitsim.replay) produce
  exactly the oracle's hit/miss sequence on random traces and budgets;
* the static top-C setting reproduces the closed form (and through it the pages' 2.86x);
* the LRU table has the shape of the pages' table: the position-agnostic cache hits at least as often at
  every budget and skew, by the most at the tightest budget, and still more often with no limit.
"""

import math

import numpy as np
import pytest

from oracle import lru as OL
from oracle import zipf as OZ
from position_agnostic_paged_amd import hitsim
from workloads import zipf_accesses, zipf_trace


# ------------------------------------------------------------------------------------ oracle pins

def test_oracle_lru_hand_worked():
    # budget 3 unit entries, one access per request: A B C A D B
    seq = OL.replay([[("A", 1)], [("B", 1)], [("C", 1)], [("A", 1)], [("D", 1)], [("B", 1)]], 3)
    # A, B, C miss; A hits (order B C A); D evicts B (order C A D); B misses again
    assert seq == [False, False, False, True, False, False]
    # pinning: budget 2; request 1 = A B, request 2 = C A: C evicts A (unpinned LRU), then A must evict B
    # (C is pinned by request 2)
    assert OL.replay([[("A", 1), ("B", 1)], [("C", 1), ("A", 1)]], 2) == [False] * 4
    # sizes: budget 5: A(3) B(2) hit A, then C(3) evicts B (LRU after A's hit), B misses
    assert OL.replay([[("A", 3)], [("B", 2)], [("A", 3)], [("C", 3)], [("B", 2)]], 5) == \
        [False, False, True, False, False]
    with pytest.raises(RuntimeError):
        OL.replay([[("A", 2), ("B", 2)]], 3)


def _stack_distance_hits(keys, capacity):
    """Mattson et al. (1970): with unit entries, an access hits an LRU cache of a given capacity iff fewer
    than `capacity` distinct keys were accessed since the previous access to the same key."""
    out, last = [], {}
    for i, k in enumerate(keys):
        if k in last:
            out.append(len(set(keys[last[k] + 1: i])) < capacity)
        else:
            out.append(False)
        last[k] = i
    return out


@pytest.mark.parametrize("capacity", [1, 2, 5, 13])
def test_oracle_lru_matches_stack_distance(capacity):
    rng = np.random.default_rng(capacity)
    keys = [int(x) for x in rng.integers(0, 20, size=400)]
    assert OL.replay([[(k, 1)] for k in keys], capacity) == _stack_distance_hits(keys, capacity)


def test_oracle_lru_unlimited_misses_are_distinct_keys():
    trace = zipf_trace(3, 50, 5, 60, 1.2)
    seq = OL.replay([[(d, 2) for d in r] for r in trace], 10 ** 9)
    assert seq.count(False) == len({d for r in trace for d in r})


# ----------------------------------------------------------------------- library vs oracle

def _oracle_sequence(trace, doc_tokens, budget_blocks, aware):
    size = -(-doc_tokens // 16)
    reqs = [[(((d, i * doc_tokens) if aware else d), size) for i, d in enumerate(r)] for r in trace]
    return OL.replay(reqs, budget_blocks)


@pytest.mark.parametrize("aware", [False, True], ids=["agnostic", "aware"])
@pytest.mark.parametrize("alpha,budget", [(0.8, 40), (1.2, 25), (2.1, 60), (1.5, 500)])
def test_library_cache_replays_exactly_like_the_oracle(aware, alpha, budget):
    trace = zipf_trace(int(10 * alpha) + budget, 60, 4, 150, alpha)
    doc_tokens = 70  # 5 blocks each
    got = hitsim.hit_sequence(trace, doc_tokens, budget, aware)
    want = _oracle_sequence(trace, doc_tokens, budget, aware)
    assert got == want
    res = hitsim.replay(trace, doc_tokens, budget, aware)
    assert res.hits == sum(want) and res.accesses == len(want)
    assert res.tokens_written == doc_tokens * want.count(False)


def test_replay_rejects_a_budget_below_one_request():
    with pytest.raises(ValueError):
        hitsim.replay([[0, 1, 2]], 16, 2, aware=False)


# ------------------------------------------------------------------------------ closed form

def test_static_top_c_reproduces_the_closed_form():
    """Fixed contents, independent Zipf accesses: the measured gain equals sum_{i<=C} i^-a / sum_{i<=C/D}
    i^-a within sampling error; at the alpha where that form gives the pages' 2.86x, so does the sample."""
    C, D, N = 100, 20, 10000
    alpha = 0.8526  # where the closed form equals 2.86 (tests/test_oracle_pack_zipf.py)
    docs, slots = zipf_accesses(7, N, 2_000_000, alpha, D)
    got = hitsim.static_hit_ratios(docs, slots, C, D)
    # the same hits counted by the oracle's static cache
    assert got["agnostic"] * len(docs) == OL.static_hits(docs.tolist(), lambda d: d < C)
    h = lambda n: sum(i ** -alpha for i in range(1, n + 1))  # noqa: E731
    assert got["agnostic"] == pytest.approx(h(C) / h(N), rel=5e-3)
    assert got["aware"] == pytest.approx(h(C // D) / h(N), rel=1e-2)
    assert got["gain"] == pytest.approx(OZ.hit_ratio_gain(C, D, alpha), rel=1.5e-2)
    assert abs(got["gain"] - 2.86) < 0.05


def test_static_slots_are_checked():
    with pytest.raises(ValueError):
        hitsim.static_hit_ratios(np.array([1]), np.array([20]), 100, 20)


# ------------------------------------------------------------------------- the table's shape

def test_lru_table_has_the_pages_shape():
    rows = hitsim.hit_ratio_table(alphas=(1.1, 2.1), budgets_gb=(1, 10, None), num_docs=4000, num_reqs=600)
    by_alpha = {}
    for r in rows:
        assert r["agnostic_hit"] >= r["aware_hit"]
        assert r["aware_tokens_written"] >= r["agnostic_tokens_written"]
        by_alpha.setdefault(r["alpha"], []).append(r)
    for a, rs in by_alpha.items():
        gains = [r["gain"] for r in rs]  # 1 GB, 10 GB, no limit
        assert gains[0] > gains[1] >= gains[2] > 1.0, (a, gains)
        # with no limit the agnostic misses are exactly the distinct documents
        trace = zipf_trace(12, 4000, 10, 600, a)
        distinct = len({d for req in trace for d in req})
        assert rs[-1]["agnostic_hit"] == pytest.approx(1 - distinct / rs[-1]["accesses"])
    assert math.isfinite(rows[0]["gain"])
