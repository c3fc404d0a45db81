"""Hit-ratio gain of a position-agnostic cache over a position-aware one (oracle; test infrastructure only).

The LazyAttention notes (papernotes.org, "Background and motivation" and
"Highlights") model document popularity as Zipf(alpha) and a KV budget of C
entries: a position-agnostic cache holds the C most popular documents, a
position-aware cache that must keep a copy per each of D possible positions
holds floor(C / D) documents, so the ratio of hit rates is

    sum_{i=1..C} i^-alpha  /  sum_{i=1..floor(C/D)} i^-alpha.

The pages quote 2.86x at D = 20, C = 100 under "moderate" Zipf without naming
alpha; the tests pin the alpha at which the formula gives 2.86.
"""

from __future__ import annotations


def harmonic(n: int, alpha: float) -> float:
    return sum(i ** (-alpha) for i in range(1, n + 1))


def hit_ratio_gain(C: int, D: int, alpha: float) -> float:
    return harmonic(C, alpha) / harmonic(C // D, alpha)
