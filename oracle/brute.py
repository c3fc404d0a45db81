"""Pure-Python scalar-loop attention for tiny cases (oracle; test infrastructure only).

Written as plainly as possible so a reader can check it by eye against the
definition of softmax attention and of a RoPE rotation as a complex
multiplication (RoFormer: channel pair (a, b) is the complex number a + ib and
position p multiplies it by e^{i p theta}).  Used to pin the vectorised oracle
and to check the LazyAttention notes' Example 3.1 ("Method: overall
framework"), where a cached document rotated from local position 0 meets a
query rotated back by the length of the document before it.
"""

from __future__ import annotations

import cmath
import math
from typing import List, Sequence


def rotate_pairs(x: Sequence[float], p: float, theta: Sequence[float], kind: str) -> List[float]:
    """Rotate one vector by position p, pair by pair, using complex arithmetic."""
    dh = len(x)
    half = dh // 2
    out = [0.0] * dh
    for k in range(half):
        if kind == "rope_half":
            i1, i2 = k, k + half
        else:
            i1, i2 = 2 * k, 2 * k + 1
        z = complex(x[i1], x[i2]) * cmath.exp(1j * p * theta[k])
        out[i1], out[i2] = z.real, z.imag
    return out


def dot(a: Sequence[float], b: Sequence[float]) -> float:
    s = 0.0
    for x, y in zip(a, b):
        s += x * y
    return s


def softmax_weighted_sum(scores: Sequence[float], values: Sequence[Sequence[float]]) -> List[float]:
    mx = max(scores)
    w = [math.exp(s - mx) for s in scores]
    tot = sum(w)
    dh = len(values[0])
    out = [0.0] * dh
    for wi, vi in zip(w, values):
        for d in range(dh):
            out[d] += wi * vi[d] / tot
    return out


def attention_one_query(q: Sequence[float], keys: Sequence[Sequence[float]],
                        values: Sequence[Sequence[float]], scale: float,
                        biases: Sequence[float] = None) -> List[float]:
    """softmax_n(scale * q.k_n + bias_n) weighted sum of v_n, with explicit loops."""
    scores = []
    for n, k in enumerate(keys):
        s = scale * dot(q, k)
        if biases is not None:
            s += biases[n]
        scores.append(s)
    return softmax_weighted_sum(scores, values)
