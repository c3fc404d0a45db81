"""Shared test plumbing: run a workload through the HIP path and the oracle on the same inputs."""

from __future__ import annotations

import sys
from typing import List, Sequence

import numpy as np

from oracle import attention as OA
from oracle import rope as OR

TOL = {"fp32": 1e-4, "bf16": 2e-2}  # max-abs vs the fp64 oracle (fp32 inputs / bf16 inputs, fp32 accumulate)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_var(wl) -> dict:
    return OR.variant(wl.pos, wl.geom.head_dim, wl.geom.num_q_heads)


def oracle_prefill(wl, step: int, reqs: Sequence[int]) -> List[np.ndarray]:
    var = oracle_var(wl)
    outs = []
    for i in reqs:
        r = wl.prefill_steps[step][i]
        docs = [wl.doc(d) for d in r.doc_ids]
        outs.append(OA.eager_prefill(docs, r.q, r.k, r.v, var))
    return outs


def oracle_decode(wl, r: int, steps: Sequence[int], step_draws) -> List[np.ndarray]:
    """Oracle outputs of decode request r at the given steps; step_draws[s] = (q, k, v) for all requests."""
    var = oracle_var(wl)
    req = wl.decode_reqs[r]
    docs = [wl.doc(d) for d in req.doc_ids]
    last = max(steps)
    seq = [(step_draws[s][0][r], step_draws[s][1][r], step_draws[s][2][r]) for s in range(last + 1)]
    return OA.eager_decode(docs, req.k, req.v, seq, var, which=list(steps))


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))
