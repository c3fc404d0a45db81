"""Shared test plumbing: run a workload through the HIP path and the oracle on the same inputs.

Parity gates.  Every GPU parity check applies two bounds to each compared
(request, step):

  * the absolute bound of the method's precision contract: max-abs 1e-4 for
    fp32 inputs, 2e-2 for bf16 inputs with fp32 accumulation;
  * a discriminating bound relative to that output's own scale:
    max-abs <= REL * max|oracle| (bf16 5e-2, fp32 1e-3).  Long contexts
    average over tens of thousands of keys, so their outputs are small
    (|o| ~ 1e-2 at 32K tokens) and the absolute bound alone would pass an
    all-zero output.  The bf16 error budget: outputs are rounded once to
    bf16 (relative 2^-9), the attention weights that multiply V are bf16
    (relative 2^-9 each, averaging out over many keys), and the re-rotated
    query or key is rounded once to bf16 (a score shift of about 2^-9 of
    the score's scale); together well under 1 % of max|o|, so 5 % leaves
    margin while a kernel that misplaces documents is off by tens of percent.

Negative control.  A parity test must be able to fail on the method's
characteristic mistake, ignoring the document offset Delta (keys used at
their document-local positions).  ``nodelta_*`` plant exactly that mistake in
the oracle, on the CPU, and ``Gate.check`` requires its relative distance
from the true oracle on the test's own inputs to exceed NEG_MARGIN x REL;
otherwise the test fails as unable to discriminate.

Large oracle workloads run in a pool of spawned CPU worker processes
(``oracle_map``); each worker rebuilds the same seeded inputs.
"""

from __future__ import annotations

import dataclasses
import os
import sys
from concurrent.futures import ProcessPoolExecutor
from typing import Dict, List, Optional, Sequence

import numpy as np

from oracle import attention as OA
from oracle import rope as OR

TOL = {"fp32": 1e-4, "bf16": 2e-2}  # max-abs vs the fp64 oracle (fp32 inputs / bf16 inputs, fp32 accumulate)
REL = {"fp32": 1e-3, "bf16": 5e-2}  # max-abs / max|oracle| of the same output
NEG_MARGIN = 2.0  # a no-Delta kernel must miss the relative bound by at least this factor


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


def oracle_decode(wl, r: int, steps: Sequence[int], step_draws=None) -> List[np.ndarray]:
    """Oracle outputs of decode request r at the given steps; step_draws[s] = (q, k, v) for all requests
    (drawn from the workload when None)."""
    var = oracle_var(wl)
    req = wl.decode_reqs[r]
    docs = [wl.doc(d) for d in req.doc_ids]
    last = max(steps)
    if step_draws is None:
        step_draws = {s: wl.decode_step(s) for s in range(last + 1)}
    seq = [(step_draws[s][0][r], step_draws[s][1][r], step_draws[s][2][r]) for s in range(last + 1)]
    return OA.eager_decode(docs, req.k, req.v, seq, var, which=list(steps))


# ---------------------------------------------------------------- negative control (planted mistake)

def _local_positions(doc_lens: Sequence[int], tail: int) -> np.ndarray:
    """Positions a no-Delta kernel would use: each document from 0, private tokens at their global ones."""
    parts = [np.arange(L, dtype=np.int64) for L in doc_lens]
    parts.append(np.arange(sum(doc_lens), sum(doc_lens) + tail, dtype=np.int64))
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def _nodelta_attend(var, q_raw, q_pos, k_raw, v, k_glob, k_local):
    """Attention whose keys carry their document-local positions (RoPE: rotated there; ALiBi: biased
    from there) while visibility follows the global order: the oracle with Delta dropped."""
    if var["kind"] == "alibi":
        # bias -slope (m - n) with n local: shift each query's distances by (n_glob - n_local)
        q = np.asarray(q_raw, np.float64)
        M, Hq, _ = q.shape
        G = Hq // k_raw.shape[1]
        kh = np.repeat(np.asarray(k_raw, np.float64), G, axis=1)
        vh = np.repeat(np.asarray(v, np.float64), G, axis=1)
        s = np.einsum("mhd,nhd->hmn", q, kh) * var["scale"]
        dist_vis = q_pos[:, None].astype(np.float64) - k_glob[None, :].astype(np.float64)
        dist_bias = q_pos[:, None].astype(np.float64) - k_local[None, :].astype(np.float64)
        s = s - var["slopes"][:, None, None] * dist_bias[None]
        s = np.where((dist_vis >= 0)[None], s, -np.inf)
        s = s - np.max(s, axis=2, keepdims=True)
        p = np.exp(s)
        p /= np.sum(p, axis=2, keepdims=True)
        return np.einsum("hmn,nhd->mhd", p, vh)
    kp = OR.rotate(k_raw, k_local, var["inv_freq"], var["kind"])
    qp = OR.rotate(q_raw, q_pos, var["inv_freq"], var["kind"])
    return OA.attend(qp, q_pos, kp, v, k_glob, var)


def nodelta_prefill(wl, step: int, i: int) -> np.ndarray:
    var = oracle_var(wl)
    r = wl.prefill_steps[step][i]
    docs = [wl.doc(d) for d in r.doc_ids]
    k, v, pos = OA.logical_sequence(docs, r.k, r.v)
    Lq = r.q.shape[0]
    local = _local_positions([wl.doc_lens[d] for d in r.doc_ids], Lq)
    return _nodelta_attend(var, r.q, pos[-Lq:], k, v, pos, local)


def nodelta_decode(wl, r: int, step: int) -> np.ndarray:
    var = oracle_var(wl)
    req = wl.decode_reqs[r]
    docs = [wl.doc(d) for d in req.doc_ids]
    draws = [wl.decode_step(s) for s in range(step + 1)]
    tail_k = np.concatenate([np.asarray(req.k, np.float32)] + [d[1][r][None] for d in draws])
    tail_v = np.concatenate([np.asarray(req.v, np.float32)] + [d[2][r][None] for d in draws])
    k, v, pos = OA.logical_sequence(docs, tail_k, tail_v)
    local = _local_positions([wl.doc_lens[d] for d in req.doc_ids], tail_k.shape[0])
    q = draws[step][0][r][None]
    return _nodelta_attend(var, q, pos[-1:], k, v, pos, local)[0]


# ---------------------------------------------------------------- gates

class Gate:
    """Accumulates the absolute and relative errors of a parity test and its negative control."""

    def __init__(self, name: str, dtype: str):
        self.name, self.dtype = name, dtype
        self.abs = 0.0
        self.rel = 0.0
        self.n = 0
        self.neg: Optional[float] = None

    def add(self, got, want) -> None:
        got = np.asarray(got, np.float64)
        want = np.asarray(want, np.float64)
        assert got.shape == want.shape, (got.shape, want.shape)
        assert np.isfinite(got).all(), f"{self.name}: non-finite output"
        err = float(np.max(np.abs(got - want))) if want.size else 0.0
        scale = float(np.max(np.abs(want))) if want.size else 0.0
        self.abs = max(self.abs, err)
        if scale > 0:
            self.rel = max(self.rel, err / scale)
        self.n += 1

    def add_negative(self, planted, want) -> None:
        """Relative distance of the planted no-Delta oracle from the true one (max over the items given)."""
        planted = np.asarray(planted, np.float64)
        want = np.asarray(want, np.float64)
        d = float(np.max(np.abs(planted - want))) / max(float(np.max(np.abs(want))), 1e-300)
        self.neg = d if self.neg is None else max(self.neg, d)

    def check(self, negative: bool = True) -> None:
        tol, rel = TOL[self.dtype], REL[self.dtype]
        neg = "n/a" if self.neg is None else f"{self.neg:.3e} (needs > {NEG_MARGIN * rel:.1e})"
        say(f"  [{self.name}] {self.n} outputs: max-abs {self.abs:.3e} (tol {tol}), "
            f"max-abs/max|oracle| {self.rel:.3e} (tol {rel}), no-Delta control {neg}")
        assert self.n > 0, f"{self.name}: nothing compared"
        assert self.abs <= tol, f"{self.name}: max-abs {self.abs} > {tol}"
        assert self.rel <= rel, f"{self.name}: relative error {self.rel} > {rel}"
        if negative:
            assert self.neg is not None, f"{self.name}: no negative control computed"
            assert self.neg > NEG_MARGIN * rel, (
                f"{self.name}: the no-Delta oracle is within {self.neg:.3e} of the oracle; this test cannot "
                f"tell a kernel that ignores the document offset from a correct one")


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


# ---------------------------------------------------------------- oracle worker pool

_WL = None


def _init_worker(wl) -> None:
    global _WL
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    _WL = wl


def _task(t):
    _WL._doc_cache.clear()  # bounded memory per worker: documents are redrawn per task
    kind = t[0]
    if kind == "decode":
        _, r, steps = t
        return oracle_decode(_WL, r, steps)
    if kind == "prefill":
        _, step, i = t
        return oracle_prefill(_WL, step, [i])[0]
    if kind == "nodelta_decode":
        _, r, step = t
        return nodelta_decode(_WL, r, step)
    if kind == "nodelta_prefill":
        _, step, i = t
        return nodelta_prefill(_WL, step, i)
    raise ValueError(kind)


def pool_size() -> int:
    n = len(os.sched_getaffinity(0))
    cap = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    return max(1, min(n, cap, 16))


def oracle_map(wl, tasks: Sequence[tuple], workers: Optional[int] = None) -> list:
    """Run oracle tasks ("decode", r, steps) / ("prefill", step, i) / ("nodelta_decode", r, step) /
    ("nodelta_prefill", step, i) over a pool of spawned CPU processes; results in task order."""
    wl = dataclasses.replace(wl, _doc_cache={})
    n = min(workers or pool_size(), max(1, len(tasks)))
    if n == 1:
        _init_worker(wl)
        return [_task(t) for t in tasks]
    import multiprocessing as mp

    with ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"), initializer=_init_worker,
                             initargs=(wl,)) as ex:
        return list(ex.map(_task, tasks))


def decode_tasks(requests: Sequence[int], steps: Sequence[int], chunk: int = 16) -> List[tuple]:
    """Oracle tasks for the given requests at the given steps, long step lists split into chunks."""
    steps = sorted(steps)
    out = []
    for r in requests:
        for i in range(0, len(steps), chunk):
            out.append(("decode", int(r), steps[i: i + chunk]))
    return out


def gather_decode(tasks: Sequence[tuple], results: Sequence[list]) -> Dict[tuple, np.ndarray]:
    """{(request, step): oracle output} from decode_tasks results."""
    out = {}
    for t, res in zip(tasks, results):
        for s, o in zip(t[2], res):
            out[(t[1], s)] = o
    return out
