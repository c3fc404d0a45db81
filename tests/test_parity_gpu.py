"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by element.

Tolerances: max-abs 1e-4 for fp32 inputs, 2e-2 for bf16 inputs (fp32
accumulate).  Workloads are the seeded synthetic ones; large decode batches are
checked on a seeded sample of requests at several steps.
"""

import numpy as np
import pytest
import torch

from tests.harness import TOL, max_abs, oracle_decode, oracle_prefill, say
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _engine(wl, shared=True, extra_blocks=0, on_the_fly=False):
    from position_agnostic_paged_amd.engine import Engine
    from position_agnostic_paged_amd.scenarios import blocks_needed, make_pos

    pos = make_pos(wl, "cuda", on_the_fly=on_the_fly)
    g = wl.geom
    nb = blocks_needed(wl, shared) + extra_blocks
    return Engine(g.num_q_heads, g.num_kv_heads, g.head_dim, g.dtype, pos, nb, "cuda")


def _check_prefill(key, shared=True, prerotated=False, on_the_fly=False):
    from position_agnostic_paged_amd.scenarios import PrefillScenario

    wl = make_workload(key)
    say(f"[prefill parity] {wl.name} shared={shared} prerotated={prerotated} on_the_fly={on_the_fly}")
    eng = _engine(wl, shared, on_the_fly=on_the_fly)
    sc = PrefillScenario(wl, eng, shared=shared, prerotated=prerotated)
    out = sc.run().float().cpu().numpy()
    torch.cuda.synchronize()
    want = oracle_prefill(wl, 0, range(len(sc.reqs)))
    err = 0.0
    for i, w in enumerate(want):
        got = out[sc.q_start_h[i]: sc.q_start_h[i + 1]]
        err = max(err, max_abs(got, w))
    say(f"  max-abs err {err:.3e} (tol {TOL[wl.geom.dtype]})")
    assert np.isfinite(out).all()
    assert err <= TOL[wl.geom.dtype]


def _check_decode(key, steps, reqs=None, shared=True, prerotated=False, num_steps=None):
    from position_agnostic_paged_amd.scenarios import DecodeScenario

    wl = make_workload(key)
    if num_steps is not None:
        wl.num_decode_steps = num_steps
    say(f"[decode parity] {wl.name} steps={list(steps)} shared={shared} prerotated={prerotated}")
    eng = _engine(wl, shared)
    sc = DecodeScenario(wl, eng, shared=shared, prerotated=prerotated)
    R = sc.R
    reqs = list(range(R)) if reqs is None else list(reqs)
    draws = {}
    got = {}
    last = max(steps)
    for s in range(last + 1):
        draws[s] = wl.decode_step(s)
        out = sc.step(s)
        if s in steps:
            got[s] = out.float().cpu().numpy()
    torch.cuda.synchronize()
    err = 0.0
    for r in reqs:
        want = oracle_decode(wl, r, steps, draws)
        for s, w in zip(steps, want):
            err = max(err, max_abs(got[s][r], w))
    say(f"  max-abs err {err:.3e} over {len(reqs)} requests (tol {TOL[wl.geom.dtype]})")
    assert err <= TOL[wl.geom.dtype]


def test_tiny_fp32_prefill():
    _check_prefill("tiny_fp32")


def test_tiny_fp32_decode():
    _check_decode("tiny_fp32", steps=list(range(8)))


def test_tiny_fp32_on_the_fly_sincos():
    _check_prefill("tiny_fp32", on_the_fly=True)


def test_llama8b_prefill():
    _check_prefill("llama8b_prefill")


def test_llama8b_prefill_interleaved():
    _check_prefill("llama8b_prefill_interleaved")


def test_llama8b_prefill_no_sharing_and_prerotated_control():
    _check_prefill("llama8b_prefill", shared=False)
    _check_prefill("llama8b_prefill", shared=False, prerotated=True)


def test_llama8b_decode_sampled():
    rng = np.random.default_rng(3)
    reqs = sorted(rng.choice(64, size=8, replace=False).tolist())
    _check_decode("llama8b_decode", steps=[0, 31, 63], reqs=reqs)


def test_falcon_alibi_decode_sampled():
    rng = np.random.default_rng(5)
    reqs = sorted(rng.choice(128, size=12, replace=False).tolist())
    _check_decode("falcon7b_alibi", steps=[0, 7], reqs=reqs, num_steps=8)
