"""End-to-end parity of the mixed serving step that bench.py times: LRU document
cache with misses, one pinned upload per step, one kv-write for every new token
of the step (queries rotated in place), prefill and decode calls.  Two steps
run; sampled outputs of the second step are compared with the fp64 oracle."""

import numpy as np
import pytest
import torch

from tests.harness import TOL, max_abs, oracle_decode, oracle_prefill, say
from workloads import make_workload

pytestmark = pytest.mark.gpu


def test_mixed_step_end_to_end():
    import bench

    wl = make_workload("llama70b_mixed", num_steps=2)
    runner = bench.MixedRunner(wl, "cuda")
    say(f"[mixed runner] {wl.name}: {runner.R} decodes, {runner.warm} warm documents")
    for s in range(2):
        runner.step(s, bench.Timer(), bench.Timer())
    torch.cuda.synchronize()
    assert runner.deferred_prefills == 0
    pre = runner.pre_out.float().cpu().numpy()
    dec = runner.dec.out.float().cpu().numpy()
    # prefill of step 1, request 2 (rows follow the admitted requests' order)
    lens = [r.q.shape[0] for r in wl.prefill_steps[1]]
    r0 = sum(lens[:2])
    want = oracle_prefill(wl, 1, [2])[0]
    e_pre = max_abs(pre[r0: r0 + lens[2]], want)
    draws = {s: wl.decode_step(s) for s in range(2)}
    e_dec = 0.0
    for r in (0, 31):
        e_dec = max(e_dec, max_abs(dec[r], oracle_decode(wl, r, [1], draws)[0]))
    say(f"  prefill max-abs {e_pre:.3e}, decode max-abs {e_dec:.3e} (tol {TOL[wl.geom.dtype]})")
    assert e_pre <= TOL[wl.geom.dtype] and e_dec <= TOL[wl.geom.dtype]
