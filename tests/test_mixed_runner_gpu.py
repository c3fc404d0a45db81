"""End-to-end parity of the mixed serving step that bench.py times: LRU document
cache with misses and evictions, one pinned upload per step, one kv-write for
every new token of the step (queries rotated in place), prefill and decode
calls.  Sixteen steps run under the 1 GiB budget.  The prefills draw their
documents with a flatter Zipf (alpha 1.1 instead of the benchmark's 2.1, same
pool), so documents keep missing, evicting least-recently-used ones and being
rewritten at local positions while the decodes' pinned documents stay; every
admitted prefill and every decode request is compared with the fp64 oracle at
the first and the last step."""

import dataclasses

import numpy as np
import pytest
import torch

from tests.harness import Gate, decode_tasks, gather_decode, oracle_map, say
from workloads import make_workload

pytestmark = pytest.mark.gpu


def test_mixed_steps_with_lru_churn():
    import bench

    steps = 16
    check = (0, steps - 1)
    wl = make_workload("llama70b_mixed", num_steps=steps, prefill_alpha=1.1)
    runner = bench.MixedRunner(wl, "cuda")
    say(f"[mixed runner] {wl.name}: {runner.R} decodes, {runner.warm} warm documents, {steps} steps")
    pre_got, dec_got, admitted = {}, {}, {}
    ev0 = runner.eng.docs.evictions
    for s in range(steps):
        runner.step(s, bench.Timer(), bench.Timer())
        if s in check:
            torch.cuda.synchronize()
            pre_got[s] = runner.pre_out.float().cpu().numpy()
            dec_got[s] = runner.dec.out.float().cpu().numpy()
            admitted[s] = list(runner.admitted_idx)
    torch.cuda.synchronize()
    evictions = runner.eng.docs.evictions - ev0
    say(f"  misses {runner.misses}, evictions {evictions}, deferred prefills {runner.deferred_prefills}")
    assert runner.misses > 0 and evictions > 0, "the run must exercise LRU eviction"
    assert all(admitted[s] for s in check)

    # oracle: the admitted prefills of the checked steps (a trimmed copy holds only those steps) and
    # every decode request at those steps
    small = dataclasses.replace(wl, prefill_steps=[wl.prefill_steps[s] for s in check], _doc_cache={})
    p_tasks = [("prefill", ci, j) for ci, s in enumerate(check) for j in admitted[s]]
    d_tasks = decode_tasks(range(runner.R), list(check))
    neg = [("nodelta_prefill", 0, admitted[check[0]][0]), ("nodelta_decode", 0, check[0]),
           ("nodelta_decode", 1, check[0])]
    res = oracle_map(small, p_tasks + d_tasks + neg)
    p_want = res[: len(p_tasks)]
    d_want = gather_decode(d_tasks, res[len(p_tasks): len(p_tasks) + len(d_tasks)])
    planted = res[len(p_tasks) + len(d_tasks):]

    gp = Gate(f"{wl.name} prefill steps {check}", wl.geom.dtype)
    k = 0
    for ci, s in enumerate(check):
        lens = [wl.prefill_steps[s][j].q.shape[0] for j in admitted[s]]
        r0 = 0
        for j, L in zip(admitted[s], lens):
            gp.add(pre_got[s][r0: r0 + L], p_want[k])
            r0 += L
            k += 1
    gp.add_negative(planted[0], p_want[0])
    gd = Gate(f"{wl.name} decode steps {check}", wl.geom.dtype)
    for (r, s), w in d_want.items():
        gd.add(dec_got[s][r], w)
    gd.add_negative(planted[1], d_want[(0, check[0])])
    gd.add_negative(planted[2], d_want[(1, check[0])])
    gp.check()
    gd.check()
