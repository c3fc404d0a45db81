"""GPU parity of the position-aware cache the pages compare against (LazyAttention notes, papernotes.org,
"Background and motivation"): one copy per (document, global offset), written with RoPE at its global
positions through lazy_kv_write, read by the kernels without deferral (LAZY_FLAG_PREROTATED).  Its outputs
equal the oracle's, as the position-agnostic cache's do, but the same batch costs it more copies."""

import pytest
import torch

from tests.harness import Gate, decode_tasks, gather_decode, oracle_map, say
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _engine(wl, aware):
    from position_agnostic_paged_amd.engine import Engine
    from position_agnostic_paged_amd.scenarios import blocks_needed, make_pos

    g = wl.geom
    return Engine(g.num_q_heads, g.num_kv_heads, g.head_dim, g.dtype, make_pos(wl, "cuda"),
                  blocks_needed(wl, True, aware), "cuda", position_aware=aware)


def test_position_aware_prefill_matches_oracle_with_more_copies():
    from position_agnostic_paged_amd.scenarios import PrefillScenario

    wl = make_workload("llama8b_prefill")
    n = len(wl.prefill_steps[0])
    agn = PrefillScenario(wl, _engine(wl, False))
    eng = _engine(wl, True)
    awr = PrefillScenario(wl, eng, aware=True)
    out = awr.run().float().cpu().numpy()
    torch.cuda.synchronize()
    docs = {d for r in wl.prefill_steps[0] for d in r.doc_ids}
    multi = sum(1 for d in docs if eng.docs.copies(d) > 1)
    say(f"[position-aware prefill] {wl.name}: {awr.doc_writes} copies written vs {agn.doc_writes} "
        f"position-agnostic; {multi} documents held at several offsets")
    assert awr.doc_writes > agn.doc_writes and multi > 0
    res = oracle_map(wl, [("prefill", 0, i) for i in range(n)] + [("nodelta_prefill", 0, i) for i in range(n)])
    gate = Gate(f"{wl.name} position-aware", wl.geom.dtype)
    for i in range(n):
        gate.add(out[awr.q_start_h[i]: awr.q_start_h[i + 1]], res[i])
        gate.add_negative(res[n + i], res[i])
    gate.check()


def test_position_aware_decode_matches_oracle():
    from position_agnostic_paged_amd.scenarios import DecodeScenario

    wl = make_workload("small_dh64_interleaved")
    steps = [0, 3]
    eng = _engine(wl, True)
    sc = DecodeScenario(wl, eng, aware=True)
    got = {}
    for s in range(max(steps) + 1):
        o = sc.step(s)
        if s in steps:
            got[s] = o.float().cpu().numpy()
    torch.cuda.synchronize()
    R = len(wl.decode_reqs)
    tasks = decode_tasks(range(R), steps)
    neg = [("nodelta_decode", r, 0) for r in range(R)]
    res = oracle_map(wl, tasks + neg)
    want = gather_decode(tasks, res[: len(tasks)])
    gate = Gate(f"{wl.name} position-aware decode", wl.geom.dtype)
    for (r, s), w in want.items():
        gate.add(got[s][r], w)
    for t, p in zip(neg, res[len(tasks):]):
        gate.add_negative(p, want[(t[1], 0)])
    gate.check()
