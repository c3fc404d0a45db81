"""GPU edge cases of the attention path against the oracle.

* Requests with no cached document, beside ordinary ones: a prefill whose
  context is its question alone, a decode request whose context is its
  question and generated tokens, and one with no question either, whose
  first token attends to itself only (per request and document-major).
  Such requests have no document offset, so they carry no no-Delta
  negative control; the ordinary requests in the same batch do.
* An empty batch through every attention entry point: success, and the
  output buffer left as it was.
"""

import numpy as np
import pytest
import torch

from tests.harness import Gate, nodelta_decode, nodelta_prefill, oracle_decode, oracle_prefill, say
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _without_documents():
    from workloads.gen import DecodeRequest, PrefillRequest

    wl = make_workload("ragged")
    pre = list(wl.prefill_steps[0])
    r0 = pre[0]
    pre[0] = PrefillRequest(doc_ids=[], q=r0.q, k=r0.k, v=r0.v)  # the question alone
    wl.prefill_steps = [pre]
    withq = next(r for r in wl.decode_reqs if r.k.shape[0] > 0 and r.doc_ids)
    wl.decode_reqs = [DecodeRequest(doc_ids=[], k=withq.k, v=withq.v),  # question + generated tokens
                      DecodeRequest(doc_ids=[], k=withq.k[:0], v=withq.v[:0]),  # generated tokens only
                      withq]
    return wl


def _engine(wl):
    from position_agnostic_paged_amd.engine import Engine
    from position_agnostic_paged_amd.scenarios import blocks_needed, make_pos

    g = wl.geom
    return Engine(g.num_q_heads, g.num_kv_heads, g.head_dim, g.dtype, make_pos(wl, "cuda"), blocks_needed(wl, True),
                  "cuda")


def test_requests_without_documents():
    from position_agnostic_paged_amd.scenarios import DecodeScenario, PrefillScenario

    wl = _without_documents()
    dt = wl.geom.dtype
    say(f"[no documents] prefill {[r.doc_ids for r in wl.prefill_steps[0]]}, "
        f"decode {[(r.doc_ids, r.k.shape[0]) for r in wl.decode_reqs]}")
    sc = PrefillScenario(wl, _engine(wl))
    out = sc.run().float().cpu().numpy()
    torch.cuda.synchronize()
    want = oracle_prefill(wl, 0, range(len(sc.reqs)))
    bare, docs = Gate("prefill, question alone", dt), Gate("prefill, with documents", dt)
    for i, w in enumerate(want):
        got = out[sc.q_start_h[i]: sc.q_start_h[i + 1]]
        if wl.prefill_steps[0][i].doc_ids:
            docs.add(got, w)
            docs.add_negative(nodelta_prefill(wl, 0, i), w)
        else:
            bare.add(got, w)
    bare.check(negative=False)
    docs.check()

    steps = [0, 1, 2]
    for doc_major in (False, True):
        sc = DecodeScenario(wl, _engine(wl), doc_major=doc_major)
        draws, got = {}, {}
        for s in range(max(steps) + 1):
            draws[s] = wl.decode_step(s)
            got[s] = sc.step(s).float().cpu().numpy()
        torch.cuda.synchronize()
        bare = Gate(f"decode doc_major={doc_major}, no documents", dt)
        docs = Gate(f"decode doc_major={doc_major}, with documents", dt)
        for r, req in enumerate(wl.decode_reqs):
            want = oracle_decode(wl, r, steps, draws)
            gate = docs if req.doc_ids else bare
            for s, w in zip(steps, want):
                gate.add(got[s][r], w)
            if req.doc_ids:
                gate.add_negative(nodelta_decode(wl, r, steps[0]), want[0])
        # the request with no context at all: its first token sees only itself, so its output is that
        # token's value row (rounded to the cache's dtype), which the oracle agrees with
        v0 = draws[0][2][1]  # [Hkv][dh] of request 1
        group = wl.geom.num_q_heads // wl.geom.num_kv_heads
        exact = np.repeat(np.asarray(v0, np.float64), group, axis=0)
        assert np.max(np.abs(got[0][1] - exact)) <= 2e-2 * max(1.0, float(np.max(np.abs(exact))))
        bare.check(negative=False)
        docs.check()


def test_empty_batch_every_entry_point():
    from position_agnostic_paged_amd import lazy_attn as L
    from position_agnostic_paged_amd.engine import StepUploads

    wl = make_workload("ragged")
    eng = _engine(wl)
    g = wl.geom
    sentinel = torch.full((4, g.num_q_heads, g.head_dim), 7.0, dtype=eng.tdtype, device="cuda")
    q0 = sentinel[:0]
    i32 = torch.zeros(1, dtype=torch.int32, device="cuda")
    tt = eng.tile_table([])
    assert tt.num_reqs == 0 and tt.total_tiles == 0
    eng.prefill(tt, q0, i32, i32, 0, out=sentinel[:0])
    eng.decode(tt, q0, i32, out=sentinel[:0])
    plan = eng.shared_plan([])
    assert plan.num_reqs == 0 and plan.num_work == 0
    eng.decode_shared(plan, q0, i32, out=sentinel[:0])
    # kv write of no tokens
    kv0 = torch.zeros((0, g.num_kv_heads, g.head_dim), dtype=eng.tdtype, device="cuda")
    eng.kv_write(kv0, kv0, None, i32[:0], i32[:0])
    # an empty step through the uploads
    up = StepUploads("cuda")
    up.begin()
    tt2 = eng.tile_table([], up, paired=True)
    up.commit()
    eng.prefill(tt2, q0, i32, i32, 0, out=sentinel[:0])
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0), "an empty batch wrote to memory"
    assert L.workspace_size(eng.geom, 0, 0, 0, 0, True) == 0
    say("[empty batch] prefill, decode, document-major decode and kv write of nothing: success, nothing written")
