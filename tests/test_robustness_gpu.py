"""GPU robustness of the attention path against the oracle.

* Unused slots of partial blocks poisoned with NaN: the kernels must mask
  them by selection (score -inf, V zeroed), never by multiplying by a zero
  weight, since 0 x NaN is NaN (and rotating NaN by Delta stays NaN).
* One document at two offsets of the same request: the same physical blocks
  are read twice and must be rotated by each occurrence's own Delta.
"""

import numpy as np
import pytest
import torch

from tests.harness import Gate, nodelta_decode, nodelta_prefill, oracle_decode, oracle_prefill, say
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _engine(wl, poison):
    from position_agnostic_paged_amd.engine import Engine
    from position_agnostic_paged_amd.scenarios import blocks_needed, make_pos

    g = wl.geom
    eng = Engine(g.num_q_heads, g.num_kv_heads, g.head_dim, g.dtype, make_pos(wl, "cuda"), blocks_needed(wl, True),
                 "cuda")
    if poison:
        eng.k_cache.fill_(float("nan"))
        eng.v_cache.fill_(float("nan"))
    return eng


def _prefill(wl, poison):
    from position_agnostic_paged_amd.scenarios import PrefillScenario

    sc = PrefillScenario(wl, _engine(wl, poison))
    out = sc.run().float().cpu().numpy()
    torch.cuda.synchronize()
    want = oracle_prefill(wl, 0, range(len(sc.reqs)))
    gate = Gate(f"{wl.name} prefill poison={poison}", wl.geom.dtype)
    for i, w in enumerate(want):
        gate.add(out[sc.q_start_h[i]: sc.q_start_h[i + 1]], w)
        gate.add_negative(nodelta_prefill(wl, 0, i), w)
    return out, gate


def _decode(wl, poison, steps, doc_major=False):
    from position_agnostic_paged_amd.scenarios import DecodeScenario

    sc = DecodeScenario(wl, _engine(wl, poison), doc_major=doc_major)
    draws, got = {}, {}
    for s in range(max(steps) + 1):
        draws[s] = wl.decode_step(s)
        out = sc.step(s)
        if s in steps:
            got[s] = out.float().cpu().numpy()
    torch.cuda.synchronize()
    gate = Gate(f"{wl.name} decode poison={poison} doc_major={doc_major}", wl.geom.dtype)
    for r in range(len(wl.decode_reqs)):
        want = oracle_decode(wl, r, steps, draws)
        for s, w in zip(steps, want):
            gate.add(got[s][r], w)
        gate.add_negative(nodelta_decode(wl, r, steps[0]), want[0])
    return got, gate


@pytest.mark.parametrize("key", ["ragged", "tiny_fp32", "small_dh64_interleaved", "falcon7b_alibi_prefill"])
def test_nan_poisoned_unused_slots_prefill(key):
    """Documents of 1..999 tokens (partial last blocks) in a pool filled with NaN before any write:
    the staged bf16 kernel (RoPE half-split, interleaved, ALiBi) and the fp32 per-wave kernel."""
    wl = make_workload(key)
    say(f"[nan-poisoned prefill] {wl.name}")
    out, gate = _prefill(wl, poison=True)
    assert np.isfinite(out).all()
    gate.check()


@pytest.mark.parametrize("doc_major", [False, True], ids=["per_request", "document_major"])
@pytest.mark.parametrize("key", ["ragged", "tiny_fp32"])
def test_nan_poisoned_unused_slots_decode(key, doc_major):
    wl = make_workload(key)
    say(f"[nan-poisoned decode] {wl.name} doc_major={doc_major}")
    got, gate = _decode(wl, poison=True, steps=[0, 2], doc_major=doc_major)
    assert all(np.isfinite(g).all() for g in got.values())
    gate.check()


def test_same_document_at_two_offsets_in_one_request():
    """doc a || doc b || doc a || question, and a decode request with its document repeated three times:
    one physical copy, read at every offset where it occurs."""
    from workloads.gen import DecodeRequest, PrefillRequest

    wl = make_workload("ragged")
    lens = wl.doc_lens
    a = next(d for d in sorted(lens) if lens[d] == 300)  # partial last block
    b = next(d for d in sorted(lens) if lens[d] == 17)
    c = next(d for d in sorted(lens) if lens[d] == 999)
    pre = [PrefillRequest(doc_ids=[a, b, a], q=r.q, k=r.k, v=r.v) for r in wl.prefill_steps[0][:2]]
    pre.append(PrefillRequest(doc_ids=[c, a, c], q=wl.prefill_steps[0][2].q, k=wl.prefill_steps[0][2].k,
                              v=wl.prefill_steps[0][2].v))
    wl.prefill_steps = [pre]
    decs = [DecodeRequest(doc_ids=[a, b, a, c, a], k=wl.decode_reqs[2].k, v=wl.decode_reqs[2].v),
            DecodeRequest(doc_ids=[c, c], k=wl.decode_reqs[0].k, v=wl.decode_reqs[0].v)]
    wl.decode_reqs = decs
    say(f"[repeated documents] prefill {[r.doc_ids for r in pre]}, decode {[r.doc_ids for r in decs]}")
    out, gate_p = _prefill(wl, poison=False)
    got, gate_d = _decode(wl, poison=False, steps=[0, 1])
    got_m, gate_m = _decode(wl, poison=False, steps=[0, 1], doc_major=True)  # read twice by one request: two slots
    assert np.isfinite(out).all()
    gate_p.check()
    gate_d.check()
    gate_m.check()
