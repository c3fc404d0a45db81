"""Stream ordering of the document-major decode.

The call's launches (the document pass, the split-K launch over any tiles
left out of it, the combine) go to the caller's stream: its output must be complete once that
stream alone is synchronised, on any stream, and repeated calls on
different streams must give the same bits (the kernels are deterministic:
no atomics, fixed reduction orders).
"""

import pytest
import torch

from tests.harness import say
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("key", ["ragged", "llama8b_decode"])
def test_shared_decode_complete_in_caller_stream_order(key):
    from position_agnostic_paged_amd.engine import Engine
    from position_agnostic_paged_amd.scenarios import DecodeScenario, blocks_needed, make_pos

    wl = make_workload(key)
    wl.num_decode_steps = 2
    g = wl.geom
    eng = Engine(g.num_q_heads, g.num_kv_heads, g.head_dim, g.dtype, make_pos(wl, "cuda"), blocks_needed(wl), "cuda")
    sc = DecodeScenario(wl, eng, doc_major=True, prebuild_tables=True)
    plan = sc.tables[0]
    say(f"[streams] {wl.name}: {plan.num_docs} shared documents, {plan.num_work} work items")
    assert plan.num_work > 0
    ref = sc.step(0).clone()
    torch.cuda.synchronize()
    assert torch.isfinite(ref.float()).all()
    q_pos = sc._inputs[0][3]
    for i in range(3):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            sc.out.fill_(float("nan"))  # a stale or partial result cannot pass
            out = sc.attend(0, sc.q, q_pos, stream=s)
            got = out.clone()
        s.synchronize()  # the caller's stream only
        assert torch.equal(got, ref), f"call {i}: differs from the first call"
    say(f"[streams] {wl.name}: 3 calls on fresh streams, bit-identical after their own stream's sync")
