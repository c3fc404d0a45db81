"""CPU checks of the test harness's negative control: the planted no-Delta oracle must coincide with the
true oracle where every document sits at offset 0 (nothing to drop) and must differ where documents are
moved, for RoPE and ALiBi alike; and the gate must fail an all-zero output on a long soft-attention
context that the absolute bound alone would pass."""

import dataclasses

import numpy as np
import pytest

from tests import harness as H
from workloads import PrefillRequest, make_workload
from workloads.gen import PosSpec


def _single_doc(wl):
    r = wl.prefill_steps[0][0]
    return dataclasses.replace(wl, prefill_steps=[[PrefillRequest(r.doc_ids[:1], r.q, r.k, r.v)]], _doc_cache={})


@pytest.mark.parametrize("kind", ["rope_half", "alibi"])
def test_nodelta_is_the_oracle_without_offsets(kind):
    wl = make_workload("tiny_fp32")
    wl.pos = PosSpec(kind, base=1e4)
    one = _single_doc(wl)
    want = H.oracle_prefill(one, 0, [0])[0]
    assert np.max(np.abs(H.nodelta_prefill(one, 0, 0) - want)) < 1e-12
    want = H.oracle_prefill(wl, 0, [0])[0]
    assert np.max(np.abs(H.nodelta_prefill(wl, 0, 0) - want)) > 0.1 * np.max(np.abs(want))


def test_nodelta_decode_tracks_generated_tokens():
    wl = make_workload("tiny_fp32")
    w = H.oracle_decode(wl, 0, [5])[0]
    n = H.nodelta_decode(wl, 0, 5)
    assert n.shape == w.shape
    assert np.max(np.abs(n - w)) > 0.1 * np.max(np.abs(w))


def test_gate_rejects_a_zero_output_that_the_absolute_bound_passes():
    want = np.full((4, 8), 0.012)  # the scale of a 32K-token soft-attention output
    g = H.Gate("zero output", "bf16")
    g.add(np.zeros_like(want), want)
    g.add_negative(want * 0.25, want)
    assert g.abs <= H.TOL["bf16"]
    with pytest.raises(AssertionError, match="relative error"):
        g.check()


def test_gate_fails_when_the_negative_control_is_too_close():
    want = np.ones((2, 3))
    g = H.Gate("weak control", "bf16")
    g.add(want, want)
    g.add_negative(want * 1.01, want)
    with pytest.raises(AssertionError, match="cannot tell"):
        g.check()
