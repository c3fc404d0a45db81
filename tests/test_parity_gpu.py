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


def _check_decode(key, steps, reqs=None, shared=True, prerotated=False, num_steps=None, on_the_fly=False):
    from position_agnostic_paged_amd.scenarios import DecodeScenario

    wl = make_workload(key)
    if num_steps is not None:
        wl.num_decode_steps = num_steps
    say(f"[decode parity] {wl.name} steps={list(steps)} shared={shared} prerotated={prerotated} "
        f"on_the_fly={on_the_fly}")
    eng = _engine(wl, shared, on_the_fly=on_the_fly)
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


def test_ragged_prefill():
    """Questions of 1..64 tokens (two row tiles), a request with no document, 1..999-token documents."""
    _check_prefill("ragged")


def test_ragged_decode_uneven_splits():
    """Requests from 7 to 11K tokens: per-request split counts differ inside one launch."""
    _check_decode("ragged", steps=[0, 2, 4])


def test_llama8b_prefill_on_the_fly_sincos():
    _check_prefill("llama8b_prefill", on_the_fly=True)


@pytest.mark.parametrize("on_the_fly", [False, True], ids=["table", "on_the_fly"])
def test_long_context_offsets_beyond_100k(on_the_fly):
    """128K-token contexts, base 1e4: document offsets up to ~128K (angles ~1.3e5 rad) through the
    fp32 table and through the in-kernel fp64-reduced sincos, 8023 tiles in one request (offsets past
    2^16 in the tile words, many splits).  The attention output averages over so many keys that it
    cannot see a small angle error; the rotation itself is checked element by element at these
    positions in test_rotation_gpu."""
    _check_prefill("long_context", on_the_fly=on_the_fly)
    _check_decode("long_context", steps=[0, 1], on_the_fly=on_the_fly)


def test_mixed_yarn_prefill_step0():
    """YaRN x8 (original 8192) 70B shape: 4 prefills of 15 x 500-token documents + 64-token questions."""
    from workloads import gen

    wl = gen._mixed_llama70b(num_steps=1)
    wl.decode_reqs = []
    _check_prefill_wl(wl)


def test_mixed_yarn_decode_sampled():
    """48 decodes at 8K-66K context (YaRN), sampled requests including the longest."""
    from workloads import gen

    wl = gen._mixed_llama70b(num_steps=3)
    wl.prefill_steps = []
    lens = [wl.decode_ctx_len(r) for r in range(len(wl.decode_reqs))]
    reqs = sorted({int(np.argmax(lens)), int(np.argmin(lens)), 7, 30})
    _check_decode_wl(wl, steps=[0, 2], reqs=reqs)


def _check_prefill_wl(wl):
    from position_agnostic_paged_amd.scenarios import PrefillScenario

    say(f"[prefill parity] {wl.name}")
    eng = _engine(wl)
    sc = PrefillScenario(wl, eng)
    out = sc.run().float().cpu().numpy()
    want = oracle_prefill(wl, 0, range(len(sc.reqs)))
    err = max(max_abs(out[sc.q_start_h[i]: sc.q_start_h[i + 1]], w) for i, w in enumerate(want))
    say(f"  max-abs err {err:.3e} (tol {TOL[wl.geom.dtype]})")
    assert err <= TOL[wl.geom.dtype]


def _check_decode_wl(wl, steps, reqs):
    from position_agnostic_paged_amd.scenarios import DecodeScenario

    say(f"[decode parity] {wl.name} steps={steps} reqs={reqs}")
    eng = _engine(wl)
    sc = DecodeScenario(wl, eng)
    draws, got = {}, {}
    for s in range(max(steps) + 1):
        draws[s] = wl.decode_step(s)
        out = sc.step(s)
        if s in steps:
            got[s] = out.float().cpu().numpy()
    err = 0.0
    for r in reqs:
        for s, w in zip(steps, oracle_decode(wl, r, steps, draws)):
            err = max(err, max_abs(got[s][r], w))
    say(f"  max-abs err {err:.3e} (tol {TOL[wl.geom.dtype]})")
    assert err <= TOL[wl.geom.dtype]


def test_device_unpack_bit_exact():
    """The kernels' own word split (through lazy_debug_unpack) equals the oracle's on boundary + random words."""
    from oracle import pack as OP
    from position_agnostic_paged_amd import lazy_attn as L

    rng = np.random.default_rng(21)
    vals = [(0, 0, 1), ((1 << 24) - 1, (1 << 24) - 1, 0xFFFF), (0, 0, 0x8000), (123, 456, 0x0F0F)]
    vals += [(int(b), int(o), int(m)) for b, o, m in zip(rng.integers(0, 1 << 24, 100000),
                                                          rng.integers(0, 1 << 24, 100000),
                                                          rng.integers(1, 1 << 16, 100000))]
    words = np.array([OP.pack(*v) for v in vals], dtype=np.uint64)
    wd = torch.from_numpy(words.view(np.int64)).cuda()
    n = len(vals)
    blk, off, msk = (torch.empty(n, dtype=torch.int32, device="cuda") for _ in range(3))
    L.debug_unpack(wd, blk, off, msk)
    got = np.stack([blk.cpu().numpy(), off.cpu().numpy(), msk.cpu().numpy()], 1).astype(np.int64)
    assert np.array_equal(got, np.array(vals, dtype=np.int64))


def test_attention_never_writes_the_cache():
    """Zero-copy reuse: prefill and decode read cached documents in place and leave the pools byte-identical."""
    from position_agnostic_paged_amd.scenarios import DecodeScenario, PrefillScenario

    wl = make_workload("ragged")
    eng = _engine(wl)
    sc = PrefillScenario(wl, eng)
    dec = DecodeScenario(wl, eng, num_steps=2)
    dec.step(0)  # writes its token
    torch.cuda.synchronize()
    kb, vb = eng.k_cache.clone(), eng.v_cache.clone()
    for _ in range(3):
        sc.run()
        eng.decode(dec.table(0), dec.q, torch.from_numpy(dec.positions(0)).cuda(), out=dec.out)
    torch.cuda.synchronize()
    assert torch.equal(kb.view(torch.int16), eng.k_cache.view(torch.int16))
    assert torch.equal(vb.view(torch.int16), eng.v_cache.view(torch.int16))


def test_falcon_alibi_prefill_mqa_dh64():
    """ALiBi bias in the LDS-staged prefill: bf16, dh 64, MQA 71/1 (rows of one KV head span 14 row tiles)."""
    _check_prefill("falcon7b_alibi_prefill")


def test_dh64_interleaved_prefill_decode_and_control():
    """dh 64 interleaved RoPE through the staged prefill (K rotated in LDS), the decode kernel and the
    pre-rotated control on the no-sharing layout."""
    _check_prefill("small_dh64_interleaved")
    _check_prefill("small_dh64_interleaved", shared=False, prerotated=True)
    _check_decode("small_dh64_interleaved", steps=[0, 1, 2, 3])


def test_uneven_decode_prerotated_control_and_alibi():
    """Uneven batches (7 to 11K tokens) run the decode build limited to three waves per SIMD: its
    pre-rotated variant (no-sharing control) and its ALiBi variant (group 4), against the oracle."""
    from workloads.gen import PosSpec

    _check_decode("ragged", steps=[0, 2], shared=False, prerotated=True)
    wl = make_workload("ragged")
    wl.pos = PosSpec("alibi")
    _check_decode_wl(wl, steps=[0, 1], reqs=range(len(wl.decode_reqs)))


def test_documents_in_request_order_without_reuse_ordering():
    """The engine lists documents most shared first by default; the request's own order (ordering
    off) is an equally valid tile list and must give the same attention (prefill and decode)."""
    from position_agnostic_paged_amd.engine import Engine

    Engine.order_for_reuse = False
    try:
        _check_prefill("ragged")
        _check_decode("ragged", steps=[0, 3])
    finally:
        Engine.order_for_reuse = True
