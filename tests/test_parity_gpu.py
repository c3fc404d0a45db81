"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by element.

Each test applies the gates of tests/harness.py: max-abs within the method's
precision contract (1e-4 fp32, 2e-2 bf16), max-abs within 5 % (bf16) of the
output's own scale, and a negative control showing that a kernel which
ignored the document offsets would fail the test on these very inputs.
Workloads are the seeded synthetic ones; the oracle runs in a pool of CPU
processes.
"""

import numpy as np
import pytest
import torch

from tests.harness import (Gate, decode_tasks, gather_decode, oracle_map, say)
from workloads import make_workload, sharpened

pytestmark = pytest.mark.gpu


def _engine(wl, shared=True, extra_blocks=0, on_the_fly=False):
    from position_agnostic_paged_amd.engine import Engine
    from position_agnostic_paged_amd.scenarios import blocks_needed, make_pos

    pos = make_pos(wl, "cuda", on_the_fly=on_the_fly)
    g = wl.geom
    nb = blocks_needed(wl, shared) + extra_blocks
    return Engine(g.num_q_heads, g.num_kv_heads, g.head_dim, g.dtype, pos, nb, "cuda")


def _wl(key_or_wl):
    return make_workload(key_or_wl) if isinstance(key_or_wl, str) else key_or_wl


# ------------------------------------------------------------------------------------------ prefill

def run_prefill(wl, variants):
    """GPU prefill outputs per variant (shared, prerotated, on_the_fly[, paired]), each on its own engine;
    paired (default True): tile lists closed to whole pairs per document, the query rotated per document;
    False: plain tile lists, K rotated per pair in LDS."""
    from position_agnostic_paged_amd.scenarios import PrefillScenario

    outs = {}
    for v in variants:
        shared, prerotated, on_the_fly = v[:3]
        eng = _engine(wl, shared, on_the_fly=on_the_fly)
        eng.prefill_pairs = v[3] if len(v) > 3 else True
        sc = PrefillScenario(wl, eng, shared=shared, prerotated=prerotated)
        out = sc.run().float().cpu().numpy()
        torch.cuda.synchronize()
        outs[tuple(v)] = [out[sc.q_start_h[i]: sc.q_start_h[i + 1]] for i in range(len(sc.reqs))]
        del sc, eng
        torch.cuda.empty_cache()
    return outs


def check_prefill(key, variants=((True, False, False),), negative=True):
    wl = _wl(key)
    n = len(wl.prefill_steps[0])
    say(f"[prefill parity] {wl.name}: {n} requests, variants (shared, prerotated, on_the_fly) {list(variants)}")
    outs = run_prefill(wl, variants)
    tasks = [("prefill", 0, i) for i in range(n)]
    neg = [("nodelta_prefill", 0, i) for i in range(n)] if negative else []
    res = oracle_map(wl, tasks + neg)
    want, planted = res[:n], res[n:]
    for v, got in outs.items():
        gate = Gate(f"{wl.name} {v}", wl.geom.dtype)
        for g_, w in zip(got, want):
            gate.add(g_, w)
        for p, w in zip(planted, want):
            gate.add_negative(p, w)
        gate.check(negative)


# ------------------------------------------------------------------------------------------- decode

def run_decode(wl, steps, shared=True, prerotated=False, on_the_fly=False, doc_major=False, num_steps=None):
    """GPU decode outputs {step: [R][Hq][dh]} over consecutive steps 0..max(steps); doc_major runs the
    document-major decode (shared documents read once for all their readers)."""
    from position_agnostic_paged_amd.scenarios import DecodeScenario

    eng = _engine(wl, shared, on_the_fly=on_the_fly)
    sc = DecodeScenario(wl, eng, shared=shared, prerotated=prerotated, num_steps=num_steps, doc_major=doc_major)
    if doc_major:
        plan = sc.table(0)
        say(f"  document-major plan at step 0: {plan.num_docs} shared documents, {plan.num_reads} reads, "
            f"{plan.num_work} work items, {plan.total_tiles} tiles left to the requests' own lists")
    got = {}
    for s in range(max(steps) + 1):
        out = sc.step(s)
        if s in steps:
            got[s] = out.float().cpu().numpy()
    torch.cuda.synchronize()
    del sc, eng
    torch.cuda.empty_cache()
    return got


def check_decode(key, steps, reqs=None, variants=((True, False, False),), num_steps=None, neg_reqs=4,
                 negative=True):
    wl = _wl(key)
    if num_steps is not None:
        wl.num_decode_steps = num_steps
    R = len(wl.decode_reqs)
    reqs = list(range(R)) if reqs is None else list(reqs)
    say(f"[decode parity] {wl.name}: requests {len(reqs)}/{R}, steps {list(steps)}, variants {list(variants)}")
    gots = {v: run_decode(wl, steps, *v) for v in variants}
    tasks = decode_tasks(reqs, steps)
    neg = [("nodelta_decode", r, steps[0]) for r in reqs[:neg_reqs]] if negative else []
    res = oracle_map(wl, tasks + neg)
    want = gather_decode(tasks, res[: len(tasks)])
    for v, got in gots.items():
        gate = Gate(f"{wl.name} {v}", wl.geom.dtype)
        for (r, s), w in want.items():
            gate.add(got[s][r], w)
        for t, p in zip(neg, res[len(tasks):]):
            gate.add_negative(p, want[(t[1], t[2])])
        gate.check(negative)


SHARED = (True, False, False)
NOSHARE_PREROT = (False, True, False)  # the overhead control: private copies at global positions, no deferral
NOSHARE = (False, False, False)
ON_THE_FLY = (True, False, True)
DOC_MAJOR = (True, False, False, True)  # decode: shared documents once for all their readers
DOC_MAJOR_FLY = (True, False, True, True)
# prefill: plain tile lists, K rotated per tile pair in LDS (the other prefill variants keep each tile pair
# within one document and rotate the query per document)
KROT = (True, False, False, False)


# ---------------------------------------------------------------------------------------- the tests

def test_tiny_fp32_prefill():
    check_prefill("tiny_fp32", variants=(SHARED, ON_THE_FLY, NOSHARE_PREROT))


def test_tiny_fp32_decode():
    check_decode("tiny_fp32", steps=list(range(8)), variants=(SHARED, ON_THE_FLY, NOSHARE_PREROT, DOC_MAJOR))


def test_tiny_fp32_decode_document_major_two_orders():
    """fp32 through the document pass: two requests read both documents, in opposite orders (each document
    at two different offsets), plus their own question tokens."""
    from workloads.gen import DecodeRequest

    wl = make_workload("tiny_fp32")
    r0 = wl.decode_reqs[0]
    wl.decode_reqs = [r0, DecodeRequest(doc_ids=[1, 0], k=r0.k[:9], v=r0.v[:9])]
    check_decode(wl, steps=[0, 3, 7], variants=(SHARED, DOC_MAJOR, DOC_MAJOR_FLY))


def test_llama8b_prefill_and_controls():
    """Config 2 (8 x (10 Zipf docs of 200 tokens + 32-token question), GQA 32/8) through the staged
    kernel, the in-kernel sincos path, and the no-sharing layout with and without deferral."""
    check_prefill("llama8b_prefill", variants=(SHARED, KROT, ON_THE_FLY, NOSHARE, NOSHARE_PREROT))


def test_llama8b_prefill_interleaved():
    check_prefill("llama8b_prefill_interleaved", variants=(SHARED, KROT, NOSHARE_PREROT))


def test_llama8b_decode_every_request_and_prerotated_control():
    """Config 3 (64 x 32K tokens): every request at steps 0, 31 and 63 of the 64-step run, through the
    shared-document cache and through the no-sharing pre-rotated control the overhead A/B times."""
    check_decode("llama8b_decode", steps=[0, 31, 63], variants=(SHARED, NOSHARE_PREROT, DOC_MAJOR))


def test_llama8b_decode_sample_every_step():
    """Config 3: a seeded sample of 8 requests checked at every one of the 64 steps."""
    rng = np.random.default_rng(3)
    reqs = sorted(rng.choice(64, size=8, replace=False).tolist())
    check_decode("llama8b_decode", steps=list(range(64)), reqs=reqs)


def test_llama8b_decode_sharp_queries():
    """Config 3 with queries x4 (sharper attention, larger outputs): sampled requests, first and last step,
    shared and no-sharing deferred layouts."""
    rng = np.random.default_rng(4)
    reqs = sorted(rng.choice(64, size=12, replace=False).tolist())
    check_decode(sharpened(make_workload("llama8b_decode")), steps=[0, 63], reqs=reqs,
                 variants=(SHARED, NOSHARE, DOC_MAJOR))


def test_falcon_alibi_decode_every_request():
    """Config 5 (MQA 71/1, dh 64, ALiBi, 128 x 16K): every request at steps 0, 31, 63 of 64, shared
    documents and the no-sharing control."""
    check_decode("falcon7b_alibi", steps=[0, 31, 63], variants=(SHARED, NOSHARE, DOC_MAJOR))


def test_ragged_prefill():
    """Questions of 1..64 tokens (two row tiles), a request with no document, 1..999-token documents."""
    check_prefill("ragged", variants=(SHARED, KROT, NOSHARE_PREROT))


def test_ragged_decode_uneven_splits():
    """Requests from 7 to 11K tokens: per-request split counts differ inside one launch (the three-wave
    build for uneven batches), with its pre-rotated control."""
    check_decode("ragged", steps=[0, 2, 4], variants=(SHARED, NOSHARE_PREROT, DOC_MAJOR))


@pytest.mark.parametrize("on_the_fly", [False, True], ids=["table", "on_the_fly"])
def test_long_context_offsets_beyond_100k(on_the_fly):
    """128K-token contexts, base 1e4: document offsets up to ~128K (angles ~1.3e5 rad) through the fp32
    table and through the in-kernel fp64-reduced sincos, 8023 tiles in one request (offsets past 2^16 in
    the tile words, many splits); queries x4 so the outputs depend on where every document sits."""
    v = ON_THE_FLY if on_the_fly else SHARED
    check_prefill(sharpened(make_workload("long_context")), variants=(v,))
    check_decode(sharpened(make_workload("long_context")), steps=[0, 1],
                 variants=(v, DOC_MAJOR_FLY if on_the_fly else DOC_MAJOR))


def test_mixed_yarn_prefill_and_prerotated_control():
    """YaRN x8 (original 8192) 70B shape: 4 prefills of 15 x 500-token documents + 64-token questions;
    the shared layout and the no-sharing pre-rotated control the overhead A/B times."""
    from workloads import gen

    wl = gen._mixed_llama70b(num_steps=1)
    wl.decode_reqs = []
    check_prefill(wl, variants=(SHARED, KROT, NOSHARE, NOSHARE_PREROT))


def test_mixed_yarn_decode_every_request():
    """48 decodes at 8K-66K context (YaRN): every request at steps 0 and 2."""
    from workloads import gen

    wl = gen._mixed_llama70b(num_steps=3)
    wl.prefill_steps = []
    check_decode(wl, steps=[0, 2], variants=(SHARED, DOC_MAJOR))


def test_pages_overhead_shape_prefill():
    """The pages' overhead experiment shape (5 x 4096-token documents, 3 shared, + 64-token question):
    prefill shared, and the no-sharing layout with and without deferral (the overhead A/B pair)."""
    wl = make_workload("pages_overhead")
    wl.decode_reqs = []
    check_prefill(wl, variants=(SHARED, KROT, NOSHARE, NOSHARE_PREROT))


def test_pages_overhead_shape_decode():
    """The pages' overhead shape in decode: 64 requests, every one at its first and last step, shared and
    the no-sharing A/B pair."""
    wl = make_workload("pages_overhead")
    wl.prefill_steps = []
    check_decode(wl, steps=[0, 3], variants=(SHARED, NOSHARE, NOSHARE_PREROT, DOC_MAJOR))


def test_falcon_alibi_prefill_mqa_dh64():
    """ALiBi bias in the LDS-staged prefill: bf16, dh 64, MQA 71/1 (rows of one KV head span 14 row tiles)."""
    check_prefill("falcon7b_alibi_prefill", variants=(SHARED, NOSHARE))


def test_dh64_interleaved_prefill_decode_and_control():
    """dh 64 interleaved RoPE through the staged prefill (K rotated in LDS), the decode kernel and the
    pre-rotated control on the no-sharing layout."""
    check_prefill("small_dh64_interleaved", variants=(SHARED, KROT, NOSHARE_PREROT))
    check_decode("small_dh64_interleaved", steps=[0, 1, 2, 3], variants=(SHARED, NOSHARE_PREROT, DOC_MAJOR))


def test_uneven_decode_alibi():
    """Uneven batches (7 to 11K tokens) run the decode build limited to three waves per SIMD: its ALiBi
    variant (group 4)."""
    from workloads.gen import PosSpec

    wl = make_workload("ragged")
    wl.pos = PosSpec("alibi")
    check_decode(wl, steps=[0, 1], variants=(SHARED, DOC_MAJOR))


def test_documents_in_request_order_without_reuse_ordering():
    """The engine lists documents most shared first by default; the request's own order (ordering
    off) is an equally valid tile list and must give the same attention (prefill and decode)."""
    from position_agnostic_paged_amd.engine import Engine

    Engine.order_for_reuse = False
    try:
        check_prefill("ragged")
        check_decode("ragged", steps=[0, 3])
    finally:
        Engine.order_for_reuse = True


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
