"""GPU parity of the document-processing pass that runs on a cache miss.

A missed document is encoded once: its K/V are written at local positions
0..L-1 (the position-agnostic copy) and its own tokens attend causally to
each other at those positions.  The output must equal plain causal attention
over the document alone (the oracle with no cached context and the document
as the suffix), and the copy it leaves behind must then serve any later
request at any offset: a request that puts the same documents, in another
order, in front of a question must match the oracle's eager-position
attention over the whole sequence.
"""

import dataclasses

import numpy as np
import pytest
import torch

from oracle import attention as OA
from tests.harness import Gate, nodelta_prefill, oracle_var, say
from workloads import PrefillRequest, make_workload

pytestmark = pytest.mark.gpu


def _dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dtype)


def test_document_processing_miss_then_reuse():
    from position_agnostic_paged_amd.engine import Engine
    from position_agnostic_paged_amd.paging import RequestLayout, Segment, blocks_for
    from position_agnostic_paged_amd.scenarios import make_pos

    wl = make_workload("ragged")
    g = wl.geom
    by_len = sorted(wl.doc_lens, key=lambda d: (wl.doc_lens[d], d))
    # the shortest and the longest documents and two between: ragged last
    # blocks, one to sixteen 256-row tiles of GQA-packed queries
    pick = [by_len[0], by_len[len(by_len) // 3], by_len[(2 * len(by_len)) // 3], by_len[-1]]
    lens = [wl.doc_lens[d] for d in pick]
    Lq = 24
    say(f"[doc processing] {wl.name}: documents {pick} of {lens} tokens, then a {Lq}-token question")
    nb = sum(blocks_for(n) for n in lens) + blocks_for(Lq) + 2
    eng = Engine(g.num_q_heads, g.num_kv_heads, g.head_dim, g.dtype, make_pos(wl, "cuda"), nb, "cuda")
    dt = eng.tdtype

    items = []
    for d in pick:
        k, v = wl.doc(d)
        items.append((d, _dev(k, dt), _dev(v, dt), _dev(wl.doc_queries(d), dt)))
    out, _ = eng.process_documents(items)
    out = out.float().cpu().numpy()
    torch.cuda.synchronize()

    var = oracle_var(wl)
    gate = Gate("document pass", g.dtype)
    off = 0
    for d, n in zip(pick, lens):
        k, v = wl.doc(d)
        want = OA.eager_prefill([], wl.doc_queries(d), k, v, var)
        gate.add(out[off: off + n], want)
        off += n
    # every document sits at offset 0 here: there is no Delta to drop, so no negative control
    gate.check(negative=False)

    # reuse: the cached copies at new offsets, in reverse order, before a question
    order = pick[::-1]
    qq, kq, vq = wl.extra_question(0, Lq)
    segs, p = [], 0
    for d in order:
        segs.append(Segment(eng.docs.blocks(d), wl.doc_lens[d], p, True))
        p += wl.doc_lens[d]
    priv = eng.docs.take_private(blocks_for(Lq))
    segs.append(Segment(priv, Lq, p, False))
    Q = _dev(qq, dt)
    eng.write_segment(priv, _dev(kq, dt), _dev(vq, dt), p, q=Q)
    tt = eng.tile_table([RequestLayout(segs)])
    q_start = torch.tensor([0, Lq], dtype=torch.int32, device="cuda")
    q_pos0 = torch.tensor([p], dtype=torch.int32, device="cuda")
    got = eng.prefill(tt, Q, q_start, q_pos0, Lq).float().cpu().numpy()
    torch.cuda.synchronize()
    want = OA.eager_prefill([wl.doc(d) for d in order], qq, kq, vq, var)
    say(f"  reuse at offsets {np.cumsum([0] + [wl.doc_lens[d] for d in order[:-1]]).tolist()}")
    reuse = dataclasses.replace(wl, prefill_steps=[[PrefillRequest(list(order), qq, kq, vq)]], _doc_cache={})
    gate = Gate("reuse at new offsets", g.dtype)
    gate.add(got, want)
    gate.add_negative(nodelta_prefill(reuse, 0, 0), want)
    gate.check()

    # a document already cached has no miss to process
    with pytest.raises(ValueError):
        eng.process_documents([items[0]])
