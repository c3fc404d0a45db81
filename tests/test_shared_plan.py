"""CPU tests of the document-major decode plan (lazy_build_shared_plan): bit-exact against a plain re-derivation
of what the plan must hold, on random batches whose requests draw documents from a shared pool (some twice
in one request) -- the shared documents, their tiles at local positions, every read's (request, slot,
Delta), each request's remaining tiles (exactly lazy_build_tiles over its unshared segments) and the
document pass's work items."""

import numpy as np
import pytest

from position_agnostic_paged_amd import lazy_attn as L
from position_agnostic_paged_amd.paging import RequestLayout, Segment, blocks_for, flatten_layouts


def _batch(rng, num_docs=12, R=7, max_docs=6, dup=True):
    doc_len = {d: int(rng.integers(1, 90)) for d in range(num_docs)}
    doc_blocks, nb = {}, 0
    for d in range(num_docs):
        doc_blocks[d] = list(range(nb, nb + blocks_for(doc_len[d])))
        nb += blocks_for(doc_len[d])
    layouts = []
    for _ in range(R):
        n = int(rng.integers(0, max_docs + 1))
        ids = [int(x) for x in rng.integers(0, num_docs, size=n)] if dup else \
            [int(x) for x in rng.choice(num_docs, size=min(n, num_docs), replace=False)]
        segs, pos = [], 0
        for d in ids:
            segs.append(Segment(doc_blocks[d], doc_len[d], pos, True))
            pos += doc_len[d]
        Lq = int(rng.integers(0, 40))
        segs.append(Segment(list(range(nb, nb + blocks_for(Lq))), Lq, pos, False))
        nb += blocks_for(Lq)
        layouts.append(RequestLayout(segs))
    return layouts, nb


def _expected(layouts, kind, num_blocks, group, hkv, rb, min_readers, few):
    """What the plan must contain, derived with plain loops (few: the work-item count under which documents are
    cut into chunks).  With min_readers 1 every request's private tokens are one more item, read once at
    Delta 0 with its tiles at their global positions, and the requests keep no tiles of their own."""
    key = lambda sg: (sg.blocks[0] << 32) | sg.length  # noqa: E731
    readers = {}
    for lay in layouts:
        for sg in lay.segments:
            if sg.ctx and sg.length > 0:
                readers[key(sg)] = readers.get(key(sg), 0) + 1
    first, nread = {}, {}
    s_index = 0
    for lay in layouts:
        for sg in lay.segments:
            if sg.ctx and sg.length > 0 and readers[key(sg)] >= min_readers and key(sg) not in first:
                first[key(sg)] = sg
                nread[key(sg)] = readers[key(sg)]
            s_index += 1
    s_index = 0
    for lay in layouts:
        for sg in lay.segments:
            if min_readers == 1 and not sg.ctx and sg.length > 0:
                k = (1 << 63) | s_index
                first[k] = sg
                nread[k] = 1
            s_index += 1
    docs = sorted(first, key=lambda k: (-((first[k].length + 15) // 16) * nread[k], k))
    index = {k: i for i, k in enumerate(docs)}
    # chunks: only when the pass holds fewer than `few` work items; then up to ceil(2 few / items) even chunks
    # of at least 32 tiles per document
    ntiles = {k: (first[k].length + 15) // 16 for k in docs}
    items = hkv * sum(-(-nread[k] * group // (16 * rb)) for k in docs)
    want = -(-2 * few // items) if 0 < items < few else 1
    ct, nchunks = {}, {}
    for k in docs:
        n = max(1, min(want, ntiles[k] // 32))
        c = -(-ntiles[k] // n)
        ct[k] = (c + 1) // 2 * 2
        nchunks[k] = -(-ntiles[k] // ct[k])
    doc_tiles = []
    doc_start = [0]
    for k in docs:
        sg = first[k]
        base = 0 if sg.ctx else sg.pos0
        for b in range((sg.length + 15) // 16):
            valid = min(16, sg.length - 16 * b)
            doc_tiles.append((sg.blocks[b] << 40) | ((base + 16 * b) << 16) | ((1 << valid) - 1))
        doc_start.append(len(doc_tiles))
    reads = [[] for _ in docs]
    req_reads, own = [], []
    s_index = 0
    for r, lay in enumerate(layouts):
        slot, keep = 0, []
        for sg in lay.segments:
            k = key(sg) if sg.ctx else (1 << 63) | s_index
            s_index += 1
            if sg.length > 0 and k in index:
                reads[index[k]].append((r << 48) | (slot << 32) | (sg.pos0 if sg.ctx else 0))
                slot += nchunks[k]
            else:
                keep.append(sg)
        req_reads.append(slot)
        own.append(RequestLayout(keep))
    f = flatten_layouts(own)
    tiles, tstart, nctx = L.build_tiles(kind, f["seg_start"], f["seg_len"], f["seg_pos0"], f["seg_is_ctx"],
                                        f["seg_block_start"], f["blocks"] or [0], num_blocks,
                                        max(1, sum(blocks_for(n) for n in f["seg_len"])))
    work = []
    for i, k in enumerate(docs):
        n_items = -(-nread[k] * group // (16 * rb))
        for c in range(nchunks[k]):
            work += [(i, b * rb, c, ct[k]) for b in range(n_items)]
    return {"doc_tiles": doc_tiles, "doc_start": doc_start, "reads": reads, "req_reads": req_reads,
            "tiles": [int(w) for w in tiles], "tile_start": list(tstart), "ctx_tiles": list(nctx), "work": work}


def _pass_shape(geom):
    """(16-row blocks per work item, chunking threshold): bf16 runs the LDS-staged pass, a workgroup of 8 waves
    x 16 rows per item; fp32 the per-wave pass, 2 (dh 128) or 4 (dh 64) row blocks per item."""
    if geom.dtype == L.LAZY_BF16:
        return 8, 256
    return (2 if geom.head_dim == 128 else 4), 1024


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("kind", ["rope_half", "alibi"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_plan_matches_a_plain_derivation(seed, kind, dtype):
    rng = np.random.default_rng(seed)
    layouts, nb = _batch(rng)
    geom = L.make_geom(8 if seed % 2 else 32, 2 if seed % 2 else 8, 128 if seed % 3 else 64, dtype)
    group = geom.num_q_heads // geom.num_kv_heads
    f = flatten_layouts(layouts)
    min_readers = 1 + seed % 3
    h = L.build_shared_plan(geom, L.KIND_BY_NAME[kind], f["seg_start"], f["seg_len"], f["seg_pos0"],
                            f["seg_is_ctx"], f["seg_block_start"], f["blocks"], nb, 0, min_readers)
    rb, few = _pass_shape(geom)
    assert h["row_blocks"] == rb
    want = _expected(layouts, L.KIND_BY_NAME[kind], nb, group, geom.num_kv_heads, rb, min_readers, few)
    assert [int(w) for w in h["doc_tiles"]] == want["doc_tiles"]
    assert list(h["doc_tile_start"]) == want["doc_start"]
    got_reads = [[int(w) for w in h["reads"][h["read_start"][i]: h["read_start"][i + 1]]]
                 for i in range(h["num_docs"])]
    assert got_reads == want["reads"]
    assert list(h["req_reads"]) == want["req_reads"] and h["max_req_reads"] == max(want["req_reads"])
    assert [int(w) for w in h["tiles"]] == want["tiles"]
    assert list(h["tile_start"]) == want["tile_start"] and list(h["ctx_tiles"]) == want["ctx_tiles"]
    assert [tuple(x) for x in h["work"].reshape(-1, 4).tolist()] == want["work"]
    # every tile of every request is in exactly one of the two passes
    n_all = sum(lay.num_tiles for lay in layouts)
    shared_tiles = sum(len(rs) * (want["doc_start"][i + 1] - want["doc_start"][i]) for i, rs in enumerate(want["reads"]))
    assert h["total_tiles"] + shared_tiles == n_all


def test_plan_refusals():
    rng = np.random.default_rng(9)
    layouts, nb = _batch(rng)
    geom = L.make_geom(32, 8, 128, "bf16")
    f = flatten_layouts(layouts)
    args = (f["seg_start"], f["seg_len"], f["seg_pos0"], f["seg_is_ctx"], f["seg_block_start"], f["blocks"])
    with pytest.raises(L.LazyError, match="min_readers"):
        L.build_shared_plan(geom, 0, *args, nb, 0, 0)
    with pytest.raises(L.LazyError, match="outside the pool"):
        L.build_shared_plan(geom, 0, *args, 3, 0, 2)
    far = max(s.pos0 for lay in layouts for s in lay.segments if s.ctx and s.length)
    with pytest.raises(L.LazyError, match="cos/sin table"):
        L.build_shared_plan(geom, 0, *args, nb, far, 2)
    # a document whose reads name different block lists is not one physical copy
    bad = [RequestLayout([Segment([0, 1], 20, 0, True), Segment([5], 1, 20, False)]),
           RequestLayout([Segment([0, 2], 20, 0, True), Segment([6], 1, 20, False)])]
    fb = flatten_layouts(bad)
    with pytest.raises(L.LazyError, match="another block list"):
        L.build_shared_plan(geom, 0, fb["seg_start"], fb["seg_len"], fb["seg_pos0"], fb["seg_is_ctx"],
                            fb["seg_block_start"], fb["blocks"], 8, 0, 2)


@pytest.mark.parametrize("min_readers", [1, 2])
def test_plan_of_an_empty_batch(min_readers):
    """No request: nothing to read and no work, and the plan still names the geometry's row blocks (the
    decode call checks them before it returns for an empty batch)."""
    f = flatten_layouts([])
    for geom in (L.make_geom(32, 8, 128, "bf16"), L.make_geom(8, 2, 64, "fp32")):
        h = L.build_shared_plan(geom, 0, f["seg_start"], f["seg_len"], f["seg_pos0"], f["seg_is_ctx"],
                                f["seg_block_start"], f["blocks"], 16, 0, min_readers)
        assert (h["num_docs"], h["num_reads"], h["num_work"], h["total_tiles"], h["max_tiles"]) == (0, 0, 0, 0, 0)
        assert h["row_blocks"] == _pass_shape(geom)[0]
        assert h["tile_start"].tolist() == [0]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_plan_chunks_few_long_documents(dtype):
    """Three 4096-token documents read by 64 requests: the pass would hold a few dozen (bf16) or a few hundred
    (fp32) work items of 256 tiles, so each document is cut into chunks and each read takes one slot per chunk."""
    blocks = {d: list(range(256 * d, 256 * (d + 1))) for d in range(3)}
    layouts, nb = [], 768
    for r in range(64):
        segs, pos = [], 0
        for d in ([0, 1, 2] if r % 2 else [2, 0, 1]):
            segs.append(Segment(blocks[d], 4096, pos, True))
            pos += 4096
        segs.append(Segment([nb], 5, pos, False))
        nb += 1
        layouts.append(RequestLayout(segs))
    geom = L.make_geom(32, 8, 128, dtype)
    f = flatten_layouts(layouts)
    h = L.build_shared_plan(geom, 0, f["seg_start"], f["seg_len"], f["seg_pos0"], f["seg_is_ctx"],
                            f["seg_block_start"], f["blocks"], nb, 0, 2)
    work = h["work"].reshape(-1, 4)
    assert h["num_docs"] == 3 and h["num_reads"] == 192
    # bf16: 8 heads x 3 documents x 2 row tiles = 48 items < 256, want ceil(512 / 48) = 11 chunks, capped at
    # 256 / 32 = 8; fp32: 8 x 3 x 8 = 192 waves < 1024, want 11, capped at 8
    assert set(work[:, 3].tolist()) == {32} and set(work[:, 2].tolist()) == set(range(8))
    assert list(h["req_reads"]) == [24] * 64  # 3 documents x 8 chunks
    rb, few = _pass_shape(geom)
    want = _expected(layouts, 0, nb, 4, 8, rb, 2, few)
    assert [tuple(x) for x in work.tolist()] == want["work"]
