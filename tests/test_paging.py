"""Host paging: block pool, document cache (one copy per document, LRU eviction of whole unpinned
documents, private blocks charged to the same budget) and request layouts."""

import pytest

from position_agnostic_paged_amd.paging import (BlockPool, CacheFull, DocCache, RequestLayout, Segment, blocks_for,
                                                layout_request, order_for_reuse)


def test_blocks_for():
    assert [blocks_for(n) for n in (0, 1, 16, 17, 200, 500, 1600)] == [0, 1, 1, 2, 13, 32, 100]


def test_one_copy_per_document_and_hits():
    c = DocCache(BlockPool(100))
    b1, hit1 = c.acquire(7, 40)
    b2, hit2 = c.acquire(7, 40)
    assert not hit1 and hit2 and b1 == b2 and len(b1) == 3
    assert c.used == 3 and c.hits == 1 and c.misses == 1


def test_lru_evicts_least_recent_unpinned_whole_documents():
    c = DocCache(BlockPool(10))
    for d in range(3):  # 3 docs x 3 blocks
        c.acquire(d, 48)
        c.release(d)
    c.acquire(0, 48)  # doc 0 becomes most recent (and pinned)
    c.acquire(3, 48)  # needs 3 blocks, 1 free -> evict doc 1 (LRU, unpinned)
    assert 1 not in c and 0 in c and 2 in c and 3 in c
    assert c.evictions == 1


def test_pinned_documents_are_never_evicted():
    c = DocCache(BlockPool(6))
    c.acquire(0, 48)
    c.acquire(1, 48)
    with pytest.raises(CacheFull):
        c.acquire(2, 16)
    c.release(1)
    blocks, hit = c.acquire(2, 16)
    assert not hit and 1 not in c and 0 in c


def test_private_blocks_share_the_budget():
    c = DocCache(BlockPool(100), budget_blocks=8)
    c.acquire(0, 64)  # 4 blocks
    c.release(0)
    assert c.room_for_private(8) and not c.room_for_private(9)
    p = c.take_private(6)  # evicts doc 0
    assert len(p) == 6 and 0 not in c and c.used == 6
    c.give_back_private(p)
    assert c.used == 0


def test_layout_places_documents_consecutively():
    lay = layout_request([([1, 2], 20), ([3], 5)], [9], 3)
    assert [(s.pos0, s.length, s.ctx) for s in lay.segments] == [(0, 20, True), (20, 5, True), (25, 3, False)]
    assert lay.length == 28 and lay.num_tiles == 4


def test_forget_drops_an_unwritten_miss_and_returns_its_blocks():
    c = DocCache(BlockPool(8))
    blocks, hit = c.acquire(5, 40)  # a miss, pinned, content not yet written
    assert not hit and c.used == 3 and c.pool.free_blocks == 5
    c.forget(5)
    assert 5 not in c and c.used == 0 and c.pool.free_blocks == 8
    b2, hit2 = c.acquire(5, 40)  # asked again: a miss again, not a hit on unwritten blocks
    assert not hit2 and sorted(b2) == sorted(blocks)


def test_order_for_reuse_lists_shared_documents_first_and_keeps_everything():
    """Each request keeps exactly its segments (offsets attached), private tokens stay last, and the
    documents go most shared first, ties by first block: a shared document gets the same rank in
    every request that reads it."""
    a, b = Segment([10, 11], 20, 0, True), Segment([3], 7, 0, True)
    c, d = Segment([40], 16, 0, True), Segment([7], 5, 0, True)

    def at(sg, pos):
        return Segment(sg.blocks, sg.length, pos, True)

    lays = [
        RequestLayout([at(c, 0), at(a, 16), at(b, 36), Segment([90], 3, 43, False)]),
        RequestLayout([at(b, 0), at(d, 7), at(a, 12), Segment([91, 92], 17, 32, False)]),
        RequestLayout([at(a, 0), at(c, 20), Segment([93], 1, 36, False)]),
        RequestLayout([Segment([94], 4, 0, False)]),
    ]
    out = order_for_reuse(lays)
    # a: 3 requests, b: 2, c: 2 (first block 40 > 3), d: 1
    firsts = [[sg.blocks[0] for sg in lay.segments] for lay in out]
    assert firsts == [[10, 3, 40, 90], [10, 3, 7, 91], [10, 40, 93], [94]]
    for before, after in zip(lays, out):
        key = lambda sg: (sg.blocks[0], sg.pos0, sg.length, sg.ctx)
        assert sorted(map(key, before.segments)) == sorted(map(key, after.segments))
        assert not after.segments[-1].ctx or all(sg.ctx for sg in after.segments)
        assert after.length == before.length


def test_unpinned_count_tracks_every_transition():
    """room_for_private relies on a running count of unpinned blocks: it must equal the plain sum after any
    mix of hits, misses, releases, forgets and evictions."""
    import numpy as np

    from position_agnostic_paged_amd.paging import BlockPool, DocCache

    rng = np.random.default_rng(0)
    cache = DocCache(BlockPool(200), budget_blocks=150)
    held = []
    for _ in range(2000):
        op = rng.integers(0, 4)
        if op < 2:
            d = int(rng.integers(0, 40))
            try:
                cache.acquire(d, int(16 * (1 + d % 5)))
                held.append(d)
            except Exception:
                pass
        elif op == 2 and held:
            cache.release(held.pop(int(rng.integers(0, len(held)))))
        elif op == 3 and len(cache):
            d = next(iter(cache._docs))
            if d not in held:
                cache.forget(d)
        want = sum(len(x.blocks) for x in cache._docs.values() if x.pins == 0)
        assert cache.unpinned == want
