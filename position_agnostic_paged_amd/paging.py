"""Host-side paging: a block pool, a position-agnostic document cache and
request layouts.  Pure Python, no device work.

One cached copy per document, reused at any position (LazyAttention notes,
papernotes.org, "Background and motivation": a position-agnostic cache keeps
the top-C documents instead of floor(C/D) position variants; repository
landing page, "Demo": one copy per document reused regardless of slot).
Documents are cached whole and evicted whole in least-recently-used order;
documents referenced by the work in flight are pinned.

``PositionAwareCache`` is the design the pages compare against (the notes'
"Background and motivation"; the gist.science summary, "Contesto": existing
systems materialise a re-encoded copy per position): an entry is a document
at one global offset, so the same document at another offset is a miss and
takes another copy from the same budget.
"""

from __future__ import annotations

from collections import OrderedDict
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

BLOCK_SIZE = 16


def blocks_for(tokens: int) -> int:
    return (tokens + BLOCK_SIZE - 1) // BLOCK_SIZE


class CacheFull(RuntimeError):
    pass


class BlockPool:
    """Free list of physical block ids [0, num_blocks)."""

    def __init__(self, num_blocks: int):
        self.num_blocks = num_blocks
        self._free: List[int] = list(range(num_blocks - 1, -1, -1))

    @property
    def free_blocks(self) -> int:
        return len(self._free)

    def alloc(self, n: int) -> List[int]:
        if n > len(self._free):
            raise CacheFull(f"need {n} blocks, {len(self._free)} free")
        out = [self._free.pop() for _ in range(n)]
        return out

    def free(self, blocks: Sequence[int]) -> None:
        self._free.extend(reversed(list(blocks)))


@dataclass
class CachedDoc:
    blocks: List[int]
    length: int
    pins: int = 0


class DocCache:
    """doc id -> blocks of its position-agnostic copy, with LRU eviction of unpinned documents."""

    def __init__(self, pool: BlockPool, budget_blocks: Optional[int] = None):
        self.pool = pool
        self.budget = budget_blocks if budget_blocks is not None else pool.num_blocks
        self._docs: "OrderedDict[int, CachedDoc]" = OrderedDict()
        self.used = 0
        self.unpinned = 0  # blocks of cached entries no work holds (what eviction can free)
        self.hits = 0
        self.misses = 0
        self.evictions = 0

    def __contains__(self, doc_id: int) -> bool:
        return doc_id in self._docs

    def __len__(self) -> int:
        return len(self._docs)

    def blocks(self, doc_id: int) -> List[int]:
        return self._docs[doc_id].blocks

    def acquire(self, doc_id: int, length: int, reserve: int = 0) -> Tuple[List[int], bool]:
        """Pin a document; returns (blocks, hit).  On a miss the caller must write its content.

        ``reserve`` blocks of the budget are kept free for other allocations
        (private suffix blocks come from the same budget).
        """
        d = self._docs.get(doc_id)
        if d is not None:
            if d.length != length:
                raise ValueError(f"doc {doc_id} cached with length {d.length}, asked {length}")
            self._docs.move_to_end(doc_id)
            if d.pins == 0:
                self.unpinned -= len(d.blocks)
            d.pins += 1
            self.hits += 1
            return d.blocks, True
        need = blocks_for(length)
        self._make_room(need + reserve)
        blocks = self.pool.alloc(need)
        self._docs[doc_id] = CachedDoc(blocks, length, pins=1)
        self.used += need
        self.misses += 1
        return blocks, False

    def release(self, doc_id: int) -> None:
        d = self._docs[doc_id]
        if d.pins <= 0:
            raise ValueError(f"doc {doc_id} is not pinned")
        d.pins -= 1
        if d.pins == 0:
            self.unpinned += len(d.blocks)

    def forget(self, doc_id: int) -> None:
        """Drop a document whatever its pins (a miss whose content was never written)."""
        d = self._docs.pop(doc_id)
        self.pool.free(d.blocks)
        self.used -= len(d.blocks)
        if d.pins == 0:
            self.unpinned -= len(d.blocks)

    def _make_room(self, need: int) -> None:
        room = min(self.budget - self.used, self.pool.free_blocks)
        if room >= need:
            return
        # least recently used first, skipping pinned entries; victims are
        # chosen before any is removed, so the walk stops as soon as enough
        # room is found (no pass over the whole cache per miss)
        victims, gain = [], 0
        for key, d in self._docs.items():
            if room + gain >= need:
                break
            if d.pins == 0:
                victims.append(key)
                gain += len(d.blocks)
        if room + gain < need:
            raise CacheFull(f"cannot free {need} blocks: everything left is pinned")
        for key in victims:
            d = self._docs.pop(key)
            self.pool.free(d.blocks)
            self.used -= len(d.blocks)
            self.unpinned -= len(d.blocks)
            self.evictions += 1

    def room_for_private(self, n: int) -> bool:
        """Whether n private blocks fit the budget after evicting every unpinned document."""
        evictable = self.unpinned
        return min(self.budget - self.used + evictable, self.pool.free_blocks + evictable) >= n

    def take_private(self, n: int) -> List[int]:
        """Blocks for private tokens, charged to the same budget (evicting if needed)."""
        self._make_room(n)
        self.used += n
        return self.pool.alloc(n)

    def give_back_private(self, blocks: Sequence[int]) -> None:
        self.pool.free(blocks)
        self.used -= len(blocks)


class PositionAwareCache(DocCache):
    """Entries keyed by (document, global offset): a copy is valid at one offset only (its keys carry RoPE at
    their global positions), so every new offset of a document is a miss and a new copy under the same
    budget and the same whole-entry LRU eviction."""

    def acquire_at(self, doc_id: int, offset: int, length: int, reserve: int = 0) -> Tuple[List[int], bool]:
        return self.acquire((doc_id, offset), length, reserve)

    def release_at(self, doc_id: int, offset: int) -> None:
        self.release((doc_id, offset))

    def copies(self, doc_id: int) -> int:
        """Cached copies of one document (one per offset it is held at)."""
        return sum(1 for k in self._docs if k[0] == doc_id)


@dataclass
class Segment:
    blocks: List[int]
    length: int
    pos0: int
    ctx: bool  # True: cached document written at local positions; False: private, at global positions


@dataclass
class RequestLayout:
    """A request's logical sequence: cached documents (in order), then private tokens."""

    segments: List[Segment] = field(default_factory=list)

    @property
    def length(self) -> int:
        return sum(s.length for s in self.segments)

    @property
    def num_tiles(self) -> int:
        return sum(blocks_for(s.length) for s in self.segments)


def layout_request(doc_blocks: Sequence[Tuple[List[int], int]], private_blocks: List[int],
                   private_len: int) -> RequestLayout:
    """Place documents consecutively from position 0, then the private tokens."""
    segs = []
    pos = 0
    for blocks, length in doc_blocks:
        segs.append(Segment(list(blocks), length, pos, True))
        pos += length
    segs.append(Segment(list(private_blocks), private_len, pos, False))
    return RequestLayout(segs)


def order_for_reuse(layouts: Sequence[RequestLayout]) -> List[RequestLayout]:
    """The same requests with each one's cached documents listed most shared first.

    A cached document is the same blocks in every request that reads it, so
    its first block names it.  Listing every request's documents by how many
    requests of the batch read them (then by that block) puts a shared
    document at about the same tile index everywhere: the split-K kernels
    then read it for all those requests at about the same time, and the
    copies after the first come from the cache hierarchy.  Each tile carries
    its own offset and the softmax does not depend on key order, so only the
    rounding order of the sums changes.  Private tokens stay after the
    documents, where the kernels expect them.
    """
    count: Dict[int, int] = {}
    for lay in layouts:
        for sg in lay.segments:
            if sg.ctx and sg.blocks:
                count[sg.blocks[0]] = count.get(sg.blocks[0], 0) + 1
    out = []
    for lay in layouts:
        docs = [sg for sg in lay.segments if sg.ctx and sg.blocks]
        rest = [sg for sg in lay.segments if not (sg.ctx and sg.blocks)]
        docs.sort(key=lambda sg: (-count[sg.blocks[0]], sg.blocks[0]))
        out.append(RequestLayout(docs + rest))
    return out


def flatten_layouts(layouts: Sequence[RequestLayout]) -> Dict[str, list]:
    """Segment arrays in the form lazy_build_tiles takes."""
    seg_start, seg_len, seg_pos0, seg_ctx, seg_bstart, blocks = [0], [], [], [], [0], []
    for lay in layouts:
        for s in lay.segments:
            seg_len.append(s.length)
            seg_pos0.append(s.pos0)
            seg_ctx.append(1 if s.ctx else 0)
            blocks.extend(s.blocks)
            seg_bstart.append(len(blocks))
        seg_start.append(len(seg_len))
    return {"seg_start": seg_start, "seg_len": seg_len, "seg_pos0": seg_pos0, "seg_is_ctx": seg_ctx,
            "seg_block_start": seg_bstart, "blocks": blocks}
