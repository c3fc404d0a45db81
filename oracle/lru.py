"""Hit/miss sequence of a least-recently-used cache of whole entries (oracle; test infrastructure only).

The LazyAttention notes (papernotes.org, "Background and motivation" and
"Main experiments": VRAM hit ratio under a KV budget, Zipf document
popularity) compare a position-agnostic cache, whose entry is a document,
with a position-aware one, whose entry is a document at one offset.  Both
evict whole entries, least recently used first, within a byte budget.  This
module is that rule written out as plainly as possible, to check the
library's host-side cache against it:

  * the cache is a Python list of (key, size), least recently used first;
  * requests are processed in order, and the entries a request has touched
    stay pinned until the request ends (all of a request's documents must be
    resident together);
  * an access to a cached key is a hit and moves the entry to the back;
  * a miss evicts from the front, skipping pinned entries, until the new
    entry fits, then appends it.

Also the static top-C limit of the notes' closed form: a cache that holds a
fixed set of keys and never evicts.
"""

from __future__ import annotations

from typing import Callable, Hashable, List, Sequence, Set, Tuple


def replay(requests: Sequence[Sequence[Tuple[Hashable, int]]], budget: int) -> List[bool]:
    """Hit (True) or miss (False) of every access, in trace order.

    ``requests[r]`` lists (key, size) accesses; ``budget`` bounds the sum of
    the cached sizes.  Raises if a request's pinned entries alone exceed it.
    """
    cache: List[Tuple[Hashable, int]] = []
    out: List[bool] = []
    for req in requests:
        pinned: Set[Hashable] = set()
        for key, size in req:
            idx = next((i for i, (k, _) in enumerate(cache) if k == key), None)
            if idx is not None:
                entry = cache.pop(idx)
                cache.append(entry)
                out.append(True)
            else:
                while sum(s for _, s in cache) + size > budget:
                    victim = next((i for i, (k, _) in enumerate(cache) if k not in pinned), None)
                    if victim is None:
                        raise RuntimeError("the request's own entries exceed the budget")
                    cache.pop(victim)
                cache.append((key, size))
                out.append(False)
            pinned.add(key)
    return out


def static_hits(accesses: Sequence[Hashable], resident: Callable[[Hashable], bool]) -> int:
    """Hits of a cache whose contents never change: the accesses whose key is resident."""
    return sum(1 for a in accesses if resident(a))
