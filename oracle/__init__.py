"""fp64 CPU oracle for deferred-position paged attention.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never calls it, and it shares no code, table or helper
with that path: it is written from the pages' description of what the method
computes.

What it computes.  The LazyAttention pages state that attention with a
position-agnostic cache and a deferred relative rotation is mathematically
identical to ordinary RoPE attention over keys rotated to their global
positions ("Equivalenza Matematica" on the gist.science summary; "Method:
overall framework" on the papernotes.org notes).  The oracle is therefore that
plain definition: it lays each request's documents out consecutively,
rotates every query and key eagerly at its *global* position and runs
textbook softmax attention in fp64.  It never sees blocks, tiles, offsets or a
cached rotation.

Modules
  rope       positional encodings: RoPE (half-split / interleaved), YaRN
             frequencies and temperature, ALiBi slopes
  attention  eager attention over a logical sequence (prefill and decode)
  brute      pure-Python scalar loops for tiny cases
  pack       the 64-bit (block id, offset, mask) tile word and the tile list
             a request implies
  zipf       position-agnostic vs position-aware hit-ratio closed form
  lru        hit/miss sequence of a whole-entry LRU cache under a budget
             (position-agnostic and position-aware keys alike)

Pins (tests/test_oracle_*.py) tie each function to something other than
itself; ``rope.yarn_inv_freq`` and ``attention`` are pinned through special
cases, library routines and brute force (see the tests).  No function here is
"parity unpinned".
"""

from . import attention, brute, lru, pack, rope, zipf  # noqa: F401
