"""64-bit tile metadata word and the tile list of a request (oracle; test infrastructure only).

The LazyAttention notes (papernotes.org, "Key designs: fused Triton kernel +
bit-packed metadata") pack (block id, offset, mask) of one KV tile into a
single 64-bit word that the decode kernel splits with register shifts.  The
pages give no field widths; the layout read here is

    bits 63..40  physical block id      (24 bits)
    bits 39..16  offset                 (24 bits)
    bits 15..0   valid-slot mask        (16 bits; bit s = slot s holds a token)

with one tile = one paged block of 16 token slots.

Meaning of the offset (per tile class):
  * context tiles (a cached document, written at document-local positions
    0..L-1): the document's start position Delta in the request under RoPE
    kinds -- the single relative rotation amount -- and the global position
    of the tile's slot 0 (Delta + 16 b) under ALiBi, whose deferral is a
    score-space bias (notes, "Generality");
  * private tiles (question / generated tokens written at their global
    positions): the global position of the tile's slot 0, for every kind.

Written with Python integers, straight from the layout above.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

BLOCK_BITS = 24
OFFSET_BITS = 24
MASK_BITS = 16
TILE = 16


def pack(block: int, offset: int, mask: int) -> int:
    if not (0 <= block < (1 << BLOCK_BITS)):
        raise ValueError("block id out of range")
    if not (0 <= offset < (1 << OFFSET_BITS)):
        raise ValueError("offset out of range")
    if not (0 < mask < (1 << MASK_BITS)):
        raise ValueError("mask out of range")
    return block * (1 << 40) + offset * (1 << 16) + mask


def unpack(word: int) -> Tuple[int, int, int]:
    block = word // (1 << 40)
    offset = (word // (1 << 16)) % (1 << OFFSET_BITS)
    mask = word % (1 << MASK_BITS)
    return block, offset, mask


def request_tiles(segments: Sequence[dict], kind: str) -> Tuple[List[int], int]:
    """Tile words of one request and how many of them are context tiles.

    Each segment is {"blocks": [...], "len": L, "pos0": p, "ctx": bool}: L tokens
    stored from slot 0 of blocks[0] onwards, whose first token sits at global
    position p.  Context segments (cached documents) come first.
    """
    words: List[int] = []
    n_ctx = 0
    seen_private = False
    for seg in segments:
        L, p0, ctx = seg["len"], seg["pos0"], seg["ctx"]
        if ctx and seen_private:
            raise ValueError("context segment after a private one")
        if not ctx:
            seen_private = True
        nblk = (L + TILE - 1) // TILE
        for b in range(nblk):
            valid = min(TILE, L - TILE * b)
            mask = (1 << valid) - 1
            if ctx and kind != "alibi":
                off = p0
            else:
                off = p0 + TILE * b
            words.append(pack(seg["blocks"][b], off, mask))
            if ctx:
                n_ctx += 1
    return words, n_ctx
