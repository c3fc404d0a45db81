"""ctypes binding of liblazyattn.so (argument marshalling only).

Every function here forwards to the C ABI declared in include/lazy_attn.h with
the same name minus the ``lazy_`` prefix.  Device buffers are torch tensors
(PyTorch supplies device memory and streams); host buffers are numpy arrays.
No arithmetic of the method happens in Python.  A non-OK status raises
``LazyError`` carrying ``lazy_last_error()``.  The library must be built
(``python -m position_agnostic_paged_amd.build``); loading fails loudly if it
is missing.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# LAZY_ATTN_LIB selects another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("LAZY_ATTN_LIB") or os.path.join(_HERE, "liblazyattn.so")

LAZY_OK, LAZY_ERR_ARG, LAZY_ERR_UNSUPPORTED, LAZY_ERR_WORKSPACE, LAZY_ERR_HIP = 0, -1, -2, -3, -4
LAZY_BF16, LAZY_FP32 = 0, 1
LAZY_ROPE_HALF, LAZY_ROPE_INTERLEAVED, LAZY_ALIBI = 0, 1, 2
LAZY_FLAG_PREROTATED = 1
LAZY_FLAG_DOC_PAIRS = 2
BLOCK_SIZE = 16

KIND_BY_NAME = {"rope_half": LAZY_ROPE_HALF, "rope_interleaved": LAZY_ROPE_INTERLEAVED, "alibi": LAZY_ALIBI}

EXPORTED = [
    "lazy_rope_freqs", "lazy_softmax_scale", "lazy_rope_table", "lazy_alibi_slopes", "lazy_pack_tiles",
    "lazy_unpack_tiles",
    "lazy_build_tiles", "lazy_build_tiles_paired", "lazy_kv_write", "lazy_attn_workspace_size", "lazy_attn_prefill", "lazy_attn_decode",
    "lazy_attn_decode_noalloc", "lazy_build_shared_plan", "lazy_attn_decode_shared_workspace_size",
    "lazy_attn_decode_shared", "lazy_debug_unpack", "lazy_last_error",
]


class LazyError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"lazy_attn status {status}: {msg}")
        self.status = status


class Geom(C.Structure):
    _fields_ = [("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("block_size", C.c_int32), ("dtype", C.c_int32)]


class PosDescC(C.Structure):
    _fields_ = [("kind", C.c_int32), ("flags", C.c_uint32), ("max_pos", C.c_int32), ("softmax_scale", C.c_float),
                ("cos_sin", C.c_void_p), ("inv_freq", C.c_void_p), ("alibi_slopes", C.c_void_p)]


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m position_agnostic_paged_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, I32, I64 = C.c_void_p, C.c_int32, C.c_int64
        sig = {
            "lazy_rope_freqs": [I32, C.c_double, C.c_double, I32, C.c_double, C.c_double, P, P],
            "lazy_softmax_scale": [I32, C.c_double, P],
            "lazy_rope_table": [I32, P, I32, P],
            "lazy_alibi_slopes": [I32, P],
            "lazy_pack_tiles": [P, P, P, I64, P],
            "lazy_unpack_tiles": [P, I64, P, P, P],
            "lazy_build_tiles": [I32, I32, P, P, P, P, P, P, I64, I32, P, I64, P, P],
            "lazy_build_tiles_paired": [I32, I32, P, P, P, P, P, P, I64, I32, P, I64, P, P],
            "lazy_kv_write": [P, P, P, P, I64, P, P, P, P, P, I32, P],
            "lazy_attn_prefill": [P, P, P, P, I64, P, P, P, P, P, P, I32, I32, I32, I64, P, P, C.c_size_t, P],
            "lazy_attn_decode": [P, P, P, P, I64, P, P, P, P, P, I32, I32, I64, P, P, C.c_size_t, P],
            "lazy_attn_decode_noalloc": [P, P, P, P, I64, P, P, P, P, P, I32, I32, I64, P, P],
            "lazy_debug_unpack": [P, I64, P, P, P, P],
            "lazy_build_shared_plan": [P, I32, I32, P, P, P, P, P, P, I64, I32, I32, P, I64, P, P, P, I64, P, P,
                                       I32, P, I64, P, P, I64, P],
            "lazy_attn_decode_shared": [P, P, P, P, I64, P, P, P, I32, I64, P, P, P, P, P, P, I32, I32, I32, I32, P,
                                        P, I32, P, P, C.c_size_t, P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = I32
        L.lazy_attn_workspace_size.argtypes = [P, I32, I32, I32, I64, I32]
        L.lazy_attn_workspace_size.restype = C.c_size_t
        L.lazy_attn_decode_shared_workspace_size.argtypes = [P, I32, I32, I64, I32]
        L.lazy_attn_decode_shared_workspace_size.restype = C.c_size_t
        L.lazy_last_error.argtypes = []
        L.lazy_last_error.restype = C.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().lazy_last_error().decode()


def _check(st: int):
    if st != LAZY_OK:
        raise LazyError(st, last_error())


def _np_ptr(a: Optional[np.ndarray]):
    # the address as a plain int (every pointer parameter is declared c_void_p); the int keeps no
    # reference, so every caller passes an array it holds in a local until the call returns
    return None if a is None else a.ctypes.data


def _dev(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    """The HIP stream handle of a torch stream (None: the current stream of the current device)."""
    if stream is None:
        import torch

        # the raw handle of torch's current stream, without building a Stream object per call
        return torch._C._cuda_getCurrentRawStream(torch._C._cuda_getDevice())
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def make_geom(num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: str) -> Geom:
    return Geom(num_q_heads, num_kv_heads, head_dim, BLOCK_SIZE, LAZY_BF16 if dtype == "bf16" else LAZY_FP32)


# ------------------------------------------------------------------ host calls

def rope_freqs(head_dim: int, base: float, yarn_factor: float = 1.0, yarn_orig_ctx: int = 0,
               beta_fast: float = 32.0, beta_slow: float = 1.0):
    out = np.zeros(head_dim // 2, np.float64)
    gain = C.c_double(0.0)
    _check(lib().lazy_rope_freqs(head_dim, base, yarn_factor, yarn_orig_ctx, beta_fast, beta_slow, _np_ptr(out),
                                 C.cast(C.pointer(gain), C.c_void_p)))
    return out, gain.value


def softmax_scale(head_dim: int, yarn_factor: float = 1.0) -> float:
    out = C.c_float(0.0)
    _check(lib().lazy_softmax_scale(head_dim, yarn_factor, C.cast(C.pointer(out), C.c_void_p)))
    return out.value


def rope_table(head_dim: int, inv_freq: np.ndarray, max_pos: int) -> np.ndarray:
    inv = np.ascontiguousarray(inv_freq, np.float64)
    out = np.empty((max_pos, head_dim), np.float32)
    _check(lib().lazy_rope_table(head_dim, _np_ptr(inv), max_pos, _np_ptr(out)))
    return out


def alibi_slopes(num_heads: int) -> np.ndarray:
    out = np.empty(num_heads, np.float32)
    _check(lib().lazy_alibi_slopes(num_heads, _np_ptr(out)))
    return out


def pack_tiles(block_ids, offsets, masks) -> np.ndarray:
    b = np.ascontiguousarray(block_ids, np.int64)
    o = np.ascontiguousarray(offsets, np.int64)
    m = np.ascontiguousarray(masks, np.uint32)
    out = np.empty(b.shape[0], np.uint64)
    _check(lib().lazy_pack_tiles(_np_ptr(b), _np_ptr(o), _np_ptr(m), b.shape[0], _np_ptr(out)))
    return out


def unpack_tiles(words):
    w = np.ascontiguousarray(words, np.uint64)
    b = np.empty(w.shape[0], np.int64)
    o = np.empty(w.shape[0], np.int64)
    m = np.empty(w.shape[0], np.uint32)
    _check(lib().lazy_unpack_tiles(_np_ptr(w), w.shape[0], _np_ptr(b), _np_ptr(o), _np_ptr(m)))
    return b, o, m


def build_tiles(kind: int, seg_start, seg_len, seg_pos0, seg_is_ctx, seg_block_start, blocks, num_blocks: int,
                tiles_cap: Optional[int] = None, max_pos: int = 0, paired: bool = False):
    """Tile words, tile_start [R+1], ctx_tiles [R] of every request (host arrays); max_pos > 0 checks every
    rotary document offset against the cos/sin table's rows; paired: lazy_build_tiles_paired (documents
    closed to whole tile pairs; tiles_cap grows by one per context segment)."""
    ss = np.ascontiguousarray(seg_start, np.int32)
    sl = np.ascontiguousarray(seg_len, np.int32)
    sp = np.ascontiguousarray(seg_pos0, np.int64)
    sc = np.ascontiguousarray(seg_is_ctx, np.uint8)
    sb = np.ascontiguousarray(seg_block_start, np.int32)
    bl = np.ascontiguousarray(blocks, np.int32)
    R = ss.shape[0] - 1
    cap = int(tiles_cap if tiles_cap is not None else max(1, bl.shape[0]))
    if paired:
        cap += int(np.count_nonzero(sc))
    tiles = np.empty(cap, np.uint64)
    tstart = np.empty(R + 1, np.int32)
    nctx = np.empty(max(R, 1), np.int32)
    fn = lib().lazy_build_tiles_paired if paired else lib().lazy_build_tiles
    _check(fn(kind, R, _np_ptr(ss), _np_ptr(sl), _np_ptr(sp), _np_ptr(sc), _np_ptr(sb), _np_ptr(bl), num_blocks,
              max_pos, _np_ptr(tiles), cap, _np_ptr(tstart), _np_ptr(nctx)))
    return tiles[: tstart[R]].copy(), tstart, nctx[:R].copy()


# ---------------------------------------------------------------- device calls

def kv_write(geom: Geom, pos: PosDescC, k_cache, v_cache, num_blocks: int, k, v, q_inout, positions, slot_mapping,
             stream=None):
    n = int(positions.shape[0])
    _check(lib().lazy_kv_write(C.byref(geom), C.byref(pos), _dev(k_cache), _dev(v_cache), num_blocks, _dev(k),
                               _dev(v), _dev(q_inout), _dev(positions), _dev(slot_mapping), n, _stream(stream)))


def workspace_size(geom: Geom, num_reqs: int, max_q_len: int, max_tiles: int, total_tiles: int,
                   is_prefill: bool) -> int:
    return int(lib().lazy_attn_workspace_size(C.byref(geom), num_reqs, max_q_len, max_tiles, total_tiles,
                                              int(is_prefill)))


def attn_prefill(geom: Geom, pos: PosDescC, k_cache, v_cache, num_blocks: int, tiles, tile_start, ctx_tiles, q,
                 q_start, q_pos0, num_reqs: int, max_q_len: int, max_tiles: int, total_tiles: int, out, workspace,
                 stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().lazy_attn_prefill(C.byref(geom), C.byref(pos), _dev(k_cache), _dev(v_cache), num_blocks,
                                   _dev(tiles), _dev(tile_start), _dev(ctx_tiles), _dev(q), _dev(q_start),
                                   _dev(q_pos0), num_reqs, max_q_len, max_tiles, total_tiles, _dev(out),
                                   _dev(workspace), ws_bytes, _stream(stream)))


def attn_decode(geom: Geom, pos: PosDescC, k_cache, v_cache, num_blocks: int, tiles, tile_start, ctx_tiles, q, q_pos,
                num_reqs: int, max_tiles: int, total_tiles: int, out, workspace, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().lazy_attn_decode(C.byref(geom), C.byref(pos), _dev(k_cache), _dev(v_cache), num_blocks, _dev(tiles),
                                  _dev(tile_start), _dev(ctx_tiles), _dev(q), _dev(q_pos), num_reqs, max_tiles,
                                  total_tiles, _dev(out), _dev(workspace), ws_bytes, _stream(stream)))


def build_shared_plan(geom: Geom, kind: int, seg_start, seg_len, seg_pos0, seg_is_ctx, seg_block_start, blocks,
                      num_blocks: int, max_pos: int = 0, min_readers: int = 2) -> dict:
    """Host plan of a document-major decode (numpy arrays, trimmed to their used lengths)."""
    ss = np.ascontiguousarray(seg_start, np.int32)
    sl = np.ascontiguousarray(seg_len, np.int32)
    sp = np.ascontiguousarray(seg_pos0, np.int64)
    sc = np.ascontiguousarray(seg_is_ctx, np.uint8)
    sb = np.ascontiguousarray(seg_block_start, np.int32)
    bl = np.ascontiguousarray(blocks if len(blocks) else [0], np.int32)
    R = ss.shape[0] - 1
    nseg = int(ss[-1])
    cap_tiles = max(1, int(sum((int(n) + 15) // 16 for n in sl)))
    cap_docs = max(1, int(sl.shape[0]))  # every segment may become an item (min_readers 1: private ones too)
    group = geom.num_q_heads // geom.num_kv_heads
    # work items: per item, (chunks <= tiles/32 + 1) x (row blocks <= readers x G / 16 + 1)
    per_doc = {}  # item -> [tokens, readers]
    for i in range(sl.shape[0]):
        if sl[i] > 0:
            k = (int(bl[sb[i]]), int(sl[i])) if sc[i] else ("private", i)
            per_doc.setdefault(k, [int(sl[i]), 0])[1] += 1
    cap_work = 1 + sum(((n + 15) // 16 // 32 + 1) * ((r * group + 15) // 16 + 4) for n, r in per_doc.values())
    out = {"tiles": np.empty(cap_tiles, np.uint64), "tile_start": np.empty(R + 1, np.int32),
           "ctx_tiles": np.empty(max(R, 1), np.int32), "doc_tiles": np.empty(cap_tiles, np.uint64),
           "doc_tile_start": np.empty(cap_docs + 1, np.int32), "read_start": np.empty(cap_docs + 1, np.int32),
           "reads": np.empty(cap_docs, np.uint64), "req_reads": np.empty(max(R, 1), np.int32),
           "work": np.empty(4 * cap_work, np.int32)}
    counts = np.zeros(8, np.int64)
    del nseg
    _check(lib().lazy_build_shared_plan(
        C.byref(geom), kind, R, _np_ptr(ss), _np_ptr(sl), _np_ptr(sp), _np_ptr(sc), _np_ptr(sb), _np_ptr(bl),
        num_blocks, max_pos, min_readers, _np_ptr(out["tiles"]), cap_tiles, _np_ptr(out["tile_start"]),
        _np_ptr(out["ctx_tiles"]), _np_ptr(out["doc_tiles"]), cap_tiles, _np_ptr(out["doc_tile_start"]),
        _np_ptr(out["read_start"]), cap_docs, _np_ptr(out["reads"]), cap_docs, _np_ptr(out["req_reads"]),
        _np_ptr(out["work"]), cap_work, _np_ptr(counts)))
    nd, nr, nw, max_reads, nt, max_tiles, ndt, rb = (int(x) for x in counts)
    return {"tiles": out["tiles"][:nt].copy(), "tile_start": out["tile_start"], "ctx_tiles": out["ctx_tiles"][:R].copy(),
            "doc_tiles": out["doc_tiles"][:ndt].copy(), "doc_tile_start": out["doc_tile_start"][: nd + 1].copy(),
            "read_start": out["read_start"][: nd + 1].copy(), "reads": out["reads"][:nr].copy(),
            "req_reads": out["req_reads"][:R].copy(), "work": out["work"][: 4 * nw].copy(), "num_docs": nd,
            "num_reads": nr, "num_work": nw, "max_req_reads": max_reads, "total_tiles": nt, "max_tiles": max_tiles,
            "row_blocks": rb}


def decode_shared_workspace_size(geom: Geom, num_reqs: int, max_tiles: int, total_tiles: int,
                                 max_req_reads: int) -> int:
    return int(lib().lazy_attn_decode_shared_workspace_size(C.byref(geom), num_reqs, max_tiles, total_tiles,
                                                            max_req_reads))


def attn_decode_shared(geom: Geom, pos: PosDescC, k_cache, v_cache, num_blocks: int, tiles, tile_start, ctx_tiles,
                       max_tiles: int, total_tiles: int, doc_tiles, doc_tile_start, read_start, reads, req_reads, work,
                       num_docs: int, num_work: int, max_req_reads: int, row_blocks: int, q, q_pos, num_reqs: int,
                       out, workspace, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().lazy_attn_decode_shared(
        C.byref(geom), C.byref(pos), _dev(k_cache), _dev(v_cache), num_blocks, _dev(tiles), _dev(tile_start),
        _dev(ctx_tiles), max_tiles, total_tiles, _dev(doc_tiles), _dev(doc_tile_start), _dev(read_start), _dev(reads),
        _dev(req_reads), _dev(work), num_docs, num_work, max_req_reads, row_blocks, _dev(q), _dev(q_pos), num_reqs,
        _dev(out), _dev(workspace), ws_bytes, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20  # LAZY_NOALLOC_SCRATCH_BYTES


def attn_decode_noalloc(geom: Geom, pos: PosDescC, k_cache, v_cache, num_blocks: int, tiles, tile_start, ctx_tiles, q,
                        q_pos, num_reqs: int, max_tiles: int, total_tiles: int, out, stream=None):
    """lazy_attn_decode without a workspace: split partials in the library's static device scratch."""
    _check(lib().lazy_attn_decode_noalloc(C.byref(geom), C.byref(pos), _dev(k_cache), _dev(v_cache), num_blocks,
                                          _dev(tiles), _dev(tile_start), _dev(ctx_tiles), _dev(q), _dev(q_pos),
                                          num_reqs, max_tiles, total_tiles, _dev(out), _stream(stream)))


def debug_unpack(words, block, offset, mask, stream=None):
    _check(lib().lazy_debug_unpack(_dev(words), int(words.numel()), _dev(block), _dev(offset), _dev(mask),
                                   _stream(stream)))


def exported_symbols() -> Sequence[str]:
    L = lib()
    return [s for s in EXPORTED if hasattr(L, s)]
