"""Device state and call sequencing for the deferred-position paged attention path.

``PosDesc`` builds the positional metadata once (host C calls for the
frequencies / cos-sin table / ALiBi slopes, then a copy to the device).
``Engine`` owns the paged K/V pools and runs the three device calls of the
library: kv-write (documents at local positions, private tokens at global
positions), prefill and decode, with tile tables built by the library's host
packer.  PyTorch provides device memory, copies and the stream; every step of
the computation runs in liblazyattn.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import lazy_attn as L
from .paging import (BlockPool, DocCache, PositionAwareCache, RequestLayout, Segment, blocks_for, flatten_layouts,
                     order_for_reuse)

TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}


class PosDesc:
    """Positional variant: kind, softmax scale and device-resident coefficients."""

    def __init__(self, kind: str, head_dim: int, num_q_heads: int, device, base: float = 1e4,
                 yarn_factor: float = 1.0, yarn_orig_ctx: int = 0, beta_fast: float = 32.0, beta_slow: float = 1.0,
                 max_pos: int = 0, on_the_fly: bool = False, prerotated: bool = False):
        self.kind = kind
        self.kind_id = L.KIND_BY_NAME[kind]
        self.head_dim = head_dim
        self.table = self.inv_freq = self.slopes = None
        if kind == "alibi":
            self.slopes = torch.from_numpy(L.alibi_slopes(num_q_heads)).to(device)
            max_pos = max(max_pos, 1)
        else:
            inv, _ = L.rope_freqs(head_dim, base, yarn_factor, yarn_orig_ctx, beta_fast, beta_slow)
            self.inv_freq = torch.from_numpy(inv).to(device)
            if not on_the_fly:
                if max_pos < 1:
                    raise ValueError("max_pos must cover every rotation position")
                self.table = torch.from_numpy(L.rope_table(head_dim, inv, max_pos)).to(device)
        self.max_pos = max_pos
        self.softmax_scale = L.softmax_scale(head_dim, yarn_factor if kind != "alibi" else 1.0)
        self.c = L.PosDescC(self.kind_id, L.LAZY_FLAG_PREROTATED if prerotated else 0, max_pos,
                            self.softmax_scale, L._dev(self.table), L._dev(self.inv_freq), L._dev(self.slopes))
        self._variants = {}

    @property
    def table_rows(self) -> int:
        """Rows of the cos/sin table the kernels index by position (0: no table)."""
        return self.max_pos if self.table is not None else 0

    def check_positions(self, positions: np.ndarray) -> None:
        """Rotation positions must address the table (or the in-kernel sincos range)."""
        if self.kind == "alibi" or positions.size == 0:
            return
        lo, hi = int(positions.min()), int(positions.max())
        limit = self.table_rows if self.table is not None else (1 << 24)
        if lo < 0 or hi >= limit:
            raise ValueError(f"rotation positions [{lo}, {hi}] outside [0, {limit})")

    def with_flags(self, prerotated: bool, doc_pairs: bool = False) -> L.PosDescC:
        """The descriptor with the given flags (one copy per combination, kept): prerotated = the control
        on keys stored at global positions; doc_pairs = the prefill's tile lists keep each tile pair within
        one document (lazy_build_tiles_paired), so it rotates the query per document."""
        key = (bool(prerotated), bool(doc_pairs))
        c = self._variants.get(key)
        if c is None:
            c = L.PosDescC.from_buffer_copy(self.c)
            c.flags = (L.LAZY_FLAG_PREROTATED if prerotated else 0) | (L.LAZY_FLAG_DOC_PAIRS if doc_pairs else 0)
            self._variants[key] = c
        return c


class StepUploads:
    """Host metadata of one step (positions, slot ids, tile words, row starts)
    packed into a pinned buffer and moved to the device with one copy.

    ``begin()`` starts a step, ``add(array)`` stages an array and returns its
    index, ``commit()`` issues the single host-to-device copy on the current
    stream and returns device views in ``add`` order (callbacks registered with
    ``on_commit`` receive them too).  Two pinned buffers alternate, and a
    buffer is refilled only after its previous copy has executed; the device
    buffer is reused in stream order (the next copy runs after the kernels that
    read the previous one)."""

    ALIGN = 256

    def __init__(self, device, capacity: int = 8 << 20):
        self.device = torch.device(device)
        self.cap = capacity
        self.host = [torch.empty(capacity, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
        self.host_np = [h.numpy() for h in self.host]
        self.dev = torch.empty(capacity, dtype=torch.uint8, device=self.device)
        # the buffer seen as each staged dtype, so a staged array's view is one slice (capacity and every
        # offset are multiples of 8 bytes)
        self.dev_as = {dt: self.dev.view(tdt) for dt, tdt in TORCH_INT.items()}
        self.done: List[Optional[torch.cuda.Event]] = [None, None]
        self.cur = 1
        self.items: List[Tuple[int, np.dtype, Tuple[int, ...]]] = []
        self.callbacks = []
        self.off = 0

    def begin(self) -> None:
        self.cur ^= 1
        if self.done[self.cur] is not None:
            self.done[self.cur].synchronize()
        self.items, self.callbacks, self.off = [], [], 0

    def add(self, arr) -> int:
        a = np.ascontiguousarray(arr)
        if a.dtype == np.uint64:
            a = a.view(np.int64)
        off = (self.off + self.ALIGN - 1) // self.ALIGN * self.ALIGN
        if off + a.nbytes > self.cap:
            raise ValueError(f"step metadata exceeds {self.cap} bytes")
        self.host_np[self.cur][off: off + a.nbytes] = a.reshape(-1).view(np.uint8)
        self.items.append((off, np.dtype(a.dtype), a.shape))
        self.off = off + a.nbytes
        return len(self.items) - 1

    def on_commit(self, fn) -> None:
        self.callbacks.append(fn)

    def commit(self) -> List[torch.Tensor]:
        n = self.off
        if n:
            self.dev[:n].copy_(self.host[self.cur][:n], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record()
        self.done[self.cur] = ev
        views = []
        for off, dt, shape in self.items:
            first = off // dt.itemsize
            if len(shape) == 1:
                views.append(self.dev_as[dt][first: first + shape[0]])
            else:
                views.append(self.dev_as[dt][first: first + int(np.prod(shape))].view(shape))
        for fn in self.callbacks:
            fn(views)
        return views


TORCH_INT = {np.dtype(np.int32): torch.int32, np.dtype(np.int64): torch.int64, np.dtype(np.uint8): torch.uint8}


class TileTable:
    """Device copy of the packed tile words of a batch of requests (uploaded on
    its own, or staged into a step's ``StepUploads``)."""

    def __init__(self, layouts: Sequence[RequestLayout], kind_id: int, num_blocks: int, device,
                 uploads: Optional[StepUploads] = None, max_pos: int = 0, paired: bool = False):
        f = flatten_layouts(layouts)
        cap = sum(blocks_for(n) for n in f["seg_len"]) or 1
        tiles, tstart, nctx = L.build_tiles(kind_id, f["seg_start"], f["seg_len"], f["seg_pos0"], f["seg_is_ctx"],
                                            f["seg_block_start"], f["blocks"] or [0], num_blocks, cap, max_pos,
                                            paired)
        self.paired = paired
        self.host_tiles, self.host_start, self.host_ctx = tiles, tstart, nctx
        self.num_reqs = len(layouts)
        self.max_tiles = int(np.max(np.diff(tstart))) if len(layouts) else 0
        self.total_tiles = int(tstart[-1]) if len(layouts) else 0
        arrays = (tiles.view(np.int64) if tiles.size else np.zeros(1, np.int64), tstart,
                  nctx if nctx.size else np.zeros(1, np.int32))
        if uploads is None:
            self.tiles, self.tile_start, self.ctx_tiles = (torch.from_numpy(a).to(device) for a in arrays)
        else:
            ids = [uploads.add(a) for a in arrays]
            uploads.on_commit(lambda views: self._bind(views, ids))

    def _bind(self, views, ids) -> None:
        self.tiles, self.tile_start, self.ctx_tiles = (views[i] for i in ids)


class SharedPlan:
    """Device copy of a document-major decode plan (lazy_build_shared_plan): each request's own tiles, every
    shared document's tiles and reads, and the document pass's work items."""

    DEVICE = ("tiles", "tile_start", "ctx_tiles", "doc_tiles", "doc_tile_start", "read_start", "reads", "req_reads",
              "work")

    def __init__(self, layouts: Sequence[RequestLayout], engine: "Engine", min_readers: int = 1):
        f = flatten_layouts(layouts)
        h = L.build_shared_plan(engine.geom, engine.pos.kind_id, f["seg_start"], f["seg_len"], f["seg_pos0"],
                                f["seg_is_ctx"], f["seg_block_start"], f["blocks"], engine.num_blocks,
                                engine.pos.table_rows, min_readers)
        self.host = h
        self.ws_bytes = None  # the decode's workspace bytes, asked for once
        self.num_reqs = len(layouts)
        for k in ("num_docs", "num_reads", "num_work", "max_req_reads", "total_tiles", "max_tiles", "row_blocks"):
            setattr(self, k, int(h[k]))
        for k in self.DEVICE:
            a = h[k]
            if a.dtype == np.uint64:
                a = a.view(np.int64)
            if a.size == 0:
                a = np.zeros(2, a.dtype)
            setattr(self, k, torch.from_numpy(np.ascontiguousarray(a)).to(engine.device))


class Engine:
    def __init__(self, num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: str, pos: PosDesc,
                 num_blocks: int, device="cuda", budget_blocks: Optional[int] = None, position_aware: bool = False):
        self.geom = L.make_geom(num_q_heads, num_kv_heads, head_dim, dtype)
        self.hq, self.hkv, self.dh, self.dtype = num_q_heads, num_kv_heads, head_dim, dtype
        self.tdtype = TORCH_DTYPE[dtype]
        self.pos = pos
        self.device = torch.device(device)
        self.num_blocks = num_blocks
        self.k_cache = torch.empty((num_blocks, num_kv_heads, 16, head_dim), dtype=self.tdtype, device=self.device)
        self.v_cache = torch.empty((num_blocks, num_kv_heads, head_dim, 16), dtype=self.tdtype, device=self.device)
        self.pool = BlockPool(num_blocks)
        # position_aware: the design the pages compare against, one copy per (document, offset)
        self.docs = (PositionAwareCache if position_aware else DocCache)(self.pool, budget_blocks)
        self._ws: Optional[torch.Tensor] = None

    # ------------------------------------------------------------- writing
    def kv_write(self, k: torch.Tensor, v: torch.Tensor, q: Optional[torch.Tensor], positions: torch.Tensor,
                 slots: torch.Tensor, pos: Optional[L.PosDescC] = None, stream=None) -> None:
        L.kv_write(self.geom, self.pos.c if pos is None else pos, self.k_cache, self.v_cache, self.num_blocks, k, v, q,
                   positions, slots, stream)

    def check_write(self, positions: np.ndarray, slots: np.ndarray) -> None:
        """Host-side validation of a kv-write's positions and slots (the library sees them only on the
        device): every position inside the rotation range, every slot inside the pool."""
        positions = np.asarray(positions)
        slots = np.asarray(slots)
        if positions.shape != slots.shape:
            raise ValueError("positions and slots differ in length")
        self.pos.check_positions(positions)
        if slots.size and int(slots.max()) >= self.num_blocks * 16:
            raise ValueError(f"slot {int(slots.max())} outside the pool of {self.num_blocks} blocks")

    def slots_for(self, blocks: Sequence[int], length: int, first: int = 0) -> np.ndarray:
        """Slot ids of tokens first .. first+length-1 of a segment stored in ``blocks``."""
        idx = np.arange(first, first + length)
        b = np.asarray(blocks, np.int64)[idx // 16]
        return b * 16 + idx % 16

    def write_segment(self, blocks: Sequence[int], k: torch.Tensor, v: torch.Tensor, pos0: int,
                      q: Optional[torch.Tensor] = None, first: int = 0, stream=None) -> None:
        """Write tokens first.. of a segment; their rotation positions are pos0 + first + i.

        For a cached document pos0 = 0 (local positions: the position-agnostic
        copy); for private tokens pos0 is the segment's global start."""
        n = k.shape[0]
        if n == 0:
            return
        pos_h = np.arange(pos0 + first, pos0 + first + n, dtype=np.int32)
        slots_h = self.slots_for(blocks, n, first)
        self.check_write(pos_h, slots_h)
        positions = torch.from_numpy(pos_h).to(self.device)
        slots = torch.from_numpy(slots_h).to(self.device)
        self.kv_write(k, v, q, positions, slots, stream=stream)

    def cache_doc(self, doc_id: int, length: int, content_fn, reserve: int = 0) -> Tuple[List[int], bool]:
        """Pin a document, writing its position-agnostic copy on a miss.  content_fn() -> (k, v) device tensors."""
        blocks, hit = self.docs.acquire(doc_id, length, reserve)
        if not hit:
            k, v = content_fn()
            self.write_segment(blocks, k, v, 0)
        return blocks, hit

    def cache_doc_at(self, doc_id: int, offset: int, length: int, content_fn, reserve: int = 0) -> Tuple[List[int], bool]:
        """Position-aware cache: pin the copy of a document placed at one global offset, writing it on a miss
        with RoPE at its global positions offset .. offset+L-1 (the eager re-encode a position-aware cache
        needs for every new offset).  Attention over such copies runs with LAZY_FLAG_PREROTATED."""
        if not isinstance(self.docs, PositionAwareCache):
            raise ValueError("cache_doc_at needs an engine built with position_aware=True")
        blocks, hit = self.docs.acquire_at(doc_id, offset, length, reserve)
        if not hit:
            k, v = content_fn()
            self.write_segment(blocks, k, v, offset)
        return blocks, hit

    def process_documents(self, items: Sequence[Tuple[int, torch.Tensor, torch.Tensor, torch.Tensor]],
                          out: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, List[List[int]]]:
        """The pass that runs on a document miss: write each document's
        position-agnostic cache entry and compute its own (block-diagonal,
        causal) attention, both at local positions 0..L-1.

        ``items`` = [(doc_id, k [L][Hkv][dh], v [L][Hkv][dh], q [L][Hq][dh])]
        of documents not yet cached.  One kv-write stores every document's
        K/V at its local positions (the copy later requests reuse at any
        offset) and rotates the queries in place; one prefill then treats
        each document as a request with no cached context whose own tokens
        are its causal suffix starting at position 0 -- for a document at
        offset 0 local and global positions coincide (LazyAttention notes,
        "Method: overall framework": a document is encoded once, on its
        first use, and reused position-agnostically afterwards).  ``q`` is
        overwritten with the rotated queries.  Returns the outputs
        ([sum L][Hq][dh], documents in order) and each document's blocks;
        the documents stay pinned until released."""
        if not items:
            raise ValueError("process_documents needs at least one document")
        ids = [int(it[0]) for it in items]
        lens = [int(it[1].shape[0]) for it in items]
        for (doc_id, k, v, q), n in zip(items, lens):
            if n < 1 or v.shape[0] != n or q.shape[0] != n:
                raise ValueError(f"document {doc_id}: k, v and q must have the same positive length")
            if doc_id in self.docs:
                raise ValueError(f"document {doc_id} is already cached: it has no miss to process")
        if len(set(ids)) != len(ids):
            raise ValueError("process_documents: a document appears twice")
        blocks_all, layouts, pos, slots = [], [], [], []
        try:
            for doc_id, n in zip(ids, lens):
                blocks, _ = self.docs.acquire(doc_id, n)
                blocks_all.append(blocks)
                layouts.append(RequestLayout([Segment(blocks, n, 0, False)]))
                pos.append(np.arange(n, dtype=np.int32))
                slots.append(self.slots_for(blocks, n))
            self.check_write(np.concatenate(pos), np.concatenate(slots))
            K = torch.cat([it[1] for it in items]).contiguous()
            V = torch.cat([it[2] for it in items]).contiguous()
            Q = torch.cat([it[3] for it in items]).contiguous()
            self.kv_write(K, V, Q, torch.from_numpy(np.concatenate(pos)).to(self.device),
                          torch.from_numpy(np.concatenate(slots)).to(self.device), stream=stream)
            tt = self.tile_table(layouts)
            q_start = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device=self.device)
            q_pos0 = torch.zeros(len(items), dtype=torch.int32, device=self.device)
            o = self.prefill(tt, Q, q_start, q_pos0, max(lens), out=out, stream=stream)
        except Exception:
            # nothing half-written stays in the cache
            for doc_id in ids[: len(blocks_all)]:
                self.docs.forget(doc_id)
            raise
        # the rotated queries go back to the callers' tensors
        off = 0
        for (_, _, _, q), n in zip(items, lens):
            q.copy_(Q[off: off + n])
            off += n
        return o, blocks_all

    # ----------------------------------------------------------- attention
    def _workspace(self, nbytes: int) -> Optional[torch.Tensor]:
        if nbytes == 0:
            return None
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self._ws

    # list each request's cached documents most shared first (paging.order_for_reuse)
    order_for_reuse = True

    def tile_table(self, layouts: Sequence[RequestLayout], uploads: Optional[StepUploads] = None,
                   paired: bool = False) -> TileTable:
        """Tile lists of a batch; paired (prefill): every document closed to whole tile pairs, so the prefill
        rotates the query once per document instead of every K pair."""
        if self.order_for_reuse:
            layouts = order_for_reuse(layouts)
        return TileTable(layouts, self.pos.kind_id, self.num_blocks, self.device, uploads, self.pos.table_rows,
                         paired)

    # prefill tile lists closed to whole pairs per document (the query rotated per document: on MI355X the
    # 70B-shape prefill call measured against the K-rotating kernel; see the prefill notes)
    prefill_pairs = True

    def prefill(self, tt: TileTable, q: torch.Tensor, q_start: torch.Tensor, q_pos0: torch.Tensor, max_q_len: int,
                out: Optional[torch.Tensor] = None, pos: Optional[L.PosDescC] = None, stream=None) -> torch.Tensor:
        if out is None:
            out = torch.empty_like(q)
        ws = self._workspace(L.workspace_size(self.geom, tt.num_reqs, max_q_len, tt.max_tiles, tt.total_tiles, True))
        if pos is None:
            pos = self.pos.with_flags(False, tt.paired)
        L.attn_prefill(self.geom, pos, self.k_cache, self.v_cache, self.num_blocks,
                       tt.tiles, tt.tile_start, tt.ctx_tiles, q, q_start, q_pos0, tt.num_reqs, max_q_len, tt.max_tiles,
                       tt.total_tiles, out, ws, stream)
        return out

    @property
    def doc_major_pays(self) -> bool:
        """Whether the document-major decode is the faster one for this geometry: with a query group of up to
        16 heads a wave's row blocks hold several reads of a shared document, so its tiles are read once for
        all of them.  A larger group (Falcon's 71 heads per KV head) fills the rows with one read each, the
        pass then shares little and adds partials (measured on MI355X: 128 x 16K MQA decode over shared
        documents 0.148 ms per request vs 0.203 ms document-major; 48 x 8K-66K GQA-8 decode 0.81 vs 0.26
        ms)."""
        return self.hq // self.hkv <= 16

    def shared_plan(self, layouts: Sequence[RequestLayout], min_readers: int = 1) -> SharedPlan:
        """Plan of a document-major decode: documents read by >= min_readers segments of the batch go through
        the document pass, the rest through the requests' own tile lists.  By default (min_readers 1) every
        cached document goes through the pass (its copies stream whole tile pairs into LDS with the streaming
        hint), and so does each request's private tail, as one more item read once at Delta 0; the split-K
        pass then has no tiles and is not launched.  On MI355X the mixed 70B step's decode call measured
        0.277 ms with documents read once left to the split-K pass, 0.257 ms with them in the pass and the
        private tokens split-K, 0.237 ms with the private tokens in the pass too."""
        return SharedPlan(layouts, self, min_readers)

    def decode_shared(self, plan: SharedPlan, q: torch.Tensor, q_pos: torch.Tensor, out: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
        """Decode with every shared document read once for all its readers (lazy_attn_decode_shared)."""
        if out is None:
            out = torch.empty_like(q)
        if plan.ws_bytes is None:
            plan.ws_bytes = L.decode_shared_workspace_size(self.geom, plan.num_reqs, plan.max_tiles,
                                                           plan.total_tiles, plan.max_req_reads)
        ws = self._workspace(plan.ws_bytes)
        L.attn_decode_shared(self.geom, self.pos.c, self.k_cache, self.v_cache, self.num_blocks, plan.tiles,
                             plan.tile_start, plan.ctx_tiles, plan.max_tiles, plan.total_tiles, plan.doc_tiles,
                             plan.doc_tile_start, plan.read_start, plan.reads, plan.req_reads, plan.work,
                             plan.num_docs, plan.num_work, plan.max_req_reads, plan.row_blocks, q, q_pos,
                             plan.num_reqs, out, ws, stream)
        return out

    def decode(self, tt: TileTable, q: torch.Tensor, q_pos: torch.Tensor, out: Optional[torch.Tensor] = None,
               pos: Optional[L.PosDescC] = None, stream=None) -> torch.Tensor:
        if out is None:
            out = torch.empty_like(q)
        ws = self._workspace(L.workspace_size(self.geom, tt.num_reqs, 1, tt.max_tiles, tt.total_tiles, False))
        L.attn_decode(self.geom, self.pos.c if pos is None else pos, self.k_cache, self.v_cache, self.num_blocks,
                      tt.tiles, tt.tile_start, tt.ctx_tiles, q, q_pos, tt.num_reqs, tt.max_tiles, tt.total_tiles, out,
                      ws, stream)
        return out
