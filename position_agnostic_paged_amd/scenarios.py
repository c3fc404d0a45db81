"""Drive the synthetic workloads through the engine.

Each scenario performs the cache-side work once (documents written at local
positions into a shared, position-agnostic cache; private question tokens
written at global positions) and exposes the per-step device work:

  PrefillScenario  one prefill batch (questions over cached documents)
  DecodeScenario   decode steps: write the new token (q rotated in place at its
                   global position), then decode over every tile

``shared=False`` builds the no-sharing control layout: every (request,
document slot) gets a private physical copy, so no two requests read the same
K/V bytes.  ``prerotated=True`` (with shared=False) writes those copies
already rotated at their global positions and runs the kernels built without
deferral (LAZY_FLAG_PREROTATED): the "same kernel on pre-rotated K" control of
the overhead measurement, with an identical tile table and access pattern.
``aware=True`` (on an engine built with position_aware=True) is the
position-aware cache the pages compare against: requests that place a
document at the same offset share its copy, every other offset takes a copy
of its own, written pre-rotated at that offset.
"""

from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np
import torch

from .engine import Engine, PosDesc, TORCH_DTYPE
from .paging import PositionAwareCache, RequestLayout, Segment, blocks_for, layout_request


def make_pos(wl, device, max_pos: Optional[int] = None, on_the_fly: bool = False) -> PosDesc:
    p = wl.pos
    if max_pos is None:
        max_pos = max_position(wl) + 1
    return PosDesc(p.kind, wl.geom.head_dim, wl.geom.num_q_heads, device, base=p.base, yarn_factor=p.yarn_factor,
                   yarn_orig_ctx=p.yarn_orig_ctx, beta_fast=p.yarn_beta_fast, beta_slow=p.yarn_beta_slow,
                   max_pos=max_pos, on_the_fly=on_the_fly)


def max_position(wl) -> int:
    m = 0
    for step in wl.prefill_steps:
        for req in step:
            m = max(m, sum(wl.doc_lens[d] for d in req.doc_ids) + req.q.shape[0])
    for r in range(len(wl.decode_reqs)):
        m = max(m, wl.decode_ctx_len(r) + wl.num_decode_steps)
    return m


def blocks_needed(wl, shared: bool = True, aware: bool = False) -> int:
    """Physical blocks for every document and private segment of the workload (no eviction)."""
    if aware:
        placed = set()
        for step in wl.prefill_steps:
            for req in step:
                placed |= _placements(wl, req.doc_ids)
        for req in wl.decode_reqs:
            placed |= _placements(wl, req.doc_ids)
        n = sum(blocks_for(wl.doc_lens[d]) for d, _ in placed)
    elif shared:
        n = sum(blocks_for(wl.doc_lens[d]) for d in wl.all_doc_ids())
    else:
        n = 0
        for step in wl.prefill_steps:
            for req in step:
                n += sum(blocks_for(wl.doc_lens[d]) for d in req.doc_ids)
        for req in wl.decode_reqs:
            n += sum(blocks_for(wl.doc_lens[d]) for d in req.doc_ids)
    for step in wl.prefill_steps:
        for req in step:
            n += blocks_for(req.q.shape[0])
    for req in wl.decode_reqs:
        n += blocks_for(req.k.shape[0] + wl.num_decode_steps)
    return n


def _placements(wl, doc_ids) -> set:
    """(document, global offset) of each document of a request laid out from position 0."""
    out, pos = set(), 0
    for d in doc_ids:
        out.add((d, pos))
        pos += wl.doc_lens[d]
    return out


def _to_dev(x: np.ndarray, dtype, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=dtype)


class _Base:
    def __init__(self, wl, engine: Engine, shared: bool, prerotated: bool, aware: bool = False):
        if aware:
            if not isinstance(engine.docs, PositionAwareCache):
                raise ValueError("the position-aware layout needs an engine built with position_aware=True")
            shared, prerotated = True, True  # copies shared per (document, offset), written at global positions
        elif prerotated and shared:
            raise ValueError("pre-rotated copies are private by construction (shared=False)")
        self.wl, self.eng = wl, engine
        self.shared, self.prerotated, self.aware = shared, prerotated, aware
        self.tdtype = TORCH_DTYPE[wl.geom.dtype]
        self.dev = engine.device
        self.doc_writes = 0
        self._staged = {}  # raw document contents on the device (private copies reuse them)

    def _doc_dev(self, d: int):
        if d in self._staged:
            return self._staged[d]
        k, v = self.wl.doc(d, cache=False)
        kv = (_to_dev(k, self.tdtype, self.dev), _to_dev(v, self.tdtype, self.dev))
        if not self.shared:
            self._staged[d] = kv
        return kv

    def release_staging(self) -> None:
        self._staged.clear()

    def _doc_segments(self, doc_ids: Sequence[int]) -> List[Segment]:
        """Context segments of a request, placed consecutively from position 0."""
        segs, pos = [], 0
        for d in doc_ids:
            L = self.wl.doc_lens[d]
            if self.aware:
                blocks, hit = self.eng.cache_doc_at(d, pos, L, lambda d=d: self._doc_dev(d))
                self.doc_writes += 0 if hit else 1
                segs.append(Segment(list(blocks), L, pos, True))
            elif self.shared:
                blocks, hit = self.eng.cache_doc(d, L, lambda d=d: self._doc_dev(d))
                self.doc_writes += 0 if hit else 1
                segs.append(Segment(list(blocks), L, pos, True))
            else:
                blocks = self.eng.docs.take_private(blocks_for(L))
                k, v = self._doc_dev(d)
                # private copy: at local positions (deferred) or at its global positions (pre-rotated control)
                self.eng.write_segment(blocks, k, v, pos if self.prerotated else 0)
                self.doc_writes += 1
                segs.append(Segment(list(blocks), L, pos, True))
            pos += L
        return segs


class PrefillScenario(_Base):
    """One prefill batch: requests = cached documents + a question whose rows are the queries."""

    def __init__(self, wl, engine: Engine, step: int = 0, shared: bool = True, prerotated: bool = False,
                 aware: bool = False):
        super().__init__(wl, engine, shared, prerotated, aware)
        reqs = wl.prefill_steps[step]
        self.reqs = reqs
        lq = [r.q.shape[0] for r in reqs]
        self.max_q_len = max(lq)
        self.q_start_h = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
        self.q = _to_dev(np.concatenate([r.q for r in reqs]), self.tdtype, self.dev)
        layouts, qpos0 = [], []
        for i, r in enumerate(reqs):
            segs = self._doc_segments(r.doc_ids)
            ctx_len = sum(s.length for s in segs)
            priv = engine.docs.take_private(blocks_for(lq[i]))
            qi = self.q[self.q_start_h[i]: self.q_start_h[i + 1]]
            engine.write_segment(priv, _to_dev(r.k, self.tdtype, self.dev), _to_dev(r.v, self.tdtype, self.dev),
                                 ctx_len, q=qi)  # question K/V at global positions, q rotated in place
            segs.append(Segment(priv, lq[i], ctx_len, False))
            layouts.append(RequestLayout(segs))
            qpos0.append(ctx_len)
        self.layouts = layouts
        self.tt = engine.tile_table(layouts, paired=engine.prefill_pairs)
        self.q_start = torch.from_numpy(self.q_start_h).to(self.dev)
        self.q_pos0 = torch.tensor(qpos0, dtype=torch.int32, device=self.dev)
        self.out = torch.empty_like(self.q)

    def run(self, stream=None) -> torch.Tensor:
        pos = self.eng.pos.with_flags(self.prerotated, self.tt.paired)
        return self.eng.prefill(self.tt, self.q, self.q_start, self.q_pos0, self.max_q_len, out=self.out, pos=pos,
                                stream=stream)

    def flops(self) -> float:
        """Unmasked query-key pairs x 4 dh x Hq (the algorithmic work)."""
        g = self.wl.geom
        tot = 0
        for lay, r in zip(self.layouts, self.reqs):
            Lq = r.q.shape[0]
            C = lay.length - Lq
            tot += sum(C + i + 1 for i in range(Lq))
        return 4.0 * g.head_dim * g.num_q_heads * tot


class DecodeScenario(_Base):
    """Decode steps of a fixed batch: documents + optional question, then one new token per step."""

    def __init__(self, wl, engine: Engine, shared: bool = True, prerotated: bool = False,
                 prebuild_tables: bool = False, num_steps: Optional[int] = None, aware: bool = False,
                 doc_major: bool = False):
        super().__init__(wl, engine, shared, prerotated, aware)
        # doc_major: documents shared by several requests go through the document-major pass
        self.doc_major = doc_major
        if doc_major and (prerotated or not shared):
            raise ValueError("the document-major decode reads shared position-agnostic documents")
        self.num_steps = wl.num_decode_steps if num_steps is None else num_steps
        R = len(wl.decode_reqs)
        self.R = R
        self.ctx_segs, self.priv, self.priv_pos0, self.pre_len = [], [], [], []
        for r, req in enumerate(wl.decode_reqs):
            segs = self._doc_segments(req.doc_ids)
            ctx_len = sum(s.length for s in segs)
            Lq = req.k.shape[0]
            priv = engine.docs.take_private(blocks_for(Lq + self.num_steps))
            if Lq:
                engine.write_segment(priv, _to_dev(req.k, self.tdtype, self.dev), _to_dev(req.v, self.tdtype, self.dev),
                                     ctx_len)
            self.ctx_segs.append(segs)
            self.priv.append(priv)
            self.priv_pos0.append(ctx_len)
            self.pre_len.append(Lq)
        self.priv_pos0 = np.asarray(self.priv_pos0, np.int64)
        self.pre_len = np.asarray(self.pre_len, np.int64)
        self.q = torch.empty((R, wl.geom.num_q_heads, wl.geom.head_dim), dtype=self.tdtype, device=self.dev)
        self.out = torch.empty_like(self.q)
        self._priv_blocks = None
        # tokens of each request's cached documents (the bytes accounting of every step)
        self._ctx_tokens = np.array([sum(sg.length for sg in segs) for segs in self.ctx_segs], np.int64)
        self.tables = [self.table(s) for s in range(self.num_steps)] if prebuild_tables else None
        self._inputs = {}

    def layouts(self, step: int) -> List[RequestLayout]:
        out = []
        for r in range(self.R):
            n = int(self.pre_len[r]) + step + 1
            out.append(RequestLayout(self.ctx_segs[r] + [Segment(self.priv[r], n, int(self.priv_pos0[r]), False)]))
        return out

    def table(self, step: int):
        if self.doc_major:
            return self.eng.shared_plan(self.layouts(step))
        return self.eng.tile_table(self.layouts(step))

    def _attend(self, tt, q, q_pos, stream):
        if self.doc_major:
            return self.eng.decode_shared(tt, q, q_pos, out=self.out, stream=stream)
        return self.eng.decode(tt, q, q_pos, out=self.out, pos=self.eng.pos.with_flags(self.prerotated), stream=stream)

    def positions(self, step: int) -> np.ndarray:
        return (self.priv_pos0 + self.pre_len + step).astype(np.int32)

    def slots(self, step: int) -> np.ndarray:
        """Slot id of each request's new token at a step."""
        if self._priv_blocks is None:
            # one row of private block ids per request (padded), so a step's slots are one gather
            width = max(len(b) for b in self.priv) if self.R else 1
            self._priv_blocks = np.zeros((self.R, max(width, 1)), np.int64)
            for r, b in enumerate(self.priv):
                self._priv_blocks[r, : len(b)] = b
        i = self.pre_len + step
        return self._priv_blocks[np.arange(self.R), i // 16] * 16 + i % 16

    def stage_inputs(self, step: int):
        """Device copies of the step's raw q/k/v, positions and slots (setup, not timed)."""
        q, k, v = self.wl.decode_step(step)
        pos = self.positions(step)
        slots = self.slots(step)
        self.eng.check_write(pos, slots)
        t = (_to_dev(q, self.tdtype, self.dev), _to_dev(k, self.tdtype, self.dev), _to_dev(v, self.tdtype, self.dev),
             torch.from_numpy(pos).to(self.dev), torch.from_numpy(slots).to(self.dev))
        self._inputs[step] = t
        return t

    def step(self, step: int, stream=None, events=None) -> torch.Tensor:
        """Device work of one decode step: kv-write of the new token (q in place), then attention.

        ``events`` = (start, end) CUDA events recorded around the attention call only."""
        q0, k, v, pos, slots = self._inputs[step] if step in self._inputs else self.stage_inputs(step)
        self.q.copy_(q0)
        self.eng.kv_write(k, v, self.q, pos, slots, stream=stream)
        tt = self.tables[step] if self.tables is not None else self.table(step)
        if events is not None:
            events[0].record()
        out = self._attend(tt, self.q, pos, stream)
        if events is not None:
            events[1].record()
        return out

    def attend(self, step: int, q: torch.Tensor, q_pos: torch.Tensor, stream=None, events=None) -> torch.Tensor:
        """The attention call of a step alone, for a caller that wrote the new tokens itself (q already
        rotated to its global position, q_pos on the device).  ``events[0]`` may be None when the
        caller's previous end event already marks the start."""
        tt = self.tables[step] if self.tables is not None else self.table(step)
        if events is not None and events[0] is not None:
            events[0].record()
        out = self._attend(tt, q, q_pos, stream)
        if events is not None:
            events[1].record()
        return out

    def kv_bytes(self, step: int) -> float:
        """Algorithmic HBM bytes of one decode step (K and V of every visible token, q in, out)."""
        g = self.wl.geom
        esz = 2 if g.dtype == "bf16" else 4
        toks = int(np.sum(self._ctx_tokens + self.pre_len)) + self.R * (step + 1)
        return toks * 2 * g.num_kv_heads * g.head_dim * esz + 2 * self.R * g.num_q_heads * g.head_dim * esz
