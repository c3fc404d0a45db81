"""Hit ratios of a position-agnostic and a position-aware KV cache on synthetic retrieval traces.

The LazyAttention notes (papernotes.org, "Background and motivation") argue
that under a fixed HBM budget a position-aware cache wastes capacity on
position variants of the same document: with Zipf(alpha) popularity, D
possible positions and room for C entries, a position-agnostic cache holds
the top C documents and a position-aware one only floor(C / D) of them, a
hit-ratio gain of sum_{i<=C} i^-a / sum_{i<=C/D} i^-a (2.86x at D = 20,
C = 100).  Their "Main experiments" table measures VRAM hit ratios under
KV budgets of 1 / 10 / 50 GB and no limit, at low / mid / high skew, on
traces of real QA datasets (not available here).

This module replays seeded synthetic traces through the library's own host
caches (``paging.DocCache`` for the position-agnostic design,
``paging.PositionAwareCache`` for the position-aware one: same budget, same
whole-entry LRU eviction, same pinning of a request's documents) and reports
both hit ratios, plus the tokens each design has to (re)write into the cache.
Budgets are given as GB of full-model KV (every layer), so a document costs
``doc_tokens x bytes_per_token`` of the budget; one block of the simulated
pool stands for 16 tokens of that footprint.

``static_hit_ratios`` is the closed form's own setting: a cache whose
contents are fixed (the top-C documents, or the top floor(C/D) documents at
every one of the D positions) and independent accesses.

Run ``python -m position_agnostic_paged_amd.hitsim`` for the table.
"""

from __future__ import annotations

import argparse
import json
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

from .paging import BlockPool, DocCache, PositionAwareCache, blocks_for

# full-model KV bytes per token of the Llama-3.1-8B attention shape: 32 layers x (K + V) x 8 KV heads x
# 128 channels x 2 bytes (bf16)
LLAMA8B_KV_BYTES_PER_TOKEN = 32 * 2 * 8 * 128 * 2


@dataclass
class ReplayResult:
    accesses: int
    hits: int
    evictions: int
    tokens_written: int  # document tokens written into the cache on misses (re-encodes for the aware design)

    @property
    def hit_ratio(self) -> float:
        return self.hits / self.accesses if self.accesses else 0.0


def _run(trace: Sequence[Sequence[int]], doc_tokens: int, budget_blocks: Optional[int], aware: bool,
         record: Optional[List[bool]] = None) -> ReplayResult:
    per_doc = blocks_for(doc_tokens)
    longest = max((len(r) for r in trace), default=0)
    if budget_blocks is None:
        budget_blocks = per_doc * sum(len(r) for r in trace) or 1
    if budget_blocks < per_doc * longest:
        raise ValueError("the budget cannot hold one request's documents")
    pool = BlockPool(budget_blocks)
    cache = PositionAwareCache(pool) if aware else DocCache(pool)
    hits = written = n = 0
    for req in trace:
        keys = []
        for slot, d in enumerate(req):
            key = (d, slot * doc_tokens) if aware else d
            _, hit = cache.acquire(key, doc_tokens)
            keys.append(key)
            hits += hit
            written += 0 if hit else doc_tokens
            n += 1
            if record is not None:
                record.append(bool(hit))
        for key in keys:
            cache.release(key)
    return ReplayResult(n, hits, cache.evictions, written)


def replay(trace: Sequence[Sequence[int]], doc_tokens: int, budget_blocks: Optional[int],
           aware: bool) -> ReplayResult:
    """Replay requests (lists of document ids, placed consecutively from position 0) through one cache.

    ``budget_blocks`` None means no limit.  Every document has ``doc_tokens`` tokens, so document slot i
    of a request starts at global offset i x doc_tokens; the position-aware cache keys on that offset.
    A request pins its documents until all of them are resident (they are read together)."""
    return _run(trace, doc_tokens, budget_blocks, aware)


def hit_sequence(trace: Sequence[Sequence[int]], doc_tokens: int, budget_blocks: Optional[int],
                 aware: bool) -> List[bool]:
    """Per-access hit flags of ``replay``, in trace order."""
    out: List[bool] = []
    _run(trace, doc_tokens, budget_blocks, aware, out)
    return out


def static_hit_ratios(docs: np.ndarray, slots: np.ndarray, C: int, D: int) -> Dict[str, float]:
    """Hit ratios of two caches with fixed contents on independent (document, slot) accesses:
    position-agnostic = the C most popular documents (ids 0..C-1), position-aware = the floor(C/D) most
    popular documents at each of the D slots.  Slots must lie in [0, D)."""
    docs = np.asarray(docs)
    slots = np.asarray(slots)
    if slots.size and (slots.min() < 0 or slots.max() >= D):
        raise ValueError("slots outside [0, D)")
    agnostic = float(np.mean(docs < C))
    aware = float(np.mean(docs < C // D))
    return {"agnostic": agnostic, "aware": aware, "gain": agnostic / aware if aware else float("inf")}


def budget_blocks_for_gb(gb: float, bytes_per_token: int = LLAMA8B_KV_BYTES_PER_TOKEN) -> int:
    """Simulated pool blocks (16 tokens each) for a budget of ``gb`` x 2^30 bytes of full-model KV."""
    return int(gb * (1 << 30) // (16 * bytes_per_token))


def hit_ratio_table(alphas: Sequence[float] = (1.1, 1.5, 2.1), budgets_gb: Sequence[Optional[float]] = (1, 10, 50, None),
                    num_docs: int = 10000, docs_per_req: int = 10, doc_tokens: int = 200, num_reqs: int = 2000,
                    seed: int = 12) -> List[dict]:
    """Hit ratios of both designs for each skew and budget on one seeded trace per skew."""
    from workloads import zipf_trace

    rows = []
    for a in alphas:
        trace = zipf_trace(seed, num_docs, docs_per_req, num_reqs, a)
        for gb in budgets_gb:
            bb = None if gb is None else budget_blocks_for_gb(gb)
            ag = replay(trace, doc_tokens, bb, aware=False)
            aw = replay(trace, doc_tokens, bb, aware=True)
            rows.append({"alpha": a, "budget_gb": gb, "agnostic_hit": ag.hit_ratio, "aware_hit": aw.hit_ratio,
                         "gain": ag.hit_ratio / aw.hit_ratio if aw.hits else float("inf"),
                         "agnostic_tokens_written": ag.tokens_written, "aware_tokens_written": aw.tokens_written,
                         "accesses": ag.accesses})
    return rows


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--num-docs", type=int, default=10000)
    ap.add_argument("--docs-per-req", type=int, default=10)
    ap.add_argument("--doc-tokens", type=int, default=200)
    ap.add_argument("--requests", type=int, default=2000)
    ap.add_argument("--json", action="store_true")
    args = ap.parse_args()
    rows = hit_ratio_table(num_docs=args.num_docs, docs_per_req=args.docs_per_req, doc_tokens=args.doc_tokens,
                           num_reqs=args.requests)
    if args.json:
        print(json.dumps(rows))
        return
    print(f"{'alpha':>5} {'budget':>8} {'agnostic %':>11} {'aware %':>8} {'gain':>6} {'aware/agnostic writes':>22}")
    for r in rows:
        b = "no limit" if r["budget_gb"] is None else f"{r['budget_gb']:g} GB"
        w = r["aware_tokens_written"] / max(1, r["agnostic_tokens_written"])
        print(f"{r['alpha']:>5} {b:>8} {100 * r['agnostic_hit']:>11.2f} {100 * r['aware_hit']:>8.2f} "
              f"{r['gain']:>6.2f} {w:>22.2f}")


if __name__ == "__main__":
    main()
