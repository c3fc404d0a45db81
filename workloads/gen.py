"""Seeded workload generators.

Every random draw comes from ``numpy.random.default_rng(SeedSequence([wid,
stream, ...]))`` where ``wid`` identifies the workload and ``stream`` the kind
of draw:

    0  document contents (per document id)
    1  document choice and order (per request)
    2  suffix (question) q/k/v (per request)
    3  decode-step q/k/v (per step)
    4  lengths (mixed-batch decode context sizes)
    5  queries of a document's own tokens (the document-processing pass
       that writes its cache entry on a miss; per document id), and extra
       question draws keyed by a caller-chosen id
    6  independent (document, position) accesses of a static-cache
       hit-ratio trace

so any single document, request or step can be regenerated on its own.  Draws
are fp32 normals; bf16 workloads round them to the nearest bf16 (ties to even)
once, here, and both sides consume the rounded values.

Nothing in this module implements the method's arithmetic (no rotation, no
attention, no packing).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

BLOCK_SIZE = 16


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 holding bf16-exact values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    r = ((u + bias) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


@dataclass(frozen=True)
class Geometry:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # "fp32" or "bf16"
    block_size: int = BLOCK_SIZE


@dataclass(frozen=True)
class PosSpec:
    """Positional-encoding variant parameters (no derived quantities)."""

    kind: str  # "rope_half", "rope_interleaved" or "alibi"
    base: float = 10000.0
    yarn_factor: float = 1.0  # 1.0 = plain RoPE
    yarn_orig_ctx: int = 0
    yarn_beta_fast: float = 32.0
    yarn_beta_slow: float = 1.0


@dataclass
class PrefillRequest:
    doc_ids: List[int]
    q: np.ndarray  # [Lq][Hq][dh] raw (pre-position) question queries
    k: np.ndarray  # [Lq][Hkv][dh]
    v: np.ndarray  # [Lq][Hkv][dh]


@dataclass
class DecodeRequest:
    doc_ids: List[int]
    # question tokens that precede generation (may be empty: Lq = 0)
    k: np.ndarray  # [Lq][Hkv][dh]
    v: np.ndarray  # [Lq][Hkv][dh]


@dataclass
class Workload:
    name: str
    wid: int
    geom: Geometry
    pos: PosSpec
    kv_scale: float
    doc_lens: Dict[int, int]
    prefill_steps: List[List[PrefillRequest]] = field(default_factory=list)
    decode_reqs: List[DecodeRequest] = field(default_factory=list)
    num_decode_steps: int = 0
    description: str = ""
    kv_budget_blocks: Optional[int] = None  # document-cache budget in blocks (None = unlimited)
    q_scale: float = 1.0  # multiplier on decode-step queries (a power of two: exact in bf16)
    _doc_cache: Dict[int, Tuple[np.ndarray, np.ndarray]] = field(default_factory=dict, repr=False)

    # ----------------------------------------------------------------- draws
    def _normal(self, seed: List[int], shape, scale: float) -> np.ndarray:
        rng = np.random.default_rng(np.random.SeedSequence([self.wid] + list(seed)))
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        if self.geom.dtype == "bf16":
            x = round_to_bf16(x)
        return x

    def doc(self, doc_id: int, cache: bool = True) -> Tuple[np.ndarray, np.ndarray]:
        """Raw (content-only) k, v of one document: two fp32 arrays [L][Hkv][dh]."""
        if doc_id in self._doc_cache:
            return self._doc_cache[doc_id]
        g = self.geom
        L = self.doc_lens[doc_id]
        both = self._normal([0, doc_id], (2, L, g.num_kv_heads, g.head_dim), self.kv_scale)
        kv = (both[0], both[1])
        if cache:
            self._doc_cache[doc_id] = kv
        return kv

    def doc_queries(self, doc_id: int) -> np.ndarray:
        """Raw queries [L][Hq][dh] of a document's own tokens (its processing pass on a miss)."""
        g = self.geom
        return self._normal([5, 0, doc_id], (self.doc_lens[doc_id], g.num_q_heads, g.head_dim), 1.0)

    def extra_question(self, key: int, length: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """A question (q [L][Hq][dh], k, v [L][Hkv][dh]) outside the workload's own requests."""
        g = self.geom
        q = self._normal([5, 1, key], (length, g.num_q_heads, g.head_dim), 1.0)
        kv = self._normal([5, 2, key], (2, length, g.num_kv_heads, g.head_dim), self.kv_scale)
        return q, kv[0], kv[1]

    def decode_step(self, step: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """q [R][Hq][dh], k [R][Hkv][dh], v [R][Hkv][dh] raw draws for every decode request at one step."""
        g = self.geom
        R = len(self.decode_reqs)
        rng = np.random.default_rng(np.random.SeedSequence([self.wid, 3, step]))
        q = rng.standard_normal(size=(R, g.num_q_heads, g.head_dim), dtype=np.float32)
        kv = rng.standard_normal(size=(2, R, g.num_kv_heads, g.head_dim), dtype=np.float32)
        kv *= np.float32(self.kv_scale)
        if g.dtype == "bf16":
            q, kv = round_to_bf16(q), round_to_bf16(kv)
        if self.q_scale != 1.0:
            q = q * np.float32(self.q_scale)  # exact: a power of two
        return q, kv[0], kv[1]

    # ------------------------------------------------------------ structure
    def decode_ctx_len(self, r: int) -> int:
        """Tokens before the first generated token of decode request r (documents + question)."""
        req = self.decode_reqs[r]
        return sum(self.doc_lens[d] for d in req.doc_ids) + req.k.shape[0]

    def all_doc_ids(self) -> List[int]:
        ids = set()
        for step in self.prefill_steps:
            for req in step:
                ids.update(req.doc_ids)
        for req in self.decode_reqs:
            ids.update(req.doc_ids)
        return sorted(ids)


def _zipf_pick(wid: int, req_key: List[int], pool: int, n: int, alpha: float) -> List[int]:
    """n distinct documents from a pool, Zipf(alpha) popularity by id rank, in a random order."""
    rng = np.random.default_rng(np.random.SeedSequence([wid, 1] + list(req_key)))
    w = np.arange(1, pool + 1, dtype=np.float64) ** (-alpha)
    ids = rng.choice(pool, size=n, replace=False, p=w / w.sum())
    return [int(i) for i in rng.permutation(ids)]


def zipf_trace(seed: int, num_docs: int, docs_per_req: int, num_reqs: int, alpha: float) -> List[List[int]]:
    """A retrieval trace: each request draws docs_per_req distinct documents from a pool of num_docs with
    Zipf(alpha) popularity by id rank (rank 1 = document 0) and places them in a random order; requests
    are independent.  Seeded by (seed, request index), stream 1 as for the workloads' requests."""
    return [_zipf_pick(seed, [r], num_docs, docs_per_req, alpha) for r in range(num_reqs)]


def zipf_accesses(seed: int, num_docs: int, n: int, alpha: float, positions: int) -> Tuple[np.ndarray, np.ndarray]:
    """n independent (document, position slot) accesses: documents Zipf(alpha) by id rank, slots uniform
    over ``positions`` (the static-cache setting of the pages' hit-ratio formula)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 6]))
    w = np.arange(1, num_docs + 1, dtype=np.float64) ** (-alpha)
    docs = rng.choice(num_docs, size=n, p=w / w.sum())
    slots = rng.integers(0, positions, size=n)
    return docs, slots


def _question(wl: Workload, req_key: List[int], Lq: int, with_q: bool):
    g = wl.geom
    rng = np.random.default_rng(np.random.SeedSequence([wl.wid, 2] + list(req_key)))
    q = rng.standard_normal(size=(Lq, g.num_q_heads, g.head_dim), dtype=np.float32)
    kv = rng.standard_normal(size=(2, Lq, g.num_kv_heads, g.head_dim), dtype=np.float32)
    kv *= np.float32(wl.kv_scale)
    if g.dtype == "bf16":
        q, kv = round_to_bf16(q), round_to_bf16(kv)
    if with_q:
        return PrefillRequest(doc_ids=[], q=q, k=kv[0], v=kv[1])
    return DecodeRequest(doc_ids=[], k=kv[0], v=kv[1])


# --------------------------------------------------------------------------- workloads

def _tiny_fp32() -> Workload:
    wl = Workload(
        name="tiny_fp32_2doc_h4kv1_d64",
        wid=1,
        geom=Geometry(4, 1, 64, "fp32"),
        pos=PosSpec("rope_half", base=1e4),
        kv_scale=1.0,
        doc_lens={0: 64, 1: 48},
        num_decode_steps=8,
        description="doc A (64 tok) || doc B (48 tok) || 16-token suffix, then 8 decode steps; fp32",
    )
    pre = _question(wl, [0], 16, True)
    pre.doc_ids = [0, 1]
    wl.prefill_steps = [[pre]]
    # the decode request continues the same sequence: documents + the 16 suffix tokens
    wl.decode_reqs = [DecodeRequest(doc_ids=[0, 1], k=pre.k, v=pre.v)]
    return wl


def _prefill_llama8b(kind: str, wid: int, name: str) -> Workload:
    wl = Workload(
        name=name,
        wid=wid,
        geom=Geometry(32, 8, 128, "bf16"),
        pos=PosSpec(kind, base=5e5),
        kv_scale=0.5,
        doc_lens={d: 200 for d in range(100)},
        description="8 requests x (10 Zipf(2.1) docs of 200 tok from a 100-doc pool + 32-tok question)",
    )
    reqs = []
    for r in range(8):
        pr = _question(wl, [r], 32, True)
        pr.doc_ids = _zipf_pick(wid, [r], 100, 10, 2.1)
        reqs.append(pr)
    wl.prefill_steps = [reqs]
    return wl


def _decode_llama8b() -> Workload:
    wl = Workload(
        name="llama8b_decode_b64_ctx32k",
        wid=3,
        geom=Geometry(32, 8, 128, "bf16"),
        pos=PosSpec("rope_half", base=5e5),
        kv_scale=0.5,
        doc_lens={d: 1600 for d in range(200)},
        num_decode_steps=64,
        description="64 requests x 20 Zipf(1.2) docs of 1600 tok (200-doc pool); 64 decode steps",
    )
    z = np.zeros((0, 8, 128), np.float32)
    wl.decode_reqs = [DecodeRequest(doc_ids=_zipf_pick(3, [r], 200, 20, 1.2), k=z, v=z) for r in range(64)]
    return wl


def _mixed_llama70b(num_steps: int = 16, prefill_alpha: float = 2.1) -> Workload:
    wl = Workload(
        name="llama70b_mixed_yarn8_p4x7.5k_d48x8k-64k",
        wid=4,
        geom=Geometry(64, 8, 128, "bf16"),
        pos=PosSpec("rope_half", base=5e5, yarn_factor=8.0, yarn_orig_ctx=8192),
        kv_scale=0.5,
        doc_lens={d: 500 for d in range(1000)},
        num_decode_steps=num_steps,
        kv_budget_blocks=16384,
        description=(
            "per step: 4 prefills (15 Zipf(2.1) docs x 500 tok + 64-tok question) + 48 decodes "
            "(n x 500-tok docs + 64-tok question, n ~ U{16..131}); 1000-doc pool; 1 GiB KV budget"
        ),
    )
    rng = np.random.default_rng(np.random.SeedSequence([4, 4]))
    ns = rng.integers(16, 132, size=48)
    decs = []
    for r in range(48):
        dr = _question(wl, [1000 + r], 64, False)
        dr.doc_ids = _zipf_pick(4, [1000 + r], 1000, int(ns[r]), 2.1)
        decs.append(dr)
    wl.decode_reqs = decs
    steps = []
    for s in range(num_steps):
        reqs = []
        for j in range(4):
            pr = _question(wl, [s, j], 64, True)
            pr.doc_ids = _zipf_pick(4, [s, j], 1000, 15, prefill_alpha)
            reqs.append(pr)
        steps.append(reqs)
    wl.prefill_steps = steps
    return wl


def _falcon_alibi() -> Workload:
    wl = Workload(
        name="falcon7b_mqa_alibi_b128_ctx16k",
        wid=5,
        geom=Geometry(71, 1, 64, "bf16"),
        pos=PosSpec("alibi"),
        kv_scale=0.5,
        doc_lens={d: 2048 for d in range(64)},
        num_decode_steps=64,
        description="128 requests x 8 Zipf(1.5) docs of 2048 tok (64-doc pool); MQA 71 heads; 64 decode steps",
    )
    z = np.zeros((0, 1, 64), np.float32)
    wl.decode_reqs = [DecodeRequest(doc_ids=_zipf_pick(5, [r], 64, 8, 1.5), k=z, v=z) for r in range(128)]
    return wl


def _ragged() -> Workload:
    """Edge cases: uneven requests, partial blocks, questions of 1..64 tokens, a request with no document."""
    wl = Workload(
        name="ragged_bf16_h8kv2_d128",
        wid=7,
        geom=Geometry(8, 2, 128, "bf16"),
        pos=PosSpec("rope_half", base=5e5),
        kv_scale=0.5,
        doc_lens={d: [300, 17, 1, 250, 16, 999][d % 6] for d in range(60)},
        num_decode_steps=5,
        description="ragged lengths: documents of 1..999 tokens, 0..40 per request, questions of 1..64 tokens",
    )
    pre = []
    for r, (ndoc, lq) in enumerate([(0, 5), (3, 1), (5, 64), (1, 33), (6, 17)]):
        pr = _question(wl, [r], lq, True)
        pr.doc_ids = _zipf_pick(7, [r], 60, ndoc, 1.0) if ndoc else []
        pre.append(pr)
    wl.prefill_steps = [pre]
    decs = []
    for r, (ndoc, lq) in enumerate([(1, 0), (40, 3), (2, 16), (12, 0), (0, 7), (25, 1)]):
        dr = _question(wl, [100 + r], lq, False)
        dr.doc_ids = _zipf_pick(7, [100 + r], 60, ndoc, 1.0) if ndoc else []
        decs.append(dr)
    wl.decode_reqs = decs
    return wl


def _falcon_alibi_prefill() -> Workload:
    """Falcon-7B attention shape (MQA 71/1, dh 64, ALiBi) on a prefill batch: 4 requests x (5 Zipf docs
    of 100..700 tokens + a question of 7..48 tokens)."""
    wl = Workload(
        name="falcon7b_mqa_alibi_prefill_b4",
        wid=8,
        geom=Geometry(71, 1, 64, "bf16"),
        pos=PosSpec("alibi"),
        kv_scale=0.5,
        doc_lens={d: 100 + 37 * d for d in range(17)},
        description="4 requests x (5 Zipf(1.3) docs of 100..692 tok from 17) + 7..48-token question; MQA 71 heads",
    )
    pre = []
    for r, lq in enumerate([48, 7, 31, 16]):
        pr = _question(wl, [r], lq, True)
        pr.doc_ids = _zipf_pick(8, [r], 17, 5, 1.3)
        pre.append(pr)
    wl.prefill_steps = [pre]
    return wl


def _small_dh64_interleaved() -> Workload:
    """dh 64 with interleaved RoPE and GQA 8/2 (bf16): a prefill batch and decode steps over documents
    whose lengths leave partial last blocks."""
    wl = Workload(
        name="gqa8x2_d64_interleaved",
        wid=9,
        geom=Geometry(8, 2, 64, "bf16"),
        pos=PosSpec("rope_interleaved", base=1e4),
        kv_scale=0.5,
        doc_lens={d: 37 + 61 * d for d in range(12)},
        num_decode_steps=4,
        description="3 prefills (4 docs of 37..708 tok + 20..60-tok question) and 5 decodes (2..6 docs)",
    )
    pre = []
    for r, lq in enumerate([20, 60, 41]):
        pr = _question(wl, [r], lq, True)
        pr.doc_ids = _zipf_pick(9, [r], 12, 4, 1.0)
        pre.append(pr)
    wl.prefill_steps = [pre]
    decs = []
    for r, nd in enumerate([2, 6, 3, 5, 4]):
        dr = _question(wl, [100 + r], 9 + r, False)
        dr.doc_ids = _zipf_pick(9, [100 + r], 12, nd, 1.0)
        decs.append(dr)
    wl.decode_reqs = decs
    return wl


def _long_context() -> Workload:
    """Documents far from position 0: eight of 15.7K-16.4K tokens and one of 5 tokens, 128K tokens in all,
    RoPE base 1e4 (rotation angles up to ~1.3e5 rad, where the table and the in-kernel sincos must stay
    exact): one prefill with an 8-token question after every document (the 5-token one last) and two
    decode requests over the documents in other orders."""
    wl = Workload(
        name="long_ctx128k_h2kv1_d128",
        wid=10,
        geom=Geometry(2, 1, 128, "bf16"),
        pos=PosSpec("rope_half", base=1e4),
        kv_scale=0.5,
        doc_lens={**{d: 16384 - 97 * d for d in range(8)}, 8: 5},
        num_decode_steps=2,
        description="9 documents (8 x ~16K + 5 tok) = 128,361 tokens; 1 prefill (8-tok question), 2 decodes; GQA 2/1",
    )
    pr = _question(wl, [0], 8, True)
    pr.doc_ids = [3, 0, 6, 1, 7, 2, 5, 4, 8]
    wl.prefill_steps = [[pr]]
    d0 = _question(wl, [100], 3, False)
    d0.doc_ids = [8, 7, 6, 5, 4, 3, 2, 1, 0]
    d1 = _question(wl, [101], 0, False)
    d1.doc_ids = list(range(9))
    wl.decode_reqs = [d0, d1]
    return wl


def _pages_overhead() -> Workload:
    """The shape of the pages' overhead experiment (LazyAttention notes, "Ablation / kernel overhead"):
    five 4096-token documents and a 64-token question per request, three documents hot (shared by
    every request, in a per-request order) and two cold (private to the request); Llama-3.1-8B
    attention shape.  4 prefill requests and 64 decode requests (4 decode steps)."""
    n_pre, n_dec = 4, 64
    hot = [0, 1, 2]
    wl = Workload(
        name="pages_overhead_5x4096_q64_llama8b",
        wid=11,
        geom=Geometry(32, 8, 128, "bf16"),
        pos=PosSpec("rope_half", base=5e5),
        kv_scale=0.5,
        doc_lens={d: 4096 for d in range(3 + 2 * (n_pre + n_dec))},
        num_decode_steps=4,
        description="5 x 4096-tok docs (3 hot, 2 private) + 64-tok question; 4 prefills, 64 decodes",
    )

    def docs_for(k: int, r: int) -> List[int]:
        rng = np.random.default_rng(np.random.SeedSequence([11, 1, k]))
        cold = [3 + 2 * r, 4 + 2 * r]
        return [int(d) for d in rng.permutation(hot + cold)]

    pre = []
    for r in range(n_pre):
        pr = _question(wl, [r], 64, True)
        pr.doc_ids = docs_for(r, r)
        pre.append(pr)
    wl.prefill_steps = [pre]
    decs = []
    for r in range(n_dec):
        dr = _question(wl, [100 + r], 64, False)
        dr.doc_ids = docs_for(100 + r, n_pre + r)
        decs.append(dr)
    wl.decode_reqs = decs
    return wl


WORKLOADS = {
    "ragged": _ragged,
    "pages_overhead": _pages_overhead,
    "long_context": _long_context,
    "tiny_fp32": _tiny_fp32,
    "llama8b_prefill": lambda: _prefill_llama8b("rope_half", 2, "llama8b_prefill_b8_10x200"),
    "llama8b_decode": _decode_llama8b,
    "llama70b_mixed": _mixed_llama70b,
    "falcon7b_alibi": _falcon_alibi,
    "falcon7b_alibi_prefill": _falcon_alibi_prefill,
    "small_dh64_interleaved": _small_dh64_interleaved,
    "llama8b_prefill_interleaved": lambda: _prefill_llama8b(
        "rope_interleaved", 2, "llama8b_prefill_b8_10x200_interleaved"
    ),
}


def make_workload(key: str, **kw) -> Workload:
    return WORKLOADS[key](**kw)


def sharpened(wl: Workload, factor: float = 4.0) -> Workload:
    """The same workload with every query multiplied by ``factor`` (a power of two, so bf16 values stay
    exact): scores grow by the factor and attention concentrates on fewer keys, so outputs are larger
    and depend more on where each key sits."""
    m, e = np.frexp(factor)
    if factor <= 0 or m != 0.5:
        raise ValueError("the sharpening factor must be a power of two")
    wl.q_scale *= factor
    wl.name = f"{wl.name}_q{factor:g}x"
    for step in wl.prefill_steps:
        for r in step:
            r.q = r.q * np.float32(factor)
    return wl
