"""Eager fp64 attention over a request's logical sequence (oracle; test infrastructure only).

The LazyAttention notes (papernotes.org, "Method: overall framework" and
Example 3.1) describe a request as documents d1 || d2 || ... || question, each
document reused from a cache, and state that the deferred computation equals
standard RoPE attention with keys at their positions in that concatenation.
This module computes exactly that standard attention:

  * document i starts at Delta_i = sum of the lengths of the documents before
    it; its token j sits at global position Delta_i + j;
  * question tokens follow the last document; generated tokens follow them;
  * queries and keys are rotated at their global positions (RoPE kinds) or
    left as they are (ALiBi, bias -slope_h * (m - n) added to the score);
  * a query at position m sees every key at position n <= m (documents are
    fully visible to the question, the question is causal, a decode token
    sees everything before it and itself);
  * softmax with max subtraction in fp64; query head h reads key/value head
    floor(h / G), G = Hq / Hkv (GQA/MQA: notes, "Generality").
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

from . import rope


def logical_sequence(docs: Sequence[Tuple[np.ndarray, np.ndarray]],
                     tail_k: np.ndarray = None, tail_v: np.ndarray = None):
    """Concatenate documents (then an optional tail of private tokens).

    Either part may be empty (a request with no cached document, a decode
    request with no question): with no document and an empty tail the context
    is the empty sequence, shaped like the tail.
    Returns raw keys [N][Hkv][dh], values [N][Hkv][dh] and global positions [N].
    """
    ks = [np.asarray(k, np.float64) for k, _ in docs]
    vs = [np.asarray(v, np.float64) for _, v in docs]
    if tail_k is not None:
        ks.append(np.asarray(tail_k, np.float64))
        vs.append(np.asarray(tail_v, np.float64))
    k = np.concatenate(ks, axis=0)
    v = np.concatenate(vs, axis=0)
    return k, v, np.arange(k.shape[0], dtype=np.int64)


def position_keys(k_raw: np.ndarray, k_pos: np.ndarray, var: dict) -> np.ndarray:
    """Keys as ordinary RoPE attention sees them: rotated at their global positions."""
    if var["kind"] == "alibi":
        return np.asarray(k_raw, np.float64)
    return rope.rotate(k_raw, k_pos, var["inv_freq"], var["kind"])


def attend(q: np.ndarray, q_pos: np.ndarray, k: np.ndarray, v: np.ndarray,
           k_pos: np.ndarray, var: dict) -> np.ndarray:
    """softmax(scale * q k^T + bias + mask) v for positioned q [M][Hq][dh], k/v [N][Hkv][dh]."""
    q = np.asarray(q, np.float64)
    M, Hq, dh = q.shape
    N, Hkv, _ = k.shape
    G = Hq // Hkv
    kh = np.repeat(np.asarray(k, np.float64), G, axis=1)  # [N][Hq][dh]: head h -> kv head h // G
    vh = np.repeat(np.asarray(v, np.float64), G, axis=1)
    s = np.einsum("mhd,nhd->hmn", q, kh) * var["scale"]
    dist = q_pos[:, None].astype(np.float64) - k_pos[None, :].astype(np.float64)  # m - n
    if var["kind"] == "alibi":
        s = s - var["slopes"][:, None, None] * dist[None, :, :]
    visible = dist >= 0
    s = np.where(visible[None, :, :], s, -np.inf)
    smax = np.max(s, axis=2, keepdims=True)
    p = np.exp(s - smax)
    p = p / np.sum(p, axis=2, keepdims=True)
    return np.einsum("hmn,nhd->mhd", p, vh)


def eager_prefill(docs, q_raw, k_raw, v_raw, var) -> np.ndarray:
    """Output [Lq][Hq][dh] of the question tokens of one request d1 || ... || dn || question."""
    k, v, pos = logical_sequence(docs, k_raw, v_raw)
    Lq = np.asarray(q_raw).shape[0]
    q_pos = pos[-Lq:] if Lq else pos[:0]
    kp = position_keys(k, pos, var)
    qp = q_raw if var["kind"] == "alibi" else rope.rotate(q_raw, q_pos, var["inv_freq"], var["kind"])
    return attend(qp, q_pos, kp, v, pos, var)


def eager_decode(docs, pre_k, pre_v, steps: List[Tuple[np.ndarray, np.ndarray, np.ndarray]], var,
                 which: Sequence[int] = None) -> List[np.ndarray]:
    """Outputs [Hq][dh] of successive decode tokens of one request.

    ``docs`` and the private prefix ``pre_k/pre_v`` (question tokens, possibly
    empty) form the context; ``steps[s] = (q, k, v)`` are the raw draws of the
    token generated at step s ([Hq][dh], [Hkv][dh], [Hkv][dh]).  The token of
    step s sits right after the context and the s earlier generated tokens.
    ``which`` selects the steps whose output is computed (default: all).
    """
    k0, v0, _ = logical_sequence(docs, pre_k, pre_v)
    n_ctx = k0.shape[0]
    S = len(steps)
    k_all = np.concatenate([k0] + [np.asarray(st[1], np.float64)[None] for st in steps], axis=0)
    v_all = np.concatenate([v0] + [np.asarray(st[2], np.float64)[None] for st in steps], axis=0)
    pos = np.arange(n_ctx + S, dtype=np.int64)
    kp = position_keys(k_all, pos, var)
    outs = []
    for s in (range(S) if which is None else which):
        m = n_ctx + s
        q = np.asarray(steps[s][0], np.float64)[None]
        qpos = np.array([m], dtype=np.int64)
        qp = q if var["kind"] == "alibi" else rope.rotate(q, qpos, var["inv_freq"], var["kind"])
        outs.append(attend(qp, qpos, kp[: m + 1], v_all[: m + 1], pos[: m + 1], var)[0])
    return outs
