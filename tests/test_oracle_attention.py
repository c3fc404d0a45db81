"""Pins for oracle.attention: deferred = eager on the pages' Example 3.1, brute force,
torch's scaled_dot_product_attention, translation invariance, variant special cases."""

import math

import numpy as np
import pytest
import torch

from oracle import attention, brute, rope

RNG = np.random.default_rng(99)


def _var(kind, dh, hq, base=1e4, slopes=None):
    if kind == "alibi":
        return {"kind": "alibi", "scale": 1 / math.sqrt(dh),
                "slopes": rope.alibi_slopes(hq) if slopes is None else slopes, "inv_freq": None}
    return {"kind": kind, "scale": 1 / math.sqrt(dh), "slopes": None, "inv_freq": rope.rope_inv_freq(dh, base)}


@pytest.mark.parametrize("kind", ["rope_half", "rope_interleaved"])
def test_example_3_1_deferred_equals_eager(kind):
    """Notes (papernotes.org), 'Method: overall framework', Example 3.1: d1 || d2 || Q.

    Deferred: each document is cached rotated from local position 0; against
    C2 the query is rotated back by |d1|.  Computed with scalar loops and
    compared with the oracle's eager global-position attention.
    """
    dh = 4
    theta = list(rope.rope_inv_freq(dh, 1e4))
    d1k, d1v = RNG.standard_normal((3, 1, dh)), RNG.standard_normal((3, 1, dh))
    d2k, d2v = RNG.standard_normal((2, 1, dh)), RNG.standard_normal((2, 1, dh))
    q, qk, qv = RNG.standard_normal((1, 1, dh)), RNG.standard_normal((1, 1, dh)), RNG.standard_normal((1, 1, dh))
    m = 5  # Q follows d1 (3 tokens) and d2 (2 tokens)
    c1 = [brute.rotate_pairs(list(d1k[j, 0]), j, theta, kind) for j in range(3)]  # cached at local 0..2
    c2 = [brute.rotate_pairs(list(d2k[j, 0]), j, theta, kind) for j in range(2)]  # cached at local 0..1
    q_glob = brute.rotate_pairs(list(q[0, 0]), m, theta, kind)
    q_back = brute.rotate_pairs(q_glob, -3, theta, kind)  # rotate Q back by |d1| for C2
    own = brute.rotate_pairs(list(qk[0, 0]), m, theta, kind)
    scale = 1 / math.sqrt(dh)
    scores = [scale * brute.dot(q_glob, c) for c in c1]
    scores += [scale * brute.dot(q_back, c) for c in c2]
    scores.append(scale * brute.dot(q_glob, own))
    vals = [list(x[0]) for x in d1v] + [list(x[0]) for x in d2v] + [list(qv[0, 0])]
    deferred = brute.softmax_weighted_sum(scores, vals)

    eager = attention.eager_prefill([(d1k, d1v), (d2k, d2v)], q, qk, qv, _var(kind, dh, 1))
    assert np.max(np.abs(eager[0, 0] - np.array(deferred))) < 1e-12


@pytest.mark.parametrize("kind", ["rope_half", "rope_interleaved", "alibi"])
def test_brute_force_matches_vectorised(kind):
    """Scalar loops (rotation as complex multiplication) vs the vectorised oracle; GQA, 3 docs, causal suffix."""
    dh, hq, hkv = 8, 4, 2
    var = _var(kind, dh, hq)
    docs = [(RNG.standard_normal((n, hkv, dh)), RNG.standard_normal((n, hkv, dh))) for n in (5, 1, 7)]
    Lq = 4
    q, k, v = RNG.standard_normal((Lq, hq, dh)), RNG.standard_normal((Lq, hkv, dh)), RNG.standard_normal((Lq, hkv, dh))
    got = attention.eager_prefill(docs, q, k, v, var)

    keys = [kk for kk, _ in docs] + [k]
    vals = [vv for _, vv in docs] + [v]
    keys = np.concatenate(keys)
    vals = np.concatenate(vals)
    n_ctx = 13
    theta = None if kind == "alibi" else list(var["inv_freq"])
    for i in range(Lq):
        m = n_ctx + i
        for h in range(hq):
            kvh = h // (hq // hkv)
            qv = list(q[i, h])
            if theta is not None:
                qv = brute.rotate_pairs(qv, m, theta, kind)
            ks, vs, bias = [], [], []
            for n in range(m + 1):
                kv = list(keys[n, kvh])
                if theta is not None:
                    kv = brute.rotate_pairs(kv, n, theta, kind)
                ks.append(kv)
                vs.append(list(vals[n, kvh]))
                bias.append(-var["slopes"][h] * (m - n) if kind == "alibi" else 0.0)
            want = brute.attention_one_query(qv, ks, vs, var["scale"], bias)
            assert np.max(np.abs(got[i, h] - np.array(want))) < 1e-12


@pytest.mark.parametrize("hq,hkv", [(4, 1), (8, 2), (4, 4)])
def test_single_document_matches_torch_sdpa(hq, hkv):
    """Delta = 0 single document + question = torch's causal scaled_dot_product_attention (CPU, fp64),
    with queries/keys rotated by transformers' apply_rotary_pos_emb (library routines)."""
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb

    dh, L, Lq, base = 64, 37, 6, 1e4
    doc = (RNG.standard_normal((L, hkv, dh)), RNG.standard_normal((L, hkv, dh)))
    q, k, v = RNG.standard_normal((Lq, hq, dh)), RNG.standard_normal((Lq, hkv, dh)), RNG.standard_normal((Lq, hkv, dh))
    var = _var("rope_half", dh, hq, base)
    got = attention.eager_prefill([doc], q, k, v, var)

    N = L + Lq
    pos = np.arange(N, dtype=np.float64)
    freqs = np.outer(pos, rope.rope_inv_freq(dh, base))
    emb = np.concatenate([freqs, freqs], -1)
    cos, sin = torch.from_numpy(np.cos(emb))[None], torch.from_numpy(np.sin(emb))[None]
    kk = torch.from_numpy(np.concatenate([doc[0], k]).transpose(1, 0, 2).copy())[None]
    vv = torch.from_numpy(np.concatenate([doc[1], v]).transpose(1, 0, 2).copy())[None]
    qq = torch.from_numpy(q.transpose(1, 0, 2).copy())[None]
    _, kr = apply_rotary_pos_emb(kk, kk, cos, sin)
    qr, _ = apply_rotary_pos_emb(qq, qq, cos[:, L:], sin[:, L:])
    mask = torch.from_numpy(np.arange(N)[None, :] <= (L + np.arange(Lq))[:, None])
    out = torch.nn.functional.scaled_dot_product_attention(qr, kr, vv, attn_mask=mask, enable_gqa=True)
    want = out[0].numpy().transpose(1, 0, 2)
    assert np.max(np.abs(got - want)) < 1e-12


def test_alibi_matches_sdpa_key_position_bias():
    """-slope (m - n) differs from slope * n by a per-row constant, so softmax agrees with torch SDPA
    given the additive mask slope_h * n (library routine); a sign error in the oracle would not."""
    dh, hq, L = 16, 6, 20
    var = _var("alibi", dh, hq)
    doc = (RNG.standard_normal((L, 1, dh)), RNG.standard_normal((L, 1, dh)))
    q, k, v = RNG.standard_normal((3, hq, dh)), RNG.standard_normal((3, 1, dh)), RNG.standard_normal((3, 1, dh))
    got = attention.eager_prefill([doc], q, k, v, var)
    N = L + 3
    n = np.arange(N, dtype=np.float64)
    bias = var["slopes"][:, None, None] * n[None, None, :] + np.zeros((hq, 3, N))
    causal = n[None, :] <= (L + np.arange(3))[:, None]
    bias = np.where(causal[None], bias, -np.inf)
    kk = torch.from_numpy(np.concatenate([doc[0], k]).transpose(1, 0, 2).copy())[None]
    vv = torch.from_numpy(np.concatenate([doc[1], v]).transpose(1, 0, 2).copy())[None]
    qq = torch.from_numpy(q.transpose(1, 0, 2).copy())[None]
    out = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=torch.from_numpy(bias)[None],
                                                           enable_gqa=True)
    assert np.max(np.abs(got - out[0].numpy().transpose(1, 0, 2))) < 1e-12


@pytest.mark.parametrize("kind", ["rope_half", "rope_interleaved", "alibi"])
def test_translation_invariance(kind):
    """Shifting every position by a constant leaves the output unchanged (relative-only positions)."""
    dh, hq, hkv = 32, 4, 2
    var = _var(kind, dh, hq, base=5e5)
    N, M = 50, 5
    k, v = RNG.standard_normal((N, hkv, dh)), RNG.standard_normal((N, hkv, dh))
    q = RNG.standard_normal((M, hq, dh))
    kpos = np.arange(N)
    qpos = np.arange(N - M, N)
    outs = []
    for c in (0, 1, 1000, 65000):
        kp = attention.position_keys(k, kpos + c, var)
        qp = q if kind == "alibi" else rope.rotate(q, qpos + c, var["inv_freq"], kind)
        outs.append(attention.attend(qp, qpos + c, kp, v, kpos + c, var))
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < 1e-9


def test_alibi_zero_slopes_is_plain_attention():
    dh, hq = 16, 3
    var0 = _var("alibi", dh, hq, slopes=np.zeros(hq))
    N = 12
    k, v, q = RNG.standard_normal((N, 1, dh)), RNG.standard_normal((N, 1, dh)), RNG.standard_normal((1, hq, dh))
    got = attention.attend(q, np.array([N - 1]), k, v, np.arange(N), var0)
    s = np.einsum("hd,nd->hn", q[0], k[:, 0]) / math.sqrt(dh)
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    assert np.max(np.abs(got[0] - p @ v[:, 0])) < 1e-13


def test_decode_matches_prefill_rows():
    """A decode step's output equals the last row of a prefill over the same sequence."""
    dh, hq, hkv = 16, 4, 2
    var = _var("rope_half", dh, hq)
    docs = [(RNG.standard_normal((9, hkv, dh)), RNG.standard_normal((9, hkv, dh)))]
    pre_k, pre_v = RNG.standard_normal((2, hkv, dh)), RNG.standard_normal((2, hkv, dh))
    steps = [(RNG.standard_normal((hq, dh)), RNG.standard_normal((hkv, dh)), RNG.standard_normal((hkv, dh)))
             for _ in range(3)]
    outs = attention.eager_decode(docs, pre_k, pre_v, steps, var)
    for s in range(3):
        # build the same sequence as a prefill whose question is pre tokens + generated tokens up to s
        qs = np.zeros((2 + s + 1, hq, dh))
        qs[-1] = steps[s][0]
        ks = np.concatenate([pre_k] + [st[1][None] for st in steps[: s + 1]])
        vs = np.concatenate([pre_v] + [st[2][None] for st in steps[: s + 1]])
        full = attention.eager_prefill(docs, qs, ks, vs, var)
        assert np.max(np.abs(full[-1] - outs[s])) < 1e-12


@pytest.mark.parametrize("kind", ["rope_half", "rope_interleaved", "alibi"])
def test_decode_without_context_attends_to_itself(kind):
    """No document and no question: the first generated token sees only itself, so every head's output is
    that token's value row of its KV head (softmax over one key is 1), whatever the position encoding; the
    next token mixes the two."""
    dh, hq, hkv = 16, 4, 2
    var = _var(kind, dh, hq)
    empty = np.zeros((0, hkv, dh))
    steps = [(RNG.standard_normal((hq, dh)), RNG.standard_normal((hkv, dh)), RNG.standard_normal((hkv, dh)))
             for _ in range(2)]
    outs = attention.eager_decode([], empty, empty, steps, var)
    want0 = np.repeat(steps[0][2], hq // hkv, axis=0)
    assert np.max(np.abs(outs[0] - want0)) < 1e-15
    # step 1: a convex combination of the two value rows, strictly between them where they differ
    v0 = np.repeat(steps[0][2], hq // hkv, axis=0)
    v1 = np.repeat(steps[1][2], hq // hkv, axis=0)
    lo, hi = np.minimum(v0, v1), np.maximum(v0, v1)
    assert np.all(outs[1] >= lo - 1e-12) and np.all(outs[1] <= hi + 1e-12)
    assert np.max(np.abs(outs[1] - v1)) > 1e-6 and np.max(np.abs(outs[1] - v0)) > 1e-6
