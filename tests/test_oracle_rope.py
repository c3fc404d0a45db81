"""Pins for oracle.rope: RoPE rotation, pairing, frequencies, YaRN, ALiBi slopes.

Each check ties the oracle to something other than itself: the RoPE relative
identity and group laws (LazyAttention notes, papernotes.org, "Background and
motivation" / "Key designs"), RoPE as a complex multiplication (brute force),
Hugging Face transformers' rotary routines (library), and closed-form
special cases of the YaRN and ALiBi definitions.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import brute, rope

RNG = np.random.default_rng(1234)


@pytest.mark.parametrize("dh,base", [(64, 1e4), (128, 5e5)])
@pytest.mark.parametrize("kind", ["rope_half", "rope_interleaved"])
def test_relative_identity(dh, base, kind):
    """(R_m q)^T (R_n k) = q^T R_{n-m} k (notes, 'Background and motivation'), m, n up to 131072."""
    inv = rope.rope_inv_freq(dh, base)
    for _ in range(20):
        q = RNG.standard_normal((1, 1, dh))
        k = RNG.standard_normal((1, 1, dh))
        m, n = RNG.integers(0, 131072, size=2)
        lhs = np.sum(rope.rotate(q, [m], inv, kind) * rope.rotate(k, [n], inv, kind))
        rhs = np.sum(q * rope.rotate(k, [n - m], inv, kind))
        assert abs(lhs - rhs) <= 1e-9 * np.linalg.norm(q) * np.linalg.norm(k)


@pytest.mark.parametrize("kind", ["rope_half", "rope_interleaved"])
def test_group_laws(kind):
    """R_a R_b = R_{a+b}; R_{-a} = R_a^T; norms preserved (single rotation = back-then-forward)."""
    dh = 128
    inv = rope.rope_inv_freq(dh, 5e5)
    x = RNG.standard_normal((5, 2, dh))
    for a, b in [(3, 7), (1600, -1600), (65535, 17), (0, 0)]:
        pa = np.full(5, a)
        pb = np.full(5, b)
        two = rope.rotate(rope.rotate(x, pb, inv, kind), pa, inv, kind)
        one = rope.rotate(x, pa + pb, inv, kind)
        assert np.max(np.abs(two - one)) < 1e-10
        # R_{-a} is the transpose of R_a: <R_a x, y> = <x, R_{-a} y>
        y = RNG.standard_normal((5, 2, dh))
        lhs = np.sum(rope.rotate(x, pa, inv, kind) * y)
        rhs = np.sum(x * rope.rotate(y, -pa, inv, kind))
        assert abs(lhs - rhs) < 1e-9
        assert np.allclose(np.linalg.norm(rope.rotate(x, pa, inv, kind), axis=-1),
                           np.linalg.norm(x, axis=-1), rtol=1e-13)


@pytest.mark.parametrize("kind", ["rope_half", "rope_interleaved"])
def test_rotation_is_complex_multiplication(kind):
    """Each channel pair (a, b) becomes (a + ib) e^{i p theta} -- catches sign and pairing errors."""
    dh = 16
    inv = rope.rope_inv_freq(dh, 1e4)
    x = RNG.standard_normal((3, 1, dh))
    pos = np.array([0, 5, 12345])
    got = rope.rotate(x, pos, inv, kind)
    for i, p in enumerate(pos):
        want = brute.rotate_pairs(list(x[i, 0]), float(p), list(inv), kind)
        assert np.max(np.abs(got[i, 0] - np.array(want))) < 1e-12


def test_first_pair_unit_vector():
    """Position 1, theta_0 = 1: (1, 0) in pair 0 turns to (cos 1, sin 1)."""
    inv = rope.rope_inv_freq(2, 1e4)
    assert inv[0] == 1.0
    out = rope.rotate(np.array([[[1.0, 0.0]]]), [1], inv, "rope_half")
    assert np.allclose(out[0, 0], [math.cos(1.0), math.sin(1.0)], atol=1e-15)


@pytest.mark.parametrize("dh,base", [(64, 1e4), (128, 5e5)])
def test_half_split_matches_transformers(dh, base):
    """Half-split RoPE equals Hugging Face Llama's apply_rotary_pos_emb (library routine)."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb

    cfg = LlamaConfig(hidden_size=dh * 4, num_attention_heads=4, head_dim=dh,
                      rope_parameters={"rope_type": "default", "rope_theta": base})
    hf_inv, _ = LlamaRotaryEmbedding.compute_default_rope_parameters(cfg)
    ours = rope.rope_inv_freq(dh, base)
    # transformers forms its frequencies in fp32
    assert np.allclose(hf_inv.double().numpy(), ours, rtol=2e-6, atol=0)

    pos = np.array([0, 1, 7, 1000, 70000])
    x = RNG.standard_normal((len(pos), 3, dh))
    freqs = np.outer(pos.astype(np.float64), ours)
    emb = np.concatenate([freqs, freqs], axis=-1)
    cos = torch.from_numpy(np.cos(emb))[None]  # [1][n][dh]
    sin = torch.from_numpy(np.sin(emb))[None]
    xt = torch.from_numpy(x.transpose(1, 0, 2).copy())[None]  # [1][heads][n][dh]
    hq, _ = apply_rotary_pos_emb(xt, xt, cos, sin, unsqueeze_dim=1)
    want = hq[0].numpy().transpose(1, 0, 2)
    got = rope.rotate(x, pos, ours, "rope_half")
    assert np.max(np.abs(got - want)) < 1e-12


def test_interleaved_is_permuted_half_split():
    """Interleaved pairing (2k, 2k+1) = half-split on channels permuted (2k -> k, 2k+1 -> k + dh/2)."""
    dh = 64
    inv = rope.rope_inv_freq(dh, 1e4)
    perm = np.concatenate([np.arange(0, dh, 2), np.arange(1, dh, 2)])  # half-split order of interleaved chans
    x = RNG.standard_normal((4, 2, dh))
    pos = np.array([0, 3, 99, 4096])
    inter = rope.rotate(x, pos, inv, "rope_interleaved")
    half = rope.rotate(x[..., perm], pos, inv, "rope_half")
    back = np.empty_like(half)
    back[..., perm] = half
    assert np.array_equal(inter, back)


def test_yarn_factor_one_is_rope():
    assert np.array_equal(rope.yarn_inv_freq(128, 5e5, 1.0, 8192), rope.rope_inv_freq(128, 5e5))
    assert rope.yarn_logit_gain(1.0) == 1.0


def test_yarn_regions_and_temperature():
    """High-frequency pairs keep theta, low-frequency pairs get theta / s, the ramp lies between;
    the temperature matches transformers' YaRN attention factor squared (library routine)."""
    dh, base, s, L = 128, 5e5, 8.0, 8192
    theta = rope.rope_inv_freq(dh, base)
    y = rope.yarn_inv_freq(dh, base, s, L)
    r = L * theta / (2 * math.pi)  # rotations over the original context
    assert np.array_equal(y[r >= 32], theta[r >= 32])
    assert np.allclose(y[r <= 1], theta[r <= 1] / s, rtol=1e-15)
    mid = (r > 1) & (r < 32)
    assert mid.any()
    assert np.all(y[mid] < theta[mid]) and np.all(y[mid] > theta[mid] / s)
    assert theta[0] == 1.0 and y[0] == 1.0

    from transformers import LlamaConfig
    from transformers.modeling_rope_utils import _compute_yarn_parameters

    cfg = LlamaConfig(hidden_size=dh * 8, num_attention_heads=8, head_dim=dh, max_position_embeddings=65536,
                      rope_parameters={"rope_type": "yarn", "rope_theta": base, "factor": s,
                                       "original_max_position_embeddings": L})
    hf_inv, attn_factor = _compute_yarn_parameters(cfg)
    assert abs(rope.yarn_logit_gain(s) - attn_factor ** 2) < 1e-12
    # transformers ramps over a truncated channel range; outside both ramps the two agree
    hf = hf_inv.double().numpy()
    outside = (r >= 64) | (r <= 0.5)
    assert np.allclose(hf[outside], y[outside], rtol=2e-6)


def test_alibi_slopes():
    """2^(-8 i / H): H = 8 gives the ALiBi paper's 1/2 .. 1/256; H = 71 ends at exactly 1/256."""
    assert np.array_equal(rope.alibi_slopes(8), 0.5 ** np.arange(1, 9))
    s71 = rope.alibi_slopes(71)
    assert s71[-1] == 1.0 / 256
    assert abs(s71[0] - 2 ** (-8 / 71)) < 1e-16
    assert np.all(np.diff(s71) < 0)


def _yarn_golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "yarn_ramp.txt")
    rows = []
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            k, th, thp = line.split()
            rows.append((int(k), float(th), float(thp)))
    return rows


def test_yarn_mid_ramp_hand_derived():
    """theta'_k inside the ramp equals values derived by hand from the YaRN paper's linear gamma(r)
    (tests/golden/yarn_ramp.txt): catches a ramp over channel index, a wrong denominator or a
    non-linear blend, none of which the end-region checks see."""
    dh, base, s, L = 128, 5e5, 8.0, 8192
    theta = rope.rope_inv_freq(dh, base)
    y = rope.yarn_inv_freq(dh, base, s, L)
    rows = _yarn_golden()
    assert len(rows) >= 3
    for k, th, thp in rows:
        assert abs(theta[k] - th) <= 1e-13 * th, (k, theta[k], th)
        assert abs(y[k] - thp) <= 1e-13 * thp, (k, y[k], thp)
    # the two regions the file's derivation names
    assert y[16] == theta[16] and abs(y[35] - theta[35] / 8) <= 1e-18
