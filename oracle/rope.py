"""Positional encodings, fp64 (oracle; test infrastructure only).

RoPE.  The LazyAttention notes (papernotes.org, "Background and motivation"
and "Key designs: Deferred Positional Encoding") rely on the RoPE identity
(R_m q)^T (R_n k) = q^T R_{n-m} k and write one rotation of a channel pair as
k1' = k1 cos(phi) - k2 sin(phi), k2' = k1 sin(phi) + k2 cos(phi).  The pages
give no frequency formula; the textbook RoFormer choice phi = pos * theta_k,
theta_k = base^(-2k/dh) is used.  The default channel pairing is (k, k + dh/2)
(the notes speak of rotating the "two halves" of a tile); the interleaved
variant pairs (2k, 2k+1) (notes, "Generality": interleaved RoPE changes
metadata only).

YaRN.  The notes ("Generality") say NTK/YaRN-scaled RoPE also changes only
metadata; they give no constants.  Frequencies follow the YaRN paper (Peng et
al., 2023): r_k = L_orig * theta_k / (2 pi), ramp gamma = clip((r_k - beta_slow)
/ (beta_fast - beta_slow), 0, 1), theta_k' = (1 - gamma) theta_k / s +
gamma theta_k, and a softmax temperature with sqrt(1/t) = 0.1 ln s + 1, i.e.
logits multiplied by (0.1 ln s + 1)^2.

ALiBi.  The notes ("Generality") apply the same deferral to ALiBi, a
score-space bias.  Slopes are 2^(-8 i / H) for i = 1..H (the workload's
explicit formula) and the bias added to a score is -slope * (m - n) for query
position m and key position n.
"""

from __future__ import annotations

import math

import numpy as np


def rope_inv_freq(head_dim: int, base: float) -> np.ndarray:
    """theta_k = base^(-2k/dh) for k = 0 .. dh/2 - 1 (fp64)."""
    k = np.arange(head_dim // 2, dtype=np.float64)
    return base ** (-2.0 * k / head_dim)


def yarn_inv_freq(head_dim: int, base: float, factor: float, orig_ctx: int,
                  beta_fast: float = 32.0, beta_slow: float = 1.0) -> np.ndarray:
    """YaRN-interpolated frequencies (YaRN paper's ramp over r = L_orig / wavelength)."""
    theta = rope_inv_freq(head_dim, base)
    if factor == 1.0:
        return theta
    r = orig_ctx * theta / (2.0 * math.pi)
    gamma = np.clip((r - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
    return (1.0 - gamma) * theta / factor + gamma * theta


def yarn_logit_gain(factor: float) -> float:
    """Multiplier on the logits from the YaRN temperature: (0.1 ln s + 1)^2 (1 for s <= 1)."""
    if factor <= 1.0:
        return 1.0
    return (0.1 * math.log(factor) + 1.0) ** 2


def alibi_slopes(num_heads: int) -> np.ndarray:
    """slope_h = 2^(-8 (h+1) / H), h = 0 .. H-1 (fp64)."""
    h = np.arange(1, num_heads + 1, dtype=np.float64)
    return 2.0 ** (-8.0 * h / num_heads)


def rotate(x: np.ndarray, pos: np.ndarray, inv_freq: np.ndarray, kind: str) -> np.ndarray:
    """Rotate x[..., n, heads, dh] eagerly at integer positions pos[n] (fp64 angles).

    kind "rope_half": pairs (k, k + dh/2); "rope_interleaved": pairs (2k, 2k+1).
    """
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.float64)
    phi = pos[:, None] * inv_freq[None, :]  # [n][dh/2]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    out = np.empty_like(x)
    half = x.shape[-1] // 2
    if kind == "rope_half":
        x1, x2 = x[..., :half], x[..., half:]
        out[..., :half] = x1 * c - x2 * s
        out[..., half:] = x1 * s + x2 * c
    elif kind == "rope_interleaved":
        x1, x2 = x[..., 0::2], x[..., 1::2]
        out[..., 0::2] = x1 * c - x2 * s
        out[..., 1::2] = x1 * s + x2 * c
    else:
        raise ValueError(f"rotate: not a rotary kind: {kind}")
    return out


def variant(pos_spec, head_dim: int, num_q_heads: int) -> dict:
    """Everything the eager attention needs from a positional spec (fp64)."""
    kind = pos_spec.kind
    scale = 1.0 / math.sqrt(head_dim)
    if kind == "alibi":
        return {"kind": kind, "scale": scale, "slopes": alibi_slopes(num_q_heads), "inv_freq": None}
    inv = yarn_inv_freq(head_dim, pos_spec.base, pos_spec.yarn_factor, pos_spec.yarn_orig_ctx,
                        pos_spec.yarn_beta_fast, pos_spec.yarn_beta_slow)
    return {"kind": kind, "scale": scale * yarn_logit_gain(pos_spec.yarn_factor),
            "slopes": None, "inv_freq": inv}
