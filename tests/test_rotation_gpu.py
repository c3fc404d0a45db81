"""GPU: the rotation itself, element by element, at positions up to 2^17 - 1 (2^24 - 1 in-kernel).

Attention outputs are too forgiving to see a small angle error (a wrong
angle in one high-frequency pair moves a softmax-weighted average by far
less than the bf16 tolerance), so the rotation is checked where it is
applied: ``lazy_kv_write`` on fp32 keys and queries at positions spread over
[0, 131072) writes R_p k into the cache and R_p q in place, through the
fp64-built fp32 table and through the in-kernel sincos (fp64 angle with
exact reduction, fp32 sincos; also at positions up to 2^24 - 1, the largest
offset a tile word carries).  Both must match the oracle's fp64 rotation
to within fp32 rounding; an angle formed in fp32 (an error near 4e-3 rad at
p ~ 1.3e5 for the pair of frequency 1) would miss by three orders of
magnitude.  The V cache must hold v unrotated, in the channel-major layout.
"""

import numpy as np
import pytest
import torch

from oracle import rope as OR
from tests.harness import say
from workloads.gen import PosSpec

pytestmark = pytest.mark.gpu

MAX_POS = 1 << 17
LIMIT = 1 << 24  # positions a tile word's 24-bit offset field can hold
N = 4096  # tokens, one slot each


CASES = {
    "half_base1e4": PosSpec("rope_half", base=1e4),
    "interleaved_base1e4": PosSpec("rope_interleaved", base=1e4),
    "yarn8_base5e5": PosSpec("rope_half", base=5e5, yarn_factor=8.0, yarn_orig_ctx=8192),
}


@pytest.mark.parametrize("on_the_fly", [False, True], ids=["table", "on_the_fly"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_kv_write_rotation_at_large_positions(case, on_the_fly):
    from position_agnostic_paged_amd.engine import Engine, PosDesc

    spec = CASES[case]
    hq, hkv, dh = 2, 1, 128
    pos = PosDesc(spec.kind, dh, hq, "cuda", base=spec.base, yarn_factor=spec.yarn_factor,
                  yarn_orig_ctx=spec.yarn_orig_ctx, beta_fast=spec.yarn_beta_fast, beta_slow=spec.yarn_beta_slow,
                  max_pos=MAX_POS, on_the_fly=on_the_fly)
    eng = Engine(hq, hkv, dh, "fp32", pos, N // 16, "cuda")
    rng = np.random.default_rng(11)
    p = rng.choice(MAX_POS, size=N, replace=False).astype(np.int32)
    p[:4] = [0, 1, MAX_POS - 1, MAX_POS - 2]
    if on_the_fly:
        # no table bounds the in-kernel sincos: half the tokens go up to the largest offset a tile
        # word can carry (2^24 - 1), where the angle of the frequency-1 pair is ~1.7e7 rad
        far = rng.choice(np.arange(MAX_POS, LIMIT), size=N // 2, replace=False).astype(np.int32)
        p[N // 2:] = far
        p[-1] = LIMIT - 1
    k = rng.standard_normal((N, hkv, dh)).astype(np.float32) * 2.0
    v = rng.standard_normal((N, hkv, dh)).astype(np.float32)
    q = rng.standard_normal((N, hq, dh)).astype(np.float32)
    slots = rng.permutation(N).astype(np.int64)  # any slot order
    say(f"[rotation] {case} on_the_fly={on_the_fly}: {N} tokens at positions up to {p.max()}")

    qd = torch.from_numpy(q).cuda()
    eng.kv_write(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), qd, torch.from_numpy(p).cuda(),
                 torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    kc = eng.k_cache.cpu().numpy()  # [NB][Hkv][16][dh]
    vc = eng.v_cache.cpu().numpy()  # [NB][Hkv][dh][16]
    k_got = kc[slots // 16, :, slots % 16, :]
    v_got = vc[slots // 16, :, :, slots % 16]
    q_got = qd.cpu().numpy()

    var = OR.variant(spec, dh, hq)
    k_want = OR.rotate(k, p, var["inv_freq"], spec.kind)
    q_want = OR.rotate(q, p, var["inv_freq"], spec.kind)
    ek = float(np.max(np.abs(k_got - k_want)))
    eq = float(np.max(np.abs(q_got - q_want)))
    say(f"  max-abs err: k {ek:.2e} (|k| <= {np.abs(k).max():.1f}), q {eq:.2e} (|q| <= {np.abs(q).max():.1f})")
    # fp32 coefficients and fp32 arithmetic: a few ulps of |x1| + |x2| (<= ~20 here), i.e. ~1e-5 at
    # most; an angle formed in fp32 would be off by ~1e-2
    assert ek < 2e-5 and eq < 2e-5
    assert np.array_equal(v_got, v)
