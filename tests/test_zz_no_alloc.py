"""The no-allocation decode (lazy_attn_decode_noalloc, split partials in the library's static device
scratch) against lazy_attn_decode with a caller workspace, through the C ABI, on two calls in a row:

1. an uneven 48-request batch (64 query heads, 8 KV heads, 100 to 4000 tiles per request) whose default
   split plan needs more partial space than the scratch holds, so the call runs fewer, longer splits:
   same result within the bf16 parity bounds (the sums are split differently);
2. then a smaller batch whose plan fits: bit-identical to lazy_attn_decode (same plan, same kernels).
"""

import numpy as np
import pytest
import torch

from tests.harness import Gate, say

pytestmark = pytest.mark.gpu

HQ, HKV, DH, NB, MAX_POS = 64, 8, 128, 4096, 65536


def _setup():
    from position_agnostic_paged_amd import lazy_attn as L

    g = L.make_geom(HQ, HKV, DH, "bf16")
    inv, _ = L.rope_freqs(DH, 5e5)
    table = torch.from_numpy(L.rope_table(DH, inv, MAX_POS)).cuda()
    pos = L.PosDescC(L.LAZY_ROPE_HALF, 0, MAX_POS, L.softmax_scale(DH), table.data_ptr(), None, None)
    gen = torch.Generator(device="cuda").manual_seed(7)
    kc = (torch.randn((NB, HKV, 16, DH), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    vc = (torch.randn((NB, HKV, DH, 16), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    return L, g, pos, table, kc, vc


def _batch(L, rng, tiles_per_req):
    """Context tiles only: random blocks, each request's tiles in documents of 100 tiles with their own
    offsets (all below the table's rows)."""
    words, start, ctx = [], [0], []
    for n in tiles_per_req:
        blocks = rng.integers(0, NB, size=n)
        offs = (np.arange(n) // 100) * 1600
        words.append(L.pack_tiles(blocks, offs, np.full(n, 0xFFFF)))
        start.append(start[-1] + n)
        ctx.append(n)
    w = np.concatenate(words)
    return (torch.from_numpy(w.view(np.int64)).cuda(), torch.tensor(start, dtype=torch.int32, device="cuda"),
            torch.tensor(ctx, dtype=torch.int32, device="cuda"), int(max(tiles_per_req)), int(start[-1]))


def _both(L, g, pos, kc, vc, batch, R, gen):
    tiles, tstart, nctx, max_tiles, total = batch
    q = torch.randn((R, HQ, DH), generator=gen, device="cuda").to(torch.bfloat16)
    q_pos = torch.zeros(R, dtype=torch.int32, device="cuda")
    ws_bytes = L.workspace_size(g, R, 1, max_tiles, total, False)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    ref = torch.empty_like(q)
    L.attn_decode(g, pos, kc, vc, NB, tiles, tstart, nctx, q, q_pos, R, max_tiles, total, ref, ws)
    out = torch.full_like(q, float("nan"))
    L.attn_decode_noalloc(g, pos, kc, vc, NB, tiles, tstart, nctx, q, q_pos, R, max_tiles, total, out)
    torch.cuda.synchronize()
    return ws_bytes, ref.float().cpu().numpy(), out.float().cpu().numpy()


def test_noalloc_decode_matches_workspace_decode_two_calls():
    L, g, pos, table, kc, vc = _setup()
    rng = np.random.default_rng(11)
    gen = torch.Generator(device="cuda").manual_seed(8)

    lens = rng.integers(100, 4001, size=48)
    big = _batch(L, rng, lens)
    need, ref, out = _both(L, g, pos, kc, vc, big, 48, gen)
    say(f"[no-alloc decode] call 1: 48 requests, {big[4]} tiles, default plan needs {need / 2**20:.1f} MiB of "
        f"partials, static scratch {L.NOALLOC_SCRATCH_BYTES / 2**20:.0f} MiB")
    assert need > L.NOALLOC_SCRATCH_BYTES  # this call runs the capped plan
    gate = Gate("no-alloc decode, capped plan", "bf16")
    for r in range(48):
        gate.add(out[r], ref[r])
    gate.check(negative=False)  # both sides are the library; the offsets are exercised by the parity tests

    small = _batch(L, rng, rng.integers(40, 301, size=5))
    need2, ref2, out2 = _both(L, g, pos, kc, vc, small, 5, gen)
    say(f"[no-alloc decode] call 2: 5 requests, {small[4]} tiles, plan needs {need2 / 2**20:.2f} MiB: "
        f"identical plan")
    assert 0 < need2 <= L.NOALLOC_SCRATCH_BYTES
    assert np.array_equal(out2.view(np.uint32), ref2.view(np.uint32))
    del table
