"""One-copy step uploads: staged arrays arrive intact, a staged tile table equals
a directly uploaded one, and alternating pinned buffers never hand out data of
a previous step."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_step_uploads_round_trip_and_tile_table():
    from position_agnostic_paged_amd.engine import StepUploads, TileTable
    from position_agnostic_paged_amd.paging import RequestLayout, Segment
    from position_agnostic_paged_amd import lazy_attn as L

    rng = np.random.default_rng(7)
    up = StepUploads("cuda", capacity=1 << 20)
    layouts = [RequestLayout([Segment([3, 4, 5], 40, 0, True), Segment([9], 7, 40, False)]),
               RequestLayout([Segment([11, 12], 17, 0, False)])]
    for step in range(5):  # both pinned buffers, reused twice
        up.begin()
        a = rng.integers(-2**31, 2**31 - 1, size=1000 + step, dtype=np.int64).astype(np.int32)
        b = rng.integers(0, 2**62, size=333, dtype=np.int64)
        ia, ib = up.add(a), up.add(b)
        tt = TileTable(layouts, L.KIND_BY_NAME["rope_half"], 64, "cuda", up)
        views = up.commit()
        torch.cuda.synchronize()
        assert np.array_equal(views[ia].cpu().numpy(), a)
        assert np.array_equal(views[ib].cpu().numpy(), b)
        ref = TileTable(layouts, L.KIND_BY_NAME["rope_half"], 64, "cuda")
        for x, y in ((tt.tiles, ref.tiles), (tt.tile_start, ref.tile_start), (tt.ctx_tiles, ref.ctx_tiles)):
            assert torch.equal(x.cpu(), y.cpu())


def test_step_uploads_overlap_never_overwrites_a_buffer_in_use():
    """Commits back to back with no host synchronisation while the device
    lags behind (a spinning kernel before each read): every step's device
    views must still hold that step's data when its kernels run.  The copies
    are enqueued on the current stream, behind the earlier steps' kernels, and
    a pinned buffer is refilled only after its previous copy has executed."""
    from position_agnostic_paged_amd.engine import StepUploads

    rng = np.random.default_rng(5)
    up = StepUploads("cuda", capacity=1 << 20)
    want, got = [], []
    for step in range(8):
        up.begin()
        a = rng.integers(-2**31, 2**31 - 1, size=4096, dtype=np.int64).astype(np.int32)
        ia = up.add(a)
        views = up.commit()
        torch.cuda._sleep(2_000_000)  # the compute stream falls behind the copies
        got.append(views[ia].clone())  # read on the compute stream, in stream order
        want.append(a)
    torch.cuda.synchronize()
    for a, g in zip(want, got):
        assert np.array_equal(g.cpu().numpy(), a)
