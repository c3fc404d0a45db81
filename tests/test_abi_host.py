"""CPU tests of the C ABI: the library loads, exports what include/lazy_attn.h declares, and its
host-side calls (packer, tile builder, RoPE/YaRN/ALiBi metadata, validation) agree with the oracle
bit for bit where the result is integer and to fp32 rounding where it is floating point.
No device work runs here."""

import ctypes as C
import math
import os
import re

import numpy as np
import pytest

from oracle import pack as OP
from oracle import rope as OR

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from position_agnostic_paged_amd import lazy_attn

    lazy_attn.lib()  # fails loudly when the library is not built
    return lazy_attn


def test_exports_every_declared_symbol(L):
    hdr = open(os.path.join(ROOT, "include", "lazy_attn.h")).read()
    declared = sorted(set(re.findall(r"\b(lazy_[a-z_]+)\s*\(", hdr)))
    assert declared, "no declarations found"
    lib = C.CDLL(L.LIB_PATH)
    missing = [s for s in declared if not hasattr(lib, s)]
    assert not missing, missing
    assert sorted(L.EXPORTED) == declared


def test_pack_golden_and_boundaries(L):
    rows = [ln.split() for ln in open(os.path.join(ROOT, "tests", "golden", "pack_words.txt"))
            if ln.strip() and not ln.startswith("#")]
    b = [int(r[0]) for r in rows]
    o = [int(r[1]) for r in rows]
    m = [int(r[2]) for r in rows]
    words = L.pack_tiles(b, o, m)
    assert [int(w) for w in words] == [int(r[3], 16) for r in rows]
    bb, oo, mm = L.unpack_tiles(words)
    assert list(bb) == b and list(oo) == o and list(mm) == m


def test_pack_random_words_match_oracle(L):
    rng = np.random.default_rng(11)
    n = 1_000_000
    b = rng.integers(0, 1 << 24, size=n)
    o = rng.integers(0, 1 << 24, size=n)
    m = rng.integers(1, 1 << 16, size=n)
    words = L.pack_tiles(b, o, m)
    for i in rng.choice(n, size=20000, replace=False):  # oracle is scalar Python: check a large sample
        assert int(words[i]) == OP.pack(int(b[i]), int(o[i]), int(m[i]))
    bb, oo, mm = L.unpack_tiles(words)  # full round trip
    assert np.array_equal(bb, b) and np.array_equal(oo, o) and np.array_equal(mm, m)


@pytest.mark.parametrize("args", [((1 << 24,), (0,), (1,)), ((0,), (1 << 24,), (1,)), ((0,), (0,), (0,)),
                                  ((0,), (0,), (1 << 16,)), ((-1,), (0,), (1,))])
def test_pack_rejects_out_of_field(L, args):
    with pytest.raises(L.LazyError) as e:
        L.pack_tiles(*args)
    assert e.value.status == L.LAZY_ERR_ARG
    assert "tile 0" in L.last_error()


def _golden_request():
    rows = [ln.split() for ln in open(os.path.join(ROOT, "tests", "golden", "request_tiles.txt"))
            if ln.strip() and not ln.startswith("#")]
    segs = []
    for spec in rows[0][1:]:
        blocks, ln, p0, ctx = spec.split(";")
        segs.append({"blocks": [int(x) for x in blocks.split(",")], "len": int(ln), "pos0": int(p0), "ctx": ctx == "1"})
    return segs, rows[1:]


def _build(L, kind, reqs, num_blocks=1 << 20, max_pos=0):
    seg_start, seg_len, seg_pos0, seg_ctx, seg_bs, blocks = [0], [], [], [], [0], []
    for segs in reqs:
        for s in segs:
            seg_len.append(s["len"])
            seg_pos0.append(s["pos0"])
            seg_ctx.append(1 if s["ctx"] else 0)
            blocks.extend(s["blocks"])
            seg_bs.append(len(blocks))
        seg_start.append(len(seg_len))
    return L.build_tiles(kind, seg_start, seg_len, seg_pos0, seg_ctx, seg_bs, blocks or [0], num_blocks,
                         max(1, len(blocks)), max_pos)


def test_build_tiles_golden(L):
    segs, expected = _golden_request()
    for row in expected:
        kind = L.KIND_BY_NAME[row[0]]
        tiles, tstart, nctx = _build(L, kind, [segs])
        assert [int(w) for w in tiles] == [int(w, 16) for w in row[2:]]
        assert list(tstart) == [0, len(row) - 2] and list(nctx) == [int(row[1])]


@pytest.mark.parametrize("kind", ["rope_half", "rope_interleaved", "alibi"])
def test_build_tiles_random_match_oracle(L, kind):
    rng = np.random.default_rng(17)
    reqs = []
    next_block = 0
    for _ in range(30):
        segs, pos = [], 0
        for _ in range(int(rng.integers(0, 6))):
            n = int(rng.integers(1, 90))
            nb = (n + 15) // 16
            segs.append({"blocks": list(range(next_block, next_block + nb)), "len": n, "pos0": pos, "ctx": True})
            next_block += nb
            pos += n
        n = int(rng.integers(0, 40))
        nb = (n + 15) // 16
        segs.append({"blocks": list(range(next_block, next_block + nb)), "len": n, "pos0": pos, "ctx": False})
        next_block += nb
        reqs.append(segs)
    tiles, tstart, nctx = _build(L, L.KIND_BY_NAME[kind], reqs)
    for r, segs in enumerate(reqs):
        want, want_ctx = OP.request_tiles(segs, kind)
        assert [int(w) for w in tiles[tstart[r]: tstart[r + 1]]] == want
        assert nctx[r] == want_ctx


def test_build_tiles_rejects_bad_layouts(L):
    ok = {"blocks": [0], "len": 5, "pos0": 0, "ctx": True}
    priv = {"blocks": [1], "len": 3, "pos0": 5, "ctx": False}
    with pytest.raises(L.LazyError):  # context after private
        _build(L, 0, [[priv, ok]])
    with pytest.raises(L.LazyError):  # block beyond the pool
        _build(L, 0, [[{"blocks": [9], "len": 5, "pos0": 0, "ctx": True}]], num_blocks=4)
    with pytest.raises(L.LazyError):  # not enough blocks for the tokens
        _build(L, 0, [[{"blocks": [0], "len": 17, "pos0": 0, "ctx": True}]])
    with pytest.raises(L.LazyError):  # offset beyond 24 bits
        _build(L, 2, [[{"blocks": [0], "len": 5, "pos0": 1 << 24, "ctx": True}]])


def test_build_tiles_checks_offsets_against_the_table(L):
    """A rotary document offset must address a row of the cos/sin table the kernels read; private tiles
    and ALiBi offsets are never table rows."""
    doc = {"blocks": [0, 1], "len": 20, "pos0": 100, "ctx": True}
    priv = {"blocks": [2], "len": 3, "pos0": 120, "ctx": False}
    _build(L, 0, [[doc, priv]], max_pos=101)  # Delta = 100 < 101
    with pytest.raises(L.LazyError, match="cos/sin table"):
        _build(L, 0, [[doc, priv]], max_pos=100)
    with pytest.raises(L.LazyError, match="cos/sin table"):
        _build(L, 1, [[doc, priv]], max_pos=50)
    _build(L, 2, [[doc, priv]], max_pos=50)  # ALiBi: no table row is read
    _build(L, 0, [[{"blocks": [0], "len": 3, "pos0": 500, "ctx": False}]], max_pos=10)  # private tile
    _build(L, 0, [[doc, priv]], max_pos=0)  # 0: no table (in-kernel sincos)


def test_softmax_scale_matches_oracle(L):
    """The logit multiplier the library hands the kernels: 1/sqrt(dh), times the YaRN gain."""
    from workloads.gen import PosSpec

    for dh, s in ((64, 1.0), (128, 1.0), (128, 8.0), (128, 4.0)):
        spec = PosSpec("rope_half", base=5e5, yarn_factor=s, yarn_orig_ctx=8192 if s > 1 else 0)
        want = OR.variant(spec, dh, 8)["scale"]
        assert L.softmax_scale(dh, s) == pytest.approx(want, rel=1e-7)
    assert L.softmax_scale(64, 1.0) == np.float32(0.125)


def test_engine_validates_kv_write_positions_and_slots():
    """Positions outside the cos/sin table and slots outside the pool are refused on the host, before any
    launch (the library sees them only on the device)."""
    from position_agnostic_paged_amd.engine import Engine, PosDesc

    pos = PosDesc("rope_half", 64, 4, "cpu", base=1e4, max_pos=100)
    eng = Engine(4, 1, 64, "fp32", pos, 8, "cpu")
    eng.check_write(np.array([0, 99]), np.array([0, 127]))
    with pytest.raises(ValueError, match="rotation positions"):
        eng.check_write(np.array([0, 100]), np.array([0, 1]))
    with pytest.raises(ValueError, match="rotation positions"):
        eng.check_write(np.array([-1]), np.array([0]))
    with pytest.raises(ValueError, match="outside the pool"):
        eng.check_write(np.array([0]), np.array([128]))
    alibi = Engine(4, 1, 64, "fp32", PosDesc("alibi", 64, 4, "cpu"), 8, "cpu")
    alibi.check_write(np.array([10_000]), np.array([5]))  # ALiBi keys are not rotated
    fly = Engine(4, 1, 64, "fp32", PosDesc("rope_half", 64, 4, "cpu", base=1e4, on_the_fly=True), 8, "cpu")
    fly.check_write(np.array([(1 << 24) - 1]), np.array([0]))


@pytest.mark.parametrize("dh,base,s", [(64, 1e4, 1.0), (128, 5e5, 1.0), (128, 5e5, 8.0)])
def test_rope_freqs_and_table_match_oracle(L, dh, base, s):
    inv, gain = L.rope_freqs(dh, base, s, 8192 if s > 1 else 0)
    want = OR.yarn_inv_freq(dh, base, s, 8192) if s > 1 else OR.rope_inv_freq(dh, base)
    assert np.allclose(inv, want, rtol=1e-14, atol=0)
    assert gain == pytest.approx(OR.yarn_logit_gain(s), rel=1e-14)
    pos = np.array([0, 1, 2, 777, 32063, 65599])
    tab = L.rope_table(dh, inv, 65600)
    phi = pos[:, None] * want[None, :]
    # table = fp64 cos/sin rounded once to fp32
    assert np.max(np.abs(tab[pos, : dh // 2] - np.cos(phi))) <= 6e-8
    assert np.max(np.abs(tab[pos, dh // 2:] - np.sin(phi))) <= 6e-8


def test_alibi_slopes_match_oracle(L):
    for h in (8, 71):
        assert np.array_equal(L.alibi_slopes(h), OR.alibi_slopes(h).astype(np.float32))


def test_device_calls_validate_before_launch(L):
    """Argument errors come back as statuses without touching the GPU (runs on CPU-only hosts)."""
    g = L.make_geom(32, 8, 128, "bf16")
    p = L.PosDescC(0, 0, 10, 0.1, 1, None, None)  # non-null fake table pointer; never dereferenced
    lib = L.lib()
    fake = C.c_void_p(16)

    def prefill(geom, pos, nb=10, nreq=1, maxq=4):
        return lib.lazy_attn_prefill(C.byref(geom), C.byref(pos), fake, fake, nb, fake, fake, fake, fake, fake, fake,
                                     nreq, maxq, 512, 0, fake, None, 0, None)

    assert prefill(L.make_geom(30, 8, 128, "bf16"), p) == L.LAZY_ERR_ARG  # Hq % Hkv
    assert prefill(L.make_geom(32, 8, 96, "bf16"), p) == L.LAZY_ERR_UNSUPPORTED  # head_dim
    bad_bs = L.make_geom(32, 8, 128, "bf16")
    bad_bs.block_size = 32
    assert prefill(bad_bs, p) == L.LAZY_ERR_UNSUPPORTED
    assert prefill(g, p, nb=0) == L.LAZY_ERR_ARG
    assert prefill(g, L.PosDescC(7, 0, 10, 0.1, 1, None, None)) == L.LAZY_ERR_ARG  # kind
    assert prefill(g, L.PosDescC(0, 0, 10, -1.0, 1, None, None)) == L.LAZY_ERR_ARG  # scale
    assert prefill(g, L.PosDescC(2, 0, 10, 0.1, None, None, None)) == L.LAZY_ERR_ARG  # ALiBi without slopes
    assert prefill(g, L.PosDescC(0, 0, 10, 0.1, None, None, None)) == L.LAZY_ERR_ARG  # RoPE without coefficients
    assert prefill(g, L.PosDescC(0, 4, 10, 0.1, 1, None, None)) == L.LAZY_ERR_ARG  # unknown flag
    # a split plan needs a workspace: none given
    assert L.workspace_size(g, 1, 4, 512, 0, True) > 0
    assert prefill(g, p) == L.LAZY_ERR_WORKSPACE
    assert "workspace" in L.last_error()
    # decode with too small a workspace
    assert lib.lazy_attn_decode(C.byref(g), C.byref(p), fake, fake, 10, fake, fake, fake, fake, fake, 64, 2048, 0,
                                fake, fake, 16, None) == L.LAZY_ERR_WORKSPACE
    # kv write: negative count, empty is a no-op
    assert lib.lazy_kv_write(C.byref(g), C.byref(p), fake, fake, 10, fake, fake, None, fake, fake, -1,
                             None) == L.LAZY_ERR_ARG
    assert lib.lazy_kv_write(C.byref(g), C.byref(p), fake, fake, 10, fake, fake, None, fake, fake, 0, None) == L.LAZY_OK
    assert lib.lazy_debug_unpack(None, -1, None, None, None, None) == L.LAZY_ERR_ARG
    # the no-allocation decode: same argument checks, an empty batch is a no-op, and a batch whose
    # partials cannot fit the static scratch even at two splits is refused before any device call
    def noalloc(geom, pos, nreq, max_tiles, total):
        return lib.lazy_attn_decode_noalloc(C.byref(geom), C.byref(pos), fake, fake, 10, fake, fake, fake, fake,
                                            fake, nreq, max_tiles, total, fake, None)

    assert noalloc(L.make_geom(30, 8, 128, "bf16"), p, 4, 64, 0) == L.LAZY_ERR_ARG
    assert noalloc(g, L.PosDescC(0, 0, 10, -1.0, 1, None, None), 4, 64, 0) == L.LAZY_ERR_ARG
    assert noalloc(g, p, 0, 64, 0) == L.LAZY_OK
    assert noalloc(g, p, 4096, 20000, 4096 * 100) == L.LAZY_ERR_WORKSPACE
    assert "static scratch" in L.last_error()


def test_paired_tiles_keep_each_pair_in_one_document():
    """lazy_build_tiles_paired: the plain list with one empty tile (mask 0) after every context segment of an
    odd tile count, so each pair (2i, 2i+1) of a request lies within one document or within its private
    tokens; ctx_tiles counts the empty tiles."""
    import numpy as np

    from position_agnostic_paged_amd import lazy_attn as LA

    rng = np.random.default_rng(5)
    for kind in (0, 1, 2):
        seg_start, seg_len, seg_pos0, seg_ctx, seg_bs, blocks = [0], [], [], [], [0], []
        nb = 0
        for r in range(6):
            pos = 0
            for d in range(int(rng.integers(0, 5))):
                n = int(rng.integers(1, 70))
                seg_len.append(n); seg_pos0.append(pos); seg_ctx.append(1)
                blocks += list(range(nb, nb + (n + 15) // 16)); nb += (n + 15) // 16; seg_bs.append(len(blocks))
                pos += n
            n = int(rng.integers(0, 40))
            seg_len.append(n); seg_pos0.append(pos); seg_ctx.append(0)
            blocks += list(range(nb, nb + (n + 15) // 16)); nb += (n + 15) // 16; seg_bs.append(len(blocks))
            seg_start.append(len(seg_len))
        args = (seg_start, seg_len, seg_pos0, seg_ctx, seg_bs, blocks or [0], max(nb, 1))
        plain, ps, pc = LA.build_tiles(kind, *args)
        paired, qs, qc = LA.build_tiles(kind, *args, paired=True)
        b, o, m = LA.unpack_tiles(paired)
        for r in range(6):
            segs = range(seg_start[r], seg_start[r + 1])
            want = []
            for s in segs:
                nt = (seg_len[s] + 15) // 16
                want += [int(w) for w in plain[ps[r] + sum((seg_len[t] + 15) // 16 for t in segs if t < s):][:nt]]
                if seg_ctx[s] and nt % 2:
                    off = seg_pos0[s] if kind != 2 else seg_pos0[s] + 16 * nt
                    want.append(off << 16)  # block 0, mask 0
            assert [int(w) for w in paired[qs[r]: qs[r + 1]]] == want
            nctx = sum((seg_len[s] + 15) // 16 + ((seg_len[s] + 15) // 16) % 2 for s in segs if seg_ctx[s])
            assert qc[r] == nctx and nctx % 2 == 0
