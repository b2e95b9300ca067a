"""Oracle pin: the single-stream encoder (skvo_encode_tile) writes exactly the
stream that the whole-container encoder (skvo_encode, itself pinned by the
hand-computed encodings, the round trips and the entropy bound) writes for
the same inputs.

The stream of id s covers 32 consecutive channels (lanes) x 128 tokens
(steps) of one slab; in checkerboard mode the slab is the pass (even tokens,
then odd tokens, token = 2 * (128 * tb + k) + pass) and an odd token's mean
adds its two decoded even neighbours, the last odd token repeating its left
one (DCKV page, 'How it differs': the checkerboard context model).  The tiles
below are gathered here from that mapping, independently of the oracle's own
gather, for every stream of small multi-slab shapes: per-channel and
exponent-class tables on bf16 and e4m3, and the checkerboard mode; with
escapes, raw-fallback streams, odd-pass neighbours and the right edge.
"""
import numpy as np
import pytest

from workloads import gen

MASK = np.uint64((1 << 63) - 1)


def streams(container: bytes):
    n = int.from_bytes(container[32:40], "little")
    head = 64 + 8 * (n + 1)
    idx = np.frombuffer(container[64:head], dtype=np.uint64)
    out = []
    for s in range(n):
        a, b = int(idx[s] & MASK), int(idx[s + 1] & MASK)
        out.append((container[head + a:head + b], bool(int(idx[s]) >> 63)))
    return out


def plant(t, p, rng, mask, far, raw_blocks):
    """Escapes (residual `far` at 1/64 of the positions) and raw-fallback
    token blocks (uniform random values over whole (slab, token block)s)."""
    t = t.copy()
    flat = t.reshape(-1)
    pos = rng.choice(flat.size, size=flat.size // 64, replace=False)
    flat[pos] = ((p.reshape(-1)[pos].astype(np.int64) + far) & mask).astype(t.dtype)
    for (l, k, tb) in raw_blocks:
        blk = t[l, k, tb * 128:(tb + 1) * 128]
        blk[...] = rng.integers(0, mask + 1, size=blk.shape).astype(np.int64).astype(t.dtype)
    return t


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
@pytest.mark.parametrize("exp", [False, True])
def test_tile_equals_container_stream_residual(orc, dtype, exp):
    cid = 0 if dtype == "bf16" else 2
    L, KV, T, C = 2, 2, 384, 96
    cfg = gen.CONFIGS[cid].with_tokens(T, layers=L, channels=C)
    t, p = (a.numpy().copy() for a in gen.residual_array(cfg))
    ct, cp = (a.numpy().copy() for a in gen.residual_array(cfg, gen.CALIB, tokens=256))
    if dtype == "bf16":
        # slab (1, 1) scaled by 2^20 (exponent field + 20): its class base
        # differs from the other slabs', so a tile coded with another slab's
        # base would differ
        for a in (t, p, ct, cp):
            a[1, 1] = (a[1, 1].astype(np.int32) + (20 << 7)).astype(np.int16)
    rng = np.random.default_rng(5 + cid + 10 * exp)
    mask, far = (0xFFFF, 600) if dtype == "bf16" else (0xFF, 60)
    t = plant(t, p, rng, mask, far, [(0, 1, 2), (1, 0, 0)])
    odt = orc.BF16 if dtype == "bf16" else orc.E4M3
    mode = orc.RESIDUAL_EXP if exp else orc.RESIDUAL
    shape = orc.make_shape(odt, mode, L, KV, T, C)
    blob = orc.fit_tables(shape, ct, cp, 256)
    if exp and dtype == "bf16":
        bases = orc.blob_bases(blob)
        assert len(set(bases.tolist())) > 1, bases
    got = streams(orc.encode(blob, shape, t, p, threads=4))
    ntb, ncg = T // 128, C // 32
    assert len(got) == L * KV * ntb * ncg
    n_raw = n_coded = 0
    for s, (data, raw) in enumerate(got):
        cg, rest = s % ncg, s // ncg
        tb, slab = rest % ntb, rest // ntb
        l, k = divmod(slab, KV)
        tt = t[l, k, tb * 128:(tb + 1) * 128, cg * 32:(cg + 1) * 32]
        ta = p[l, k, tb * 128:(tb + 1) * 128, cg * 32:(cg + 1) * 32]
        if exp:
            lanes = np.full(32, slab, dtype=np.uint32)
        else:
            lanes = (slab * C + cg * 32 + np.arange(32)).astype(np.uint32)
        tile, tile_raw = orc.encode_tile(blob, shape, tt, ta, lanes)
        assert tile_raw == raw, s
        assert tile == data, s
        n_raw += raw
        n_coded += not raw
    # both planted raw blocks fall back whole; the rest is coded
    assert n_raw == 2 * ncg and n_coded == len(got) - n_raw


def test_tile_equals_container_stream_checkerboard(orc):
    T, C = 768, 64
    cfg = gen.CONFIGS[4].with_tokens(T, channels=C)
    coef, G = (a.numpy() for a in gen.dckv_draw(cfg))
    cc, cg_ = (a.numpy() for a in gen.dckv_draw(cfg, gen.CALIB, tokens=256))
    rng = np.random.default_rng(31)
    coef = coef.copy()
    # escapes on both passes, including the last odd token (right edge)
    pos = rng.choice(coef.size, size=coef.size // 50, replace=False)
    coef.reshape(-1)[pos] = rng.integers(-30000, 30000, size=pos.size).astype(np.int16)
    coef[T - 1, :] = 2000
    # a raw-fallback stream on each pass: token block 1 of channel group 0
    for ps in (0, 1):
        toks = 2 * (128 * 1 + np.arange(128)) + ps
        coef[toks, 0:32] = rng.integers(-32768, 32768, size=(128, 32)).astype(np.int16)
    shape = orc.make_shape(orc.INT16, orc.CHECKERBOARD, 1, 1, T, C)
    blob = orc.fit_tables(shape, cc, cg_, 256)
    got = streams(orc.encode(blob, shape, coef, G, threads=4))
    ntb, ncg = T // 2 // 128, C // 32
    assert len(got) == 2 * ntb * ncg
    n_raw = 0
    for s, (data, raw) in enumerate(got):
        cgi, rest = s % ncg, s // ncg
        tb, ps = rest % ntb, rest // ntb
        toks = 2 * (128 * tb + np.arange(128)) + ps
        cols = slice(cgi * 32, cgi * 32 + 32)
        nl = nr = None
        if ps == 1:
            nl = coef[toks - 1, cols]
            right = np.where(toks + 1 < T, toks + 1, toks - 1)
            nr = coef[right, cols]
        lanes = (cgi * 32 + np.arange(32)).astype(np.uint32)
        tile, tile_raw = orc.encode_tile(blob, shape, coef[toks, cols], G[toks, cols], lanes, nl, nr)
        assert tile_raw == raw, s
        assert tile == data, s
        n_raw += raw
    assert n_raw == 2


def test_tile_neighbours_matter(orc):
    """The odd pass really depends on the neighbours handed to the tile
    encoder: swapping in other neighbours changes the stream (so the
    comparison above would catch a wrong neighbour gather)."""
    T, C = 512, 32
    cfg = gen.CONFIGS[4].with_tokens(T, channels=C)
    coef, G = (a.numpy() for a in gen.dckv_draw(cfg))
    cc, cg_ = (a.numpy() for a in gen.dckv_draw(cfg, gen.CALIB, tokens=256))
    shape = orc.make_shape(orc.INT16, orc.CHECKERBOARD, 1, 1, T, C)
    blob = orc.fit_tables(shape, cc, cg_, 256)
    got = streams(orc.encode(blob, shape, coef, G, threads=2))
    toks = 2 * np.arange(128) + 1
    lanes = np.arange(32, dtype=np.uint32)
    right = np.where(toks + 1 < T, toks + 1, toks - 1)
    good, _ = orc.encode_tile(blob, shape, coef[toks], G[toks], lanes, coef[toks - 1], coef[right])
    assert good == got[2][0]          # pass 1, token block 0, group 0 is stream 2 (2 token blocks per pass)
    bad, _ = orc.encode_tile(blob, shape, coef[toks], G[toks], lanes, coef[toks - 1], coef[toks - 1])
    assert bad != good
