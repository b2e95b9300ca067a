"""Oracle pins of the decoded-neighbour map (checkerboard mode with a
low-rank map over the decoded neighbours; DCKV page, 'How it differs': odd
positions are predicted from both decoded neighbours and their own token
embedding through a low-rank linear map).

The map is pinned by hand-computed cases (tests/golden/dckv_map_pins.json:
index conventions, right edge, saturation, rounding half up, both clamps),
by its reduction to a plain integer matrix product when no rounding or
clamping acts, and by its reduction to the plain checkerboard mode when U is
zero; the container codec of the mode by round trips, its dependence on the
map, and the single-stream encoder.
"""
import json
import os

import numpy as np
import pytest

from workloads import gen

HERE = os.path.dirname(os.path.abspath(__file__))
PINS = json.load(open(os.path.join(HERE, "golden", "dckv_map_pins.json")))


@pytest.mark.parametrize("case", PINS["cases"], ids=[c["name"][:2] for c in PINS["cases"]])
def test_map_hand_cases(orc, case):
    out = orc.dckv_map(np.array(case["coef"], np.int16), np.array(case["G"], np.int16),
                       np.array(case["V"], np.int8), np.array(case["U"], np.int8), case["sh1"], case["sh2"])
    assert out.tolist() == case["Gout"], case["note"]


def test_map_is_a_matrix_product_without_rounding(orc):
    """sh1 = sh2 = 0 and |V n| <= 127: the map is G + U (V n) exactly, with
    n the left row followed by the right row (the last odd token's right row
    is its left one); even rows are G."""
    rng = np.random.default_rng(3)
    T, C, k = 10, 24, 16
    coef = rng.integers(-2, 3, size=(T, C)).astype(np.int16)
    G = rng.integers(-1000, 1000, size=(T, C)).astype(np.int16)
    V = np.zeros((k, 2 * C), np.int8)
    for j in range(k):                                     # 8 entries of +-1 per row: |h| <= 16
        V[j, rng.choice(2 * C, 8, replace=False)] = rng.choice([-1, 1], 8)
    U = rng.integers(-3, 4, size=(C, k)).astype(np.int8)
    out = orc.dckv_map(coef, G, V, U, 0, 0)
    want = G.astype(np.int64).copy()
    for t in range(1, T, 2):
        right = coef[t + 1] if t + 1 < T else coef[t - 1]
        n = np.concatenate([coef[t - 1], right]).astype(np.int64)
        want[t] += U.astype(np.int64) @ (V.astype(np.int64) @ n)
    assert np.array_equal(out, want.astype(np.int16))
    # a swapped neighbour order gives a different result (the pin sees the order)
    Vs = np.concatenate([V[:, C:], V[:, :C]], axis=1)
    assert not np.array_equal(orc.dckv_map(coef, G, Vs, U, 0, 0), out)


def _map_case(orc, T=768, C=64, rank=16, u_zero=False):
    cfg = gen.CONFIGS[4].with_tokens(T, channels=C)
    V, U, sh1, sh2 = gen.dckv_map_weights(cfg, rank)
    if u_zero:
        U = np.zeros_like(U)
    coef, G = (a.numpy() for a in gen.dckv_draw(cfg, nbr_map=(V, U, sh1, sh2)))
    cc, cg = (a.numpy() for a in gen.dckv_draw(cfg, gen.CALIB, tokens=256, nbr_map=(V, U, sh1, sh2)))
    shape = orc.make_shape(orc.INT16, orc.CHECKERBOARD_MAP, 1, 1, T, C)
    blob = orc.fit_tables_map(shape, cc, cg, 256, V, U, sh1, sh2)
    return cfg, coef, G, cc, cg, V, U, sh1, sh2, shape, blob


def test_map_zero_reduces_to_checkerboard(orc):
    """U = 0: the side input is unchanged, the tables equal the plain
    checkerboard mode's, and so do the index and every stream."""
    cfg, coef, G, cc, cg, V, U, sh1, sh2, shape, blob = _map_case(orc, u_zero=True)
    assert np.array_equal(orc.dckv_map(coef, G, V, U, sh1, sh2), G)
    s1 = orc.make_shape(orc.INT16, orc.CHECKERBOARD, 1, 1, cfg.tokens, cfg.channels)
    blob1 = orc.fit_tables(s1, cc, cg, 256)
    n_rec = 64 + 514 * 16 * cfg.channels
    # the header differs in the mode byte and the total size (the map section follows the records)
    assert blob[8:32] == blob1[8:32] and blob[40:n_rec] == blob1[40:n_rec] and blob[7] == orc.CHECKERBOARD_MAP
    c3 = orc.encode(blob, shape, coef, G, threads=4)
    c1 = orc.encode(blob1, s1, coef, G, threads=4)
    assert c3[64:] == c1[64:] and c3[7] == orc.CHECKERBOARD_MAP and c1[7] == orc.CHECKERBOARD


def test_map_mode_round_trip_and_dependence(orc):
    cfg, coef, G, cc, cg, V, U, sh1, sh2, shape, blob = _map_case(orc)
    c = orc.encode(blob, shape, coef, G, threads=4)
    back = orc.decode(blob, c, G, coef, threads=4)
    assert np.array_equal(back, coef)
    # a different map (other U) codes the odd pass differently
    U2 = U.copy()
    U2[0, 0] = U2[0, 0] // 2 + 1
    blob2 = orc.fit_tables_map(shape, cc, cg, 256, V, U2, sh1, sh2)
    c2 = orc.encode(blob2, shape, coef, G, threads=4)
    assert c2 != c
    assert np.array_equal(orc.decode(blob2, c2, G, coef, threads=4), coef)
    # the plain checkerboard tables code the same data in more bytes: the map
    # explains part of the odd tokens' means
    s1 = orc.make_shape(orc.INT16, orc.CHECKERBOARD, 1, 1, cfg.tokens, cfg.channels)
    c1 = orc.encode(orc.fit_tables(s1, cc, cg, 256), s1, coef, G, threads=4)
    assert len(c) < len(c1)


def test_map_mode_tiles_equal_container_streams(orc):
    """Every stream of a map-mode container equals the single-stream encoder's
    output with the side input G' (the map of the true even rows)."""
    cfg, coef, G, cc, cg, V, U, sh1, sh2, shape, blob = _map_case(orc, T=512, C=64)
    Gm = orc.dckv_map(coef, G, V, U, sh1, sh2)
    c = orc.encode(blob, shape, coef, G, threads=2)
    n = int.from_bytes(c[32:40], "little")
    head = 64 + 8 * (n + 1)
    idx = np.frombuffer(c[64:head], dtype=np.uint64) & np.uint64((1 << 63) - 1)
    T, C = cfg.tokens, cfg.channels
    ntb, ncg = T // 2 // 128, C // 32
    for s in range(n):
        cgi, rest = s % ncg, s // ncg
        tb, ps = rest % ntb, rest // ntb
        toks = 2 * (128 * tb + np.arange(128)) + ps
        cols = slice(cgi * 32, cgi * 32 + 32)
        nl = nr = None
        if ps == 1:
            nl = coef[toks - 1, cols]
            nr = coef[np.where(toks + 1 < T, toks + 1, toks - 1), cols]
        tile, _ = orc.encode_tile(blob, shape, coef[toks, cols], Gm[toks, cols],
                                  (cgi * 32 + np.arange(32)).astype(np.uint32), nl, nr)
        assert tile == c[head + int(idx[s]):head + int(idx[s + 1])], s


def test_map_blob_checks(orc):
    """The plain fit refuses the map mode; the map fit refuses ranks the
    blob cannot hold (not a power of two from 16 to 256)."""
    cfg = gen.CONFIGS[4].with_tokens(512, channels=32)
    cc, cg = (a.numpy() for a in gen.dckv_draw(cfg, gen.CALIB, tokens=256))
    shape = orc.make_shape(orc.INT16, orc.CHECKERBOARD_MAP, 1, 1, 512, 32)
    with pytest.raises(RuntimeError):
        orc.fit_tables(shape, cc, cg, 256)
    for k in (8, 24, 48, 512):
        with pytest.raises(RuntimeError):
            orc.fit_tables_map(shape, cc, cg, 256, np.zeros((k, 64), np.int8), np.zeros((32, k), np.int8), 0, 0)
