"""Oracle container: layout, stream mapping, raw fallback, round trips,
corruption detection and the entropy bound.

The container carries the residual of the target cache against the
predictor's cache, coded losslessly (Speculative KV coding summary, 'Core
idea'); checkerboard mode codes even tokens, then odd tokens conditioned on
their decoded neighbours (DCKV page, 'How it differs').
"""
import math
import struct

import numpy as np
import pytest

from workloads import gen


def manual_blob(orc, dtype, mode, layers, kv, channels, tables):
    """Build a blob from explicit (n, freq) tables in the documented layout."""
    nt = len(tables)
    head = bytearray(64)
    head[0:4] = b"SKVT"
    struct.pack_into("<HBBIIII", head, 4, 1, dtype, mode, nt, layers, kv, channels)
    total = 64 + 514 * nt
    struct.pack_into("<Q", head, 32, total)
    body = bytearray()
    for n, f in tables:
        rec = np.zeros(257, dtype=np.uint16)
        rec[0] = n
        rec[1:n + 2] = f
        body += rec.tobytes()
    return bytes(head + body)


def parse(container):
    h = container[:64]
    n = struct.unpack_from("<Q", h, 32)[0]
    idx = np.frombuffer(container[64:64 + 8 * (n + 1)], dtype=np.uint64)
    pay = container[64 + 8 * (n + 1):]
    return h, n, idx, pay


def stream_bytes(idx, pay, s):
    mask = np.uint64((1 << 63) - 1)
    a, b = int(idx[s] & mask), int(idx[s + 1] & mask)
    return pay[a:b], bool(int(idx[s]) >> 63)


@pytest.fixture(scope="module")
def cfg0(orc):
    cfg = gen.CONFIGS[0]
    t, p = gen.residual_array(cfg)
    ct, cp = gen.residual_array(cfg, gen.CALIB, tokens=256)
    shape = orc.make_shape(orc.BF16, orc.RESIDUAL, 1, 2, 1024, 1024)
    blob = orc.fit_tables(shape, ct.numpy(), cp.numpy(), 256)
    return shape, blob, t.numpy(), p.numpy()


def test_header_and_index(orc, cfg0):
    shape, blob, t, p = cfg0
    c = orc.encode(blob, shape, t, p, threads=4)
    h, n, idx, pay = parse(c)
    assert h[:4] == b"SKV1"
    ver, dt, mode, pb, lanes, steps = struct.unpack_from("<HBBBBH", h, 4)
    assert (ver, dt, mode, pb, lanes, steps) == (1, 1, 0, 12, 32, 128)
    assert struct.unpack_from("<IIII", h, 12) == (1, 2, 1024, 1024)
    assert n == 2 * (1024 // 128) * (1024 // 32) == 512
    assert struct.unpack_from("<Q", h, 40)[0] == orc.fnv1a64(blob)
    assert struct.unpack_from("<Q", h, 48)[0] == len(pay) == int(idx[-1])
    offs = idx & np.uint64((1 << 63) - 1)
    assert offs[0] == 0 and np.all(np.diff(offs.astype(np.int64)) > 0)
    assert np.all(offs % 4 == 0)


def test_impulse_maps_to_stream_lane_step(orc):
    """One element differs from the predictor: exactly one stream carries a
    non-zero symbol, at the (step, lane) that the layout assigns."""
    layers, kv, T, C = 2, 2, 256, 64
    tab = (3, [4000, 40, 40, 16])
    blob = manual_blob(orc, 1, 0, layers, kv, C, [tab] * (layers * kv * C))
    shape = orc.make_shape(orc.BF16, orc.RESIDUAL, layers, kv, T, C)
    p = np.full((layers, kv, T, C), 0x3F80, dtype=np.uint16)
    t = p.copy()
    L, K, tok, ch = 1, 0, 200, 37
    t[L, K, tok, ch] = 0x3F81            # one ulp above: r = +1 -> z = 2
    c = orc.encode(blob, shape, t, p)
    _, n, idx, pay = parse(c)
    ncg, ntb = C // 32, T // 128
    want = ((L * kv + K) * ntb + tok // 128) * ncg + ch // 32
    for s in range(n):
        data, raw = stream_bytes(idx, pay, s)
        assert not raw
        rc, z = orc.stream_decode(data, np.zeros(4096, np.uint32), [tab], 128, 2)
        assert rc == 0
        nz = np.nonzero(z)[0]
        if s == want:
            assert list(nz) == [(tok % 128) * 32 + ch % 32] and z[nz[0]] == 2
        else:
            assert len(nz) == 0


def test_checkerboard_impulse_and_neighbours(orc):
    """Checkerboard: pass 0 streams carry even tokens, pass 1 odd ones, and an
    even coefficient moves the mean of both odd neighbours by 8*value
    sixteenths (choosing another shifted table)."""
    T, C = 512, 32
    # table f: direct 0..2; use a distinct n per shift so the choice is visible
    tables = []
    for comp in range(C):
        for f in range(16):
            tables.append((1 + f % 3, [4000] + [32] * (f % 3) + [4096 - 4000 - 32 * (f % 3)]))
    blob = manual_blob(orc, 3, 1, 1, 1, C, tables)
    shape = orc.make_shape(orc.INT16, orc.CHECKERBOARD, 1, 1, T, C)
    G = np.zeros((T, C), dtype=np.int16)
    coef = np.zeros((T, C), dtype=np.int16)
    coef[300, 5] = 1                     # even token 300 -> means of tokens 299, 301 grow by 8
    out = orc.encode(blob, shape, coef, G)
    back = orc.decode(blob, out, G, coef)
    assert np.array_equal(back, coef)
    _, n, idx, pay = parse(out)
    assert n == 2 * (T // 2 // 128) * (C // 32)
    ntb = T // 2 // 128
    # even pass: token 300 = 2 * 150 -> tb 1, step 22, lane 5
    data, raw = stream_bytes(idx, pay, 0 * ntb + 1)
    tab_of = np.zeros(4096, np.uint32)    # every even position uses f = 0 here (G = 0)
    rc, z = orc.stream_decode(data, tab_of, [tables[5 * 16 + 0]], 128, 2)
    assert rc == 0 and list(np.nonzero(z)[0]) == [22 * 32 + 5] and z[22 * 32 + 5] == 2
    # odd pass: tokens 299 (j=149) and 301 (j=150) see mean 8 -> k=0, f=8
    data, raw = stream_bytes(idx, pay, ntb + 1)
    tab_list = [tables[(i % 32) * 16] for i in range(32)] + [tables[5 * 16 + 8]]
    tab_of = np.array([i % 32 for i in range(4096)], np.uint32)
    tab_of[21 * 32 + 5] = 32
    tab_of[22 * 32 + 5] = 32
    rc, z = orc.stream_decode(data, tab_of, tab_list, 128, 2)
    assert rc == 0 and not z.any()


def test_raw_fallback_stores_target_tile(orc):
    layers, kv, T, C = 1, 1, 256, 32
    tab = (1, [4095, 1])                 # everything but zero escapes at ~12 bits
    blob = manual_blob(orc, 1, 0, layers, kv, C, [tab] * C)
    shape = orc.make_shape(orc.BF16, orc.RESIDUAL, layers, kv, T, C)
    rng = np.random.default_rng(5)
    t = rng.integers(0, 65536, size=(1, 1, T, C), dtype=np.uint16)
    p = t.copy()
    p[0, 0, :128] ^= rng.integers(1, 65536, size=(128, C), dtype=np.uint16)   # block 0 incompressible
    c = orc.encode(blob, shape, t, p)
    _, n, idx, pay = parse(c)
    d0, raw0 = stream_bytes(idx, pay, 0)
    d1, raw1 = stream_bytes(idx, pay, 1)
    assert raw0 and len(d0) == 8192
    assert np.array_equal(np.frombuffer(d0, np.uint16).reshape(128, 32), t[0, 0, :128])
    assert not raw1 and len(d1) < 8192
    assert np.array_equal(orc.decode(blob, c, p, t), t)


@pytest.mark.parametrize("kind", ["equal", "random", "maxz", "cfg0"])
def test_roundtrip_edge_cases_bf16(orc, cfg0, kind):
    shape, blob, t, p = cfg0
    rng = np.random.default_rng(11)
    if kind == "equal":
        t = p.copy()
    elif kind == "random":
        t = rng.integers(0, 65536, size=p.shape, dtype=np.uint16).view(np.int16)
    elif kind == "maxz":
        # r = -32768 everywhere -> z = 65535, the largest escape value
        o = np.array([orc.ord_(int(x), 16) for x in range(65536)], dtype=np.uint32)
        inv = np.empty(65536, np.uint16)
        inv[o] = np.arange(65536, dtype=np.uint16)
        po = o[p.view(np.uint16)]
        t = inv[(po + 32768) % 65536].view(np.int16)
    c = orc.encode(blob, shape, t, p, threads=4)
    assert np.array_equal(orc.decode(blob, c, p, t, threads=4), t)
    if kind == "equal":
        assert len(c) < t.nbytes / 3          # z = 0 is the most likely symbol of every table


def test_roundtrip_e4m3_and_checkerboard(orc):
    cfg = gen.CONFIGS[2].with_tokens(512, layers=2)
    t, p = gen.residual_array(cfg)
    ct, cp = gen.residual_array(cfg, gen.CALIB, tokens=256)
    shape = orc.make_shape(orc.E4M3, orc.RESIDUAL, 2, 2, 512, 1024)
    blob = orc.fit_tables(shape, ct.numpy(), cp.numpy(), 256)
    c = orc.encode(blob, shape, t.numpy(), p.numpy(), threads=4)
    assert np.array_equal(orc.decode(blob, c, p.numpy(), t.numpy(), threads=4), t.numpy())
    assert t.numpy().nbytes / len(c) > 2.5
    cfg4 = gen.CONFIGS[4].with_tokens(512, channels=128)
    coef, G = gen.dckv_draw(cfg4)
    cc, cg = gen.dckv_draw(cfg4, gen.CALIB, tokens=256)
    shape = orc.make_shape(orc.INT16, orc.CHECKERBOARD, 1, 1, 512, 128)
    blob = orc.fit_tables(shape, cc.numpy(), cg.numpy(), 256)
    c = orc.encode(blob, shape, coef.numpy(), G.numpy(), threads=4)
    assert np.array_equal(orc.decode(blob, c, G.numpy(), coef.numpy(), threads=4), coef.numpy())


def test_corruption_is_detected(orc, cfg0):
    shape, blob, t, p = cfg0
    c = orc.encode(blob, shape, t, p, threads=4)
    out = np.zeros_like(t)
    assert orc.decode_rc(blob, c[:-4], p, out) == orc.E_CORRUPT            # truncated
    assert orc.decode_rc(blob, c[:40], p, out) == orc.E_CORRUPT
    bad = bytearray(c)
    bad[0] = ord("X")
    assert orc.decode_rc(blob, bytes(bad), p, out) == orc.E_CORRUPT        # magic
    other = bytearray(blob)
    other[64 + 2] ^= 1
    assert orc.decode_rc(bytes(other), c, p, out) == orc.E_TABLES          # wrong tables
    _, n, idx, pay = parse(c)
    head = 64 + 8 * (n + 1)
    rng = np.random.default_rng(2)
    for _ in range(12):
        s = int(rng.integers(0, n))
        a = int(idx[s] & np.uint64((1 << 63) - 1))
        b = int(idx[s + 1] & np.uint64((1 << 63) - 1))
        nw = int.from_bytes(c[head + a + 128:head + a + 132], "little")
        pos = head + int(rng.integers(a, a + 132 + 2 * nw))  # states, word count or a word
        flip = bytearray(c)
        flip[pos] ^= 1 << int(rng.integers(0, 8))
        assert orc.decode_rc(blob, bytes(flip), p, out) == orc.E_CORRUPT
    assert orc.decode_rc(blob, c, p, out) == 0 and np.array_equal(out, t)


def test_shape_errors(orc, cfg0):
    _, blob, t, p = cfg0
    for bad in [orc.make_shape(orc.BF16, orc.RESIDUAL, 1, 2, 1000, 1024),     # ragged tokens
                orc.make_shape(orc.BF16, orc.RESIDUAL, 1, 2, 1024, 1000),     # ragged channels
                orc.make_shape(orc.INT16, orc.RESIDUAL, 1, 2, 1024, 1024),
                orc.make_shape(orc.INT16, orc.CHECKERBOARD, 1, 1, 384, 32)]:  # odd number of pass blocks
        with pytest.raises(RuntimeError, match="-2"):
            orc.encode(blob, bad, t, p)


def test_coded_size_within_half_percent_of_cross_entropy(orc, cfg0):
    """Bits spent on words plus the information held in the final states
    versus sum(-log2 f/4096) + 8 bits per escape chunk under the tables."""
    shape, blob, t, p = cfg0
    c = orc.encode(blob, shape, t, p, threads=4)
    _, n, idx, pay = parse(c)
    tabs = [orc.blob_table(blob, j) for j in range(2048)]
    # symbol values through lookup tables built from the (separately pinned) oracle maps
    ordt = np.array([orc.ord_(x, 16) for x in range(65536)], dtype=np.int64)
    zig = np.array([orc.zigzag(r) for r in range(-32768, 32768)], dtype=np.int64)
    tu, pu = t.view(np.uint16).astype(np.int64), p.view(np.uint16).astype(np.int64)
    r = (ordt[tu] - ordt[pu]) % 65536
    r = np.where(r >= 32768, r - 65536, r)
    z = zig[r + 32768][0]                      # [kv][tokens][channels]
    ideal = 0.0
    for kv in range(2):
        for ch in range(1024):
            n_j, f = tabs[kv * 1024 + ch]
            bits = np.log2(4096.0 / f.astype(np.float64))
            zz = z[kv, :, ch]
            ideal += bits[np.minimum(zz, n_j)].sum() + 16.0 * (zz >= n_j).sum()
    coded = 0.0
    nesc_total = 0
    for s in range(n):
        data, raw = stream_bytes(idx, pay, s)
        assert not raw
        st = np.frombuffer(data[:128], np.uint32).astype(np.float64)
        nw = int.from_bytes(data[128:132], "little")
        nesc = (len(data) - 132 - 2 * nw) // 2          # u16 escapes; the pad is at most one u16
        coded += 16.0 * nw + np.log2(st / 65536.0).sum() + 16.0 * nesc
        nesc_total += nesc
    slack = 16.0 * n                                    # a pad u16 counted as an escape
    assert ideal * 0.995 <= coded <= ideal * 1.005 + slack
