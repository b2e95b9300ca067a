"""Oracle pins: hand-computed worked examples, closed forms and brute force.

Each test ties the oracle to something other than itself: values computed by
hand from the definitions (fixtures under tests/golden with their
citations), exhaustive enumeration of the symbol maps, the uniform-table
special case where rANS reduces to bit insertion, and brute force on tiny
streams.
"""
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- rANS primitive
def test_e1_single_lane_two_symbols(orc):
    e = _load("rans_pins.json")["E1"]
    x = e["start"]
    for (f, c), want, w in zip(e["puts"], e["states"], e["words"]):
        x, out = orc.rans_put(x, f, c)
        assert x == want and out == w
    freq, cum = [2048, 1024], [0, 2048]
    for slot, want in zip(e["pop_slots"], e["pop_states"]):
        assert x & 4095 == slot
        s, x = orc.rans_pop(x, freq, cum)
        assert x == want
    assert x == 65536


def test_e2_renormalization(orc):
    e = _load("rans_pins.json")["E2"]
    x = e["start"]
    for (f, c), want, w in zip(e["puts"], e["states"], e["words"]):
        x, out = orc.rans_put(x, f, c)
        assert x == want and out == w


def test_e3_lane_order(orc):
    e = _load("rans_pins.json")["E3"]
    steps = e["steps"]
    # lane i codes the symbol with cum 4095 - i, i.e. symbol j = 32 - i.  All 33
    # symbols must be direct, so the table lists them as 0..32 and puts its ESC
    # (never coded here) at index 33 with frequency 0.
    z = np.array([[32 - i for i in range(32)]] * steps, dtype=np.uint32)
    tab = (33, [4064] + [1] * 32 + [0])
    data = orc.stream_encode(z, np.zeros(steps * 32, np.uint32), [tab], steps, 2)
    assert int.from_bytes(data[128:132], "little") == len(e["words"])
    words = np.frombuffer(data[132:], dtype=np.uint16)
    assert list(words) == e["words"]
    assert len(data) == e["bytes"]
    states = np.frombuffer(data[:128], dtype=np.uint32)
    assert list(states) == [e["state_lane0"] - i for i in range(32)]
    rc, zz = orc.stream_decode(data, np.zeros(steps * 32, np.uint32), [tab], steps, 2)
    assert rc == 0 and np.array_equal(zz, z.reshape(-1))


@pytest.mark.parametrize("name", ["E4", "E5"])
def test_escape_region(orc, name):
    e = _load("rans_pins.json")[name]
    steps = e["steps"]
    z = np.zeros((steps, 32), dtype=np.uint32)
    for key, v in e["z"].items():
        k, i = (0, int(key)) if "," not in key else map(int, key.split(","))
        z[k, i] = v
    tab = (1, e["table"])
    data = orc.stream_encode(z, np.zeros(steps * 32, np.uint32), [tab], steps, e["ebytes"])
    assert len(data) == e["bytes"]
    st = np.frombuffer(data[:128], dtype=np.uint32)
    for i in range(32):
        assert st[i] == e["states"].get(str(i), e["states"]["other"]), i
    nw = int.from_bytes(data[128:132], "little")
    assert nw == len(e["words"])
    esc = np.frombuffer(data[132 + 2 * nw:132 + 2 * nw + 2 * len(e["escapes"])], dtype=np.uint16)
    assert list(esc) == e["escapes"]
    assert not any(data[132 + 2 * nw + 2 * len(e["escapes"]):])     # zero pad
    rc, zz = orc.stream_decode(data, np.zeros(steps * 32, np.uint32), [tab], steps, e["ebytes"])
    assert rc == 0 and np.array_equal(zz, z.reshape(-1))
    # any change in the pad or a truncated escape region is rejected
    if len(data) > 132 + 2 * nw + 2 * len(e["escapes"]):
        bad = bytearray(data)
        bad[-1] ^= 1
        rc, _ = orc.stream_decode(bytes(bad), np.zeros(steps * 32, np.uint32), [tab], steps, e["ebytes"])
        assert rc == orc.E_CORRUPT


def test_uniform_table_is_bit_insertion(orc):
    """255 direct values at frequency 16 plus ESC at 16: each put shifts the
    state left by exactly 8 bits and each word removes 16, so
    sum_i (floor(log2 x_i) - 16) = 8 * symbols - 16 * words; escaped values
    (255) are stored raw, one byte each."""
    rng = np.random.default_rng(1)
    steps = 16
    z = rng.integers(0, 256, size=steps * 32).astype(np.uint32)
    tab = (255, [16] * 256)
    data = orc.stream_encode(z, np.zeros(steps * 32, np.uint32), [tab], steps, 1)
    nesc = int((z == 255).sum())
    st = np.frombuffer(data[:128], dtype=np.uint32).astype(np.int64)
    nw = int.from_bytes(data[128:132], "little")
    bitlen = sum(int(x).bit_length() - 17 for x in st)
    assert bitlen == 8 * steps * 32 - 16 * nw
    assert len(data) == (132 + 2 * nw + nesc + 3) // 4 * 4
    esc = data[132 + 2 * nw:132 + 2 * nw + nesc]
    assert list(esc) == [255] * nesc
    rc, zz = orc.stream_decode(data, np.zeros(steps * 32, np.uint32), [tab], steps, 1)
    assert rc == 0 and np.array_equal(zz, z)
    # closed form of one put: x' = ((x >> 4) << 12) | (s << 4) | (x & 15)
    for x in (65536, 65537, 1 << 20, (1 << 24) - 1, 12345678):
        for s in (0, 1, 77, 254):
            y, w = orc.rans_put(x, 16, 16 * s)
            xx = x if w is None else x >> 16
            assert y == ((xx >> 4) << 12) | (s << 4) | (xx & 15)


def test_brute_force_tiny_streams(orc):
    """Every assignment of 4 values (incl. escapes) to a 2-step stream where
    all lanes repeat the pattern: decode(encode) is the identity and distinct
    inputs give distinct streams."""
    tab = (2, [3000, 1000, 96])
    vals = [0, 1, 2, 300]
    seen = {}
    for a in vals:
        for b in vals:
            for lane_shift in (0, 1):
                z = np.array([[(a if (i + lane_shift) % 2 else b) for i in range(32)],
                              [(b if (i + lane_shift) % 3 else a) for i in range(32)]], dtype=np.uint32)
                data = orc.stream_encode(z, np.zeros(64, np.uint32), [tab], 2, 2)
                rc, zz = orc.stream_decode(data, np.zeros(64, np.uint32), [tab], 2, 2)
                assert rc == 0 and np.array_equal(zz, z.reshape(-1))
                key = z.tobytes()
                assert seen.setdefault(data, key) == key


# ---------------------------------------------------------------- symbolizer
def test_symbolizer_examples(orc):
    g = _load("symbolizer_pins.json")
    for c in g["S"]:
        n = c["nbits"]
        assert orc.ord_(c["t"], n) == c["ord_t"]
        assert orc.ord_(c["p"], n) == c["ord_p"]
        assert orc.residual(c["t"], c["p"], n) == c["r"]
        assert orc.zigzag(c["r"]) == c["z"]
        assert orc.reconstruct(c["p"], orc.unzigzag(c["z"]), n) == c["t"]


def test_dckv_split_examples(orc):
    g = _load("symbolizer_pins.json")
    for c in g["D"]:
        k, f = orc.dckv_split(c["mu_q"])
        if "k" in c:
            assert (k, f) == (c["k"], c["f"])
        if "c" in c:
            z, _ = orc.dckv_symbol(c["c"], c["mu_q"])
            assert orc.unzigzag(z) == c["d"] and z == c["z"]
            assert orc.dckv_reconstruct(z, c["mu_q"]) == c["c"]
    m = g["mean"]
    coef = np.array(m["coef"], np.int16)[:, None]
    G = np.array(m["G"], np.int16)[:, None]
    assert [orc.dckv_mean(coef, G, t, 0) for t in range(4)] == m["mean"]


def _bf16_values(u):
    return (np.asarray(u, dtype=np.uint32) << 16).view(np.float32)


def test_bf16_ord_exhaustive(orc):
    u = np.arange(65536, dtype=np.uint32)
    o = np.array([orc.ord_(int(x), 16) for x in u], dtype=np.int64)
    assert sorted(o) == list(range(65536))                       # a permutation
    assert all(orc.inv_ord(int(a), 16) == int(b) for a, b in zip(o, u))
    with np.errstate(invalid="ignore"):
        v = _bf16_values(u).astype(np.float64)
    ok = ~np.isnan(v)
    order = np.argsort(o[ok], kind="stable")
    vs = v[ok][order]
    assert np.all(np.diff(vs) >= 0)                               # monotone on non-NaN
    # equal values only for -0/+0, and -0 sorts first
    eq = np.where(np.diff(vs) == 0)[0]
    assert len(eq) == 1


def _e4m3_values():
    import torch
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_exhaustive(orc):
    vals = _e4m3_values()
    o = np.array([orc.ord_(x, 8) for x in range(256)])
    assert sorted(o) == list(range(256))
    ok = ~np.isnan(vals)
    vs = vals[ok][np.argsort(o[ok])]
    assert np.all(np.diff(vs) >= 0)
    # every (target, predictor) pair round-trips and the zigzag covers 0..255
    for t in range(256):
        for p in range(0, 256, 7):
            r = orc.residual(t, p, 8)
            z = orc.zigzag(r)
            assert 0 <= z < 256
            assert orc.reconstruct(p, orc.unzigzag(z), 8) == t


def test_bf16_residual_roundtrip_sampled(orc):
    rng = np.random.default_rng(7)
    for t, p in rng.integers(0, 65536, size=(4000, 2)):
        r = orc.residual(int(t), int(p), 16)
        z = orc.zigzag(r)
        assert 0 <= z < 65536 and -32768 <= r < 32768
        assert orc.reconstruct(int(p), orc.unzigzag(z), 16) == t


def test_zigzag_is_bijection(orc):
    zs = [orc.zigzag(r) for r in range(-32768, 32768)]
    assert sorted(zs) == list(range(65536))
    assert [orc.zigzag(r) for r in (0, -1, 1, -2, 2)] == [0, 1, 2, 3, 4]


# ---------------------------------------------------------------- quantization
@pytest.mark.parametrize("q,want", [
    ([2048.5, 2047.5], [2049, 2047]),                  # tie on remainder -> smaller index
    ([4095.9, 0.1], [4095, 1]),                        # minimum frequency 1
    ([4095.5, 0.3, 0.2], [4094, 1, 1]),                # excess taken from the largest
    ([1000.2, 1000.7, 2095.1], [1000, 1001, 2095]),    # largest remainder
])
def test_quantize_examples(orc, q, want):
    assert list(orc.quantize(q)) == want
