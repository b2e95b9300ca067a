"""Oracle pins for the exponent-conditioned residual mode.

The table of a value is chosen by its predictor's exponent field (the class
E - base clamped to [0, 15], base fixed per slab at fit time), the finer
residual model the Speculative KV coding summary leaves open ('Early
results') in the conditional-model form of the DCKV page ('How it differs').
Each table is the same discretized Laplace as the per-channel mode, fitted
to the slab's calibration values of that class.
"""
import numpy as np
import pytest

from test_oracle_tables import _check_table, _scipy_mass, _tail_floor, _unzig, _zigzag_residuals
from workloads import gen


def _exp_field(p, dtype, orc):
    p = np.asarray(p).astype(np.int64)
    return (p >> 3) & 0xF if dtype == orc.E4M3 else (p >> 7) & 0xFF


def _e4m3_value(u):
    """Value of an e4m3 pattern (OCP FP8: bias 7, subnormals, 0x7F/0xFF NaN)."""
    s, e, m = (u >> 7) & 1, (u >> 3) & 0xF, u & 7
    if e == 0xF and m == 7:
        return float("nan")
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def test_exp_class_properties(orc):
    # e4m3, base 0: independent of sign and mantissa, monotone in magnitude, 16 classes
    cls = np.array([orc.exp_class(u, orc.E4M3, 0) for u in range(256)])
    assert cls.min() == 0 and cls.max() == 15 and len(set(cls.tolist())) == 16
    assert all(cls[u] == cls[u ^ 0x80] for u in range(256))
    assert all(len(set(cls[(u & ~7):(u & ~7) + 8].tolist())) == 1 for u in range(0, 256, 8))
    pos = [u for u in range(128) if not np.isnan(_e4m3_value(u))]
    order = sorted(pos, key=_e4m3_value)
    assert all(cls[a] <= cls[b] for a, b in zip(order, order[1:]))
    # bf16 with a base: exponents base .. base + 15 get classes 0 .. 15, the rest clamp
    base = 117
    for e in range(256):
        for u in (e << 7, (e << 7) | 0x55, 0x8000 | (e << 7) | 0x7F):
            want = min(max(e - base, 0), 15)
            assert orc.exp_class(u, orc.BF16, base) == want


def _fit(orc, dtype, cfg, ct, cp):
    shape = orc.make_shape(dtype, orc.RESIDUAL_EXP, cfg.layers, cfg.kv, 128, cfg.channels)
    return orc.fit_tables(shape, ct, cp, ct.shape[2])


@pytest.mark.parametrize("cid", [2, 0])
def test_expmode_fit_matches_laplace(orc, cid):
    cfg = gen.CONFIGS[cid].with_tokens(256, layers=1, channels=256)
    dtype = orc.E4M3 if cfg.dtype == "e4m3" else orc.BF16
    nbits = 8 if dtype == orc.E4M3 else 16
    ct, cp = [a.numpy() for a in gen.residual_array(cfg, gen.CALIB, tokens=256)]
    blob = _fit(orc, dtype, cfg, ct, cp)
    slabs = cfg.layers * cfg.kv
    assert len(blob) == 64 + slabs * 16 * 514 + slabs
    assert int.from_bytes(blob[8:12], "little") == slabs * 16 and blob[7] == orc.RESIDUAL_EXP
    bases = orc.blob_bases(blob)
    emax = 15 if dtype == orc.E4M3 else 255
    for sl in range(slabs):
        l, k = divmod(sl, cfg.kv)
        t, p = ct[l, k].ravel(), cp[l, k].ravel()
        e = _exp_field(p.view(np.uint8 if nbits == 8 else np.uint16), dtype, orc)
        hist = np.bincount(e, minlength=256)
        win = [hist[b:b + 16].sum() for b in range(emax - 14)]
        assert bases[sl] == int(np.argmax(win))                  # first window with the most predictors
        cls = np.clip(e - int(bases[sl]), 0, 15)
        z = _zigzag_residuals(t, p, nbits)
        r = _unzig(z)
        floor_n = _tail_floor(z)
        inr = np.abs(r) <= 127
        b_all = max(0.05, np.abs(r[inr]).mean())
        for q in range(16):
            members = cls == q
            sel = members & inr
            b = max(0.05, np.abs(r[sel]).mean()) if sel.sum() >= 64 else b_all
            masses = np.array([_scipy_mass(v, 0.0, b) for v in _unzig(np.arange(255))])
            n, f = orc.blob_table(blob, sl * 16 + q)
            pe = (np.count_nonzero(z[members] >= n) + 1.0) / (members.sum() + 2.0)
            _check_table(n, f, masses, pe, floor_n)


def test_expmode_empty_classes_share_the_pooled_table(orc):
    cfg = gen.CONFIGS[2].with_tokens(256, layers=1, channels=64)
    ct, cp = [a.numpy() for a in gen.residual_array(cfg, gen.CALIB, tokens=256)]
    blob = _fit(orc, orc.E4M3, cfg, ct, cp)
    e = _exp_field(cp[0, 0].ravel(), orc.E4M3, orc)
    empty = [q for q in range(16) if not np.any(e == q)]
    assert len(empty) >= 2
    recs = [orc.blob_table(blob, q) for q in empty]
    for n, f in recs[1:]:
        assert n == recs[0][0] and np.array_equal(f, recs[0][1])


def test_expmode_fit_ignores_channel_order(orc):
    """The tables pool a slab's values by class, so permuting channels leaves
    the blob unchanged (the per-channel mode's blob permutes with them)."""
    cfg = gen.CONFIGS[0].with_tokens(256, layers=1, channels=128)
    ct, cp = [a.numpy() for a in gen.residual_array(cfg, gen.CALIB, tokens=256)]
    perm = np.random.default_rng(5).permutation(cfg.channels)
    a = _fit(orc, orc.BF16, cfg, ct, cp)
    b = _fit(orc, orc.BF16, cfg, np.ascontiguousarray(ct[..., perm]), np.ascontiguousarray(cp[..., perm]))
    assert a == b


def test_expmode_stream_uses_the_class_tables(orc):
    """One 32 x 128 stream: the container's payload equals the generic stream
    codec fed with the table of each position's class."""
    cfg = gen.Config(98, "exp-wiring", "e4m3", 1, 1, 128, 32)
    t, p = [a.numpy() for a in gen.residual_array(cfg)]
    ct, cp = [a.numpy() for a in gen.residual_array(cfg, gen.CALIB, tokens=256)]
    blob = _fit(orc, orc.E4M3, cfg, ct, cp)
    shape = orc.make_shape(orc.E4M3, orc.RESIDUAL_EXP, 1, 1, 128, 32)
    cont = orc.encode(blob, shape, t, p)
    assert cont[7] == orc.RESIDUAL_EXP
    tables = [orc.blob_table(blob, q) for q in range(16)]
    tt, pp = t[0, 0], p[0, 0]                                 # [128 steps][32 lanes]
    z = _zigzag_residuals(tt, pp, 8).astype(np.uint32)
    tab_of = np.array([[orc.exp_class(int(v), orc.E4M3, 0) for v in row] for row in pp], dtype=np.uint32)
    want = orc.stream_encode(z, tab_of, tables, 128, 1)
    head = 64 + 16
    assert cont[head:] == want
    back = orc.decode(blob, cont, p, t)
    assert np.array_equal(back, t)


@pytest.mark.parametrize("cid", [2, 0])
def test_expmode_roundtrip_and_ratio(orc, cid):
    cfg = gen.CONFIGS[cid].with_tokens(512, layers=2, channels=256)
    dtype = orc.E4M3 if cfg.dtype == "e4m3" else orc.BF16
    t, p = [a.numpy() for a in gen.residual_array(cfg)]
    ct, cp = [a.numpy() for a in gen.residual_array(cfg, gen.CALIB, tokens=256)]
    sizes = {}
    for mode in (orc.RESIDUAL, orc.RESIDUAL_EXP):
        shape = orc.make_shape(dtype, mode, cfg.layers, cfg.kv, cfg.tokens, cfg.channels)
        blob = orc.fit_tables(shape, ct, cp, 256)
        cont = orc.encode(blob, shape, t, p, threads=8)
        assert np.array_equal(orc.decode(blob, cont, p, t, threads=8), t)
        sizes[mode] = len(cont)
    # the synthetic predictor's error grows with magnitude (e4m3 rounding), so the
    # exponent classes separate narrow and wide residuals
    assert sizes[orc.RESIDUAL_EXP] < sizes[orc.RESIDUAL]


@pytest.mark.parametrize("exp", [False, True])
def test_layer_slice_of_a_blob_is_the_fit_of_those_layers(orc, exp):
    """Tables are fitted per (layer, K|V) slab from that slab's calibration
    alone, so the blob fitted on a run of layers holds exactly the parent
    blob's records (and, with exponent classes, base bytes) of those layers;
    the transfer pipeline's per-chunk containers rely on this."""
    cfg = gen.CONFIGS[0].with_tokens(256, layers=3, channels=64)
    mode = orc.RESIDUAL_EXP if exp else orc.RESIDUAL
    ct, cp = [a.numpy() for a in gen.residual_array(cfg, gen.CALIB, tokens=256)]
    full = orc.fit_tables(orc.make_shape(orc.BF16, mode, 3, cfg.kv, 128, cfg.channels), ct, cp, 256)
    part = orc.fit_tables(orc.make_shape(orc.BF16, mode, 2, cfg.kv, 128, cfg.channels),
                          np.ascontiguousarray(ct[1:]), np.ascontiguousarray(cp[1:]), 256)
    per_layer = cfg.kv * (16 if exp else cfg.channels)
    rec = 514
    assert part[64 + 0:64 + 2 * per_layer * rec] == full[64 + per_layer * rec:64 + 3 * per_layer * rec]
    if exp:
        assert list(orc.blob_bases(part)) == list(orc.blob_bases(full))[cfg.kv:]
    assert int.from_bytes(part[12:16], "little") == 2
    assert int.from_bytes(part[8:12], "little") == 2 * per_layer
    assert int.from_bytes(part[32:40], "little") == len(part)
    # everything else in the header is the parent's
    assert part[:8] == full[:8] and part[16:32] == full[16:32] and part[40:64] == full[40:64]
