"""Oracle table fit against the textbook Laplace distribution (scipy).

Tables: per-channel (residual mode) or per-component x 16 shifts
(checkerboard mode) discretized Laplace, masses integrated over unit
quantization cells (DCKV page, 'How it differs'), fitted once on calibration
draws (Speculative KV coding summary, 'What to use as the predictor').
"""
import numpy as np
import pytest
import scipy.stats as st

from workloads import gen


def _unzig(z):
    z = np.asarray(z, dtype=np.int64)
    return np.where(z % 2 == 0, z // 2, -(z + 1) // 2)


def _scipy_mass(v, m, b):
    return st.laplace.cdf(v + 0.5, loc=m, scale=b) - st.laplace.cdf(v - 0.5, loc=m, scale=b)


@pytest.mark.parametrize("m", [0.0, 0.25, 0.5, 15 / 16])
@pytest.mark.parametrize("b", [0.05, 0.4, 3.0, 20.0, 300.0])
def test_cell_mass_matches_scipy(orc, m, b):
    for v in range(-40, 41):
        want = _scipy_mass(v, m, b)
        got = orc.cell_mass(float(v), m, b)
        if want > 1e-300:
            assert got == pytest.approx(want, rel=1e-9, abs=1e-15)


def _zigzag_residuals(t, p, nbits):
    """Zigzag of the ordered-integer residual, vectorized (the definition:
    order-preserving integer of each bit pattern, difference mod 2^N read as
    signed, zigzag)."""
    span, half = 1 << nbits, 1 << (nbits - 1)
    t = np.asarray(t).astype(np.int64) & (span - 1)
    p = np.asarray(p).astype(np.int64) & (span - 1)
    ordv = lambda u: np.where(u & half, (span - 1) ^ u, u ^ half)
    r = (ordv(t) - ordv(p)) % span
    r = np.where(r >= half, r - span, r)
    return np.where(r >= 0, 2 * r, -2 * r - 1)


def _tail_floor(z):
    """Smallest z0 in [1, 255] with at most len(z) // 1024 symbols >= z0."""
    allow = len(z) // 1024
    for z0 in range(1, 256):
        if np.count_nonzero(z >= z0) <= allow:
            return z0
    return 255


def _check_table(n, f, masses, pe, floor_n=1):
    f = np.asarray(f, dtype=np.int64)
    assert f.sum() == 4096 and (f >= 1).all() and 1 <= n <= 255 and len(f) == n + 1
    # direct range: z = 0 always, then up to the last z <= 254 with mass >= 2^-12,
    # and at least the slab's calibration tail floor
    big = [z for z in range(255) if masses[z] >= 2.0 ** -12]
    assert n == max(max([0] + big) + 1, floor_n)
    q = np.empty(n + 1)
    q[:n] = 4096.0 * masses[:n] * (1.0 - pe) / masses[:n].sum()
    q[n] = 4096.0 * pe
    # the quantization rule applied to the scipy masses: floor with minimum 1,
    # then +1 on the largest remainders or -1 on the largest frequencies; a
    # last-bit difference between the two mass evaluations can move one unit
    g = np.maximum(np.floor(q), 1.0).astype(np.int64)
    left = 4096 - int(g.sum())
    if left > 0:
        for i in sorted(range(n + 1), key=lambda i: (-(q[i] - g[i]), i))[:left]:
            g[i] += 1
    for _ in range(-left):
        g[int(np.argmax(np.where(g > 1, g, -1)))] -= 1
    assert np.all(np.abs(f - g) <= 1)


def test_residual_fit_matches_laplace(orc):
    cfg = gen.CONFIGS[0]
    ct, cp = gen.residual_array(cfg, gen.CALIB, tokens=256)
    ct, cp = ct.numpy(), cp.numpy()
    shape = orc.make_shape(orc.BF16, orc.RESIDUAL, 1, 2, 128, 1024)
    blob = orc.fit_tables(shape, ct, cp, 256)
    assert len(blob) == 64 + 2048 * 514
    floors = [_tail_floor(_zigzag_residuals(ct[0, kv], cp[0, kv], 16).ravel()) for kv in range(2)]
    rng = np.random.default_rng(3)
    for j in rng.choice(2048, 24, replace=False):
        kv, ch = divmod(int(j), 1024)
        r = np.array([orc.residual(int(a), int(b), 16) for a, b in zip(ct[0, kv, :, ch], cp[0, kv, :, ch])])
        small = np.abs(r)[np.abs(r) <= 127]
        b = max(0.05, small.mean() if len(small) else 0.0)
        masses = np.array([_scipy_mass(v, 0.0, b) for v in _unzig(np.arange(255))])
        n, f = orc.blob_table(blob, int(j))
        z = np.array([orc.zigzag(int(x)) for x in r])
        pe = ((z >= n).sum() + 1.0) / (256 + 2.0)
        _check_table(n, f, masses, pe, floors[kv])


def test_e4m3_fit_matches_laplace(orc):
    cfg = gen.CONFIGS[2].with_tokens(256, layers=1)
    ct, cp = gen.residual_array(cfg, gen.CALIB, tokens=256)
    ct, cp = ct.numpy(), cp.numpy()
    shape = orc.make_shape(orc.E4M3, orc.RESIDUAL, 1, 2, 128, 1024)
    blob = orc.fit_tables(shape, ct, cp, 256)
    floors = [_tail_floor(_zigzag_residuals(ct[0, kv], cp[0, kv], 8).ravel()) for kv in range(2)]
    for j in (0, 1, 517, 1500, 2047):
        kv, ch = divmod(j, 1024)
        r = np.array([orc.residual(int(a), int(b), 8) for a, b in zip(ct[0, kv, :, ch], cp[0, kv, :, ch])])
        small = np.abs(r)[np.abs(r) <= 127]
        b = max(0.05, small.mean())
        masses = np.array([_scipy_mass(v, 0.0, b) for v in _unzig(np.arange(255))])
        n, f = orc.blob_table(blob, j)
        z = np.array([orc.zigzag(int(x)) for x in r])
        pe = ((z >= n).sum() + 1.0) / 258.0
        _check_table(n, f, masses, pe, floors[kv])


@pytest.mark.parametrize("tail, floor_n", [(256, None), (257, 101)])
def test_tail_floor_boundary(orc, tail, floor_n):
    """262,144 calibration symbols of one slab allow 256 escapes: 256
    symbols at z = 100 leave the Laplace direct range alone, 257 push every
    table of the slab to n = 101."""
    C, T = 1024, 256
    p = np.full((1, 1, T, C), 0x3F80, dtype=np.uint16)           # bf16 1.0
    t = p.copy()
    rng = np.random.default_rng(11)
    # small residuals everywhere (ordered step +-1 or 0) so that the Laplace scale is small
    t[0, 0] = (p[0, 0].astype(np.int64) + rng.integers(-1, 2, size=(T, C))).astype(np.uint16)
    flat = t.reshape(-1)
    pos = rng.choice(T * C, size=tail, replace=False)
    flat[pos] = 0x3F80 + 50                                         # residual +50 -> z = 100
    z = _zigzag_residuals(t, p, 16).ravel()
    assert np.count_nonzero(z >= 100) == tail and z.max() == 100
    shape = orc.make_shape(orc.BF16, orc.RESIDUAL, 1, 1, 128, C)
    blob = orc.fit_tables(shape, t.view(np.int16), p.view(np.int16), T)
    ns = [orc.blob_table(blob, j)[0] for j in range(0, C, 37)]
    if floor_n is None:
        assert max(ns) < 101
    else:
        assert ns == [floor_n] * len(ns)


def test_checkerboard_fit_matches_laplace(orc):
    cfg = gen.CONFIGS[4].with_tokens(256, channels=64)
    coef, G = gen.dckv_draw(cfg, gen.CALIB, tokens=256)
    coef, G = coef.numpy(), G.numpy()
    shape = orc.make_shape(orc.INT16, orc.CHECKERBOARD, 1, 1, 256, 64)
    blob = orc.fit_tables(shape, coef, G, 256)
    assert len(blob) == 64 + 64 * 16 * 514
    for comp in (0, 13, 63):
        mu = np.array([orc.dckv_mean(coef, G, t, comp) for t in range(256)])
        e = coef[:, comp] - mu / 16.0
        small = np.abs(e)[np.abs(e) <= 127]
        b = max(0.05, small.mean())
        nf = []
        for f in range(16):
            n, fr = orc.blob_table(blob, comp * 16 + f)
            nf.append((n, fr))
        zs = [orc.dckv_symbol(int(c), int(m)) for c, m in zip(coef[:, comp], mu)]
        pe = (sum(z >= nf[f][0] for z, f in zs) + 1.0) / 258.0
        for f in range(16):
            masses = np.array([_scipy_mass(v, f / 16.0, b) for v in _unzig(np.arange(255))])
            _check_table(nf[f][0], nf[f][1], masses, pe)


def test_blob_header(orc):
    cfg = gen.CONFIGS[0]
    ct, cp = gen.residual_array(cfg, gen.CALIB, tokens=256)
    shape = orc.make_shape(orc.BF16, orc.RESIDUAL, 1, 2, 128, 1024)
    blob = orc.fit_tables(shape, ct.numpy(), cp.numpy(), 256)
    h = np.frombuffer(blob[:64], dtype=np.uint8)
    assert bytes(h[:4]) == b"SKVT"
    assert int.from_bytes(blob[4:6], "little") == 1 and blob[6] == 1 and blob[7] == 0
    assert int.from_bytes(blob[8:12], "little") == 2048
    assert int.from_bytes(blob[32:40], "little") == len(blob)


def test_fnv1a64_published_vectors(orc):
    # FNV-1a 64-bit test vectors from the FNV reference (Fowler/Noll/Vo)
    assert orc.fnv1a64(b"") == 0xcbf29ce484222325
    assert orc.fnv1a64(b"a") == 0xaf63dc4c8601ec8c
    assert orc.fnv1a64(b"foobar") == 0x85944171f73967e8
