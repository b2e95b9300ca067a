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


def _check_table(n, f, masses, pe):
    f = np.asarray(f, dtype=np.int64)
    assert f.sum() == 4096 and (f >= 1).all() and 1 <= n <= 255 and len(f) == n + 1
    # direct range: z = 0 always, then up to the last z <= 254 with mass >= 2^-12
    big = [z for z in range(255) if masses[z] >= 2.0 ** -12]
    assert n == max([0] + big) + 1
    q = np.empty(n + 1)
    q[:n] = 4096.0 * masses[:n] * (1.0 - pe) / masses[:n].sum()
    q[n] = 4096.0 * pe
    assert np.all(np.abs(f - np.maximum(q, 1.0)) <= 1.0 + 1e-9)


def test_residual_fit_matches_laplace(orc):
    cfg = gen.CONFIGS[0]
    ct, cp = gen.residual_array(cfg, gen.CALIB, tokens=256)
    ct, cp = ct.numpy(), cp.numpy()
    shape = orc.make_shape(orc.BF16, orc.RESIDUAL, 1, 2, 128, 1024)
    blob = orc.fit_tables(shape, ct, cp, 256)
    assert len(blob) == 64 + 2048 * 514
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
        _check_table(n, f, masses, pe)


def test_e4m3_fit_matches_laplace(orc):
    cfg = gen.CONFIGS[2].with_tokens(256, layers=1)
    ct, cp = gen.residual_array(cfg, gen.CALIB, tokens=256)
    ct, cp = ct.numpy(), cp.numpy()
    shape = orc.make_shape(orc.E4M3, orc.RESIDUAL, 1, 2, 128, 1024)
    blob = orc.fit_tables(shape, ct, cp, 256)
    for j in (0, 1, 517, 1500, 2047):
        kv, ch = divmod(j, 1024)
        r = np.array([orc.residual(int(a), int(b), 8) for a, b in zip(ct[0, kv, :, ch], cp[0, kv, :, ch])])
        small = np.abs(r)[np.abs(r) <= 127]
        b = max(0.05, small.mean())
        masses = np.array([_scipy_mass(v, 0.0, b) for v in _unzig(np.arange(255))])
        n, f = orc.blob_table(blob, j)
        z = np.array([orc.zigzag(int(x)) for x in r])
        pe = ((z >= n).sum() + 1.0) / 258.0
        _check_table(n, f, masses, pe)


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
