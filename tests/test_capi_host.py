"""libskv on the CPU: the library loads and exports every call declared in
include/skv.h; the host table fit matches the oracle's fit byte for byte;
blob validation and size queries behave as documented.  No device calls."""
import ctypes
import os
import re

import numpy as np
import pytest

from workloads import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def skv():
    from lossless_kv_cache_amd import skv as m
    if not os.path.exists(m.LIB_PATH):
        from lossless_kv_cache_amd import build
        build.build()
    m.lib()
    return m


def test_exports_every_declared_symbol(skv):
    text = open(os.path.join(ROOT, "include", "skv.h")).read()
    names = set(re.findall(r"^\s*(?:int|void|uint32_t|const char\*)\s+(skv_\w+)\s*\(", text, re.M))
    assert {"skv_fit_tables", "skv_load_tables", "skv_encode", "skv_decode", "skv_decode_range", "skv_transfer",
            "skv_free", "skv_version", "skv_strerror"} <= names
    L = ctypes.CDLL(skv.LIB_PATH)
    for n in sorted(names):
        assert hasattr(L, n), n
    assert skv.lib().skv_version() == 1


def _residual_calib(cfg):
    ct, cp = gen.residual_array(cfg, gen.CALIB, tokens=256)
    return ct.numpy(), cp.numpy()


@pytest.mark.parametrize("cid,layers", [(0, 1), (1, 2), (2, 2), (3, 1)])
def test_fit_matches_oracle_residual(skv, orc, cid, layers):
    cfg = gen.CONFIGS[cid].with_tokens(256, layers=layers)
    ct, cp = _residual_calib(cfg)
    dt = skv.E4M3 if cfg.dtype == "e4m3" else skv.BF16
    tabs = skv.fit_tables(dt, skv.RESIDUAL, cfg.layers, cfg.kv, cfg.channels, ct, cp, 256)
    shape = orc.make_shape(dt, orc.RESIDUAL, cfg.layers, cfg.kv, 128, cfg.channels)
    want = orc.fit_tables(shape, ct, cp, 256)
    got = tabs.bytes()
    assert len(got) == len(want)
    assert got == want


@pytest.mark.parametrize("cid,layers", [(0, 1), (1, 2), (2, 2), (3, 1)])
def test_fit_matches_oracle_exponent_mode(skv, orc, cid, layers):
    cfg = gen.CONFIGS[cid].with_tokens(256, layers=layers)
    ct, cp = _residual_calib(cfg)
    dt = skv.E4M3 if cfg.dtype == "e4m3" else skv.BF16
    tabs = skv.fit_tables(dt, skv.RESIDUAL_EXP, cfg.layers, cfg.kv, cfg.channels, ct, cp, 256)
    shape = orc.make_shape(dt, orc.RESIDUAL_EXP, cfg.layers, cfg.kv, 128, cfg.channels)
    assert tabs.bytes() == orc.fit_tables(shape, ct, cp, 256)
    # the blob loads back through validation
    again = skv.load_tables(tabs.bytes())
    assert again.bytes() == tabs.bytes()


def test_fit_matches_oracle_checkerboard(skv, orc):
    cfg = gen.CONFIGS[4].with_tokens(256, channels=256)
    cc, cg = gen.dckv_draw(cfg, gen.CALIB, tokens=256)
    tabs = skv.fit_tables(skv.INT16, skv.CHECKERBOARD, 1, 1, 256, cc.numpy(), cg.numpy(), 256)
    shape = orc.make_shape(orc.INT16, orc.CHECKERBOARD, 1, 1, 256, 256)
    assert tabs.bytes() == orc.fit_tables(shape, cc.numpy(), cg.numpy(), 256)


def test_fit_matches_oracle_adversarial(skv, orc):
    """Calibration with constant channels, sign crossings and all-escape
    channels exercises the floor on b, tiny direct ranges and R < 0."""
    rng = np.random.default_rng(9)
    T, C = 64, 64
    t = rng.integers(0, 65536, size=(1, 2, T, C), dtype=np.uint16)
    p = t.copy()
    p[0, 0, :, :8] = t[0, 0, :, :8]                      # exact: b -> floor
    p[0, 0, :, 8:16] ^= 0x8000                            # sign flips: huge residuals
    p[0, 1] = (t[0, 1].astype(np.int32) + rng.integers(-3, 4, size=(T, C))).astype(np.uint16)
    tabs = skv.fit_tables(skv.BF16, skv.RESIDUAL, 1, 2, C, t, p, T)
    shape = orc.make_shape(orc.BF16, orc.RESIDUAL, 1, 2, 128, C)
    assert tabs.bytes() == orc.fit_tables(shape, t, p, T)


def test_load_tables_validates(skv, orc):
    cfg = gen.CONFIGS[0].with_tokens(256)
    ct, cp = _residual_calib(cfg)
    good = orc.fit_tables(orc.make_shape(orc.BF16, orc.RESIDUAL, 1, 2, 128, 1024), ct, cp, 256)
    t = skv.load_tables(good)
    assert t.bytes() == good
    bad = bytearray(good)
    bad[64 + 2] ^= 1                                      # freq[0] changes: sum != 4096
    with pytest.raises(skv.SkvError, match="-5"):
        skv.load_tables(bytes(bad))
    bad = bytearray(good)
    bad[64] = 0                                           # n = 0
    with pytest.raises(skv.SkvError):
        skv.load_tables(bytes(bad))
    with pytest.raises(skv.SkvError):
        skv.load_tables(good[:-2])


def test_size_queries_and_shape_errors(skv):
    cfg = gen.CONFIGS[0].with_tokens(256)
    ct, cp = _residual_calib(cfg)
    tabs = skv.fit_tables(skv.BF16, skv.RESIDUAL, 1, 2, 1024, ct, cp, 256)
    L = skv.lib()
    ob, wb = ctypes.c_size_t(), ctypes.c_size_t()
    s = tabs.shape(1024)
    assert L.skv_encode(tabs.ptr, ctypes.byref(s), None, None, None, 0, ctypes.byref(ob), None, ctypes.byref(wb), None) == 0
    n = 2 * 8 * 32
    assert ob.value == 64 + 8 * (n + 1) + n * 8192
    assert wb.value >= n * 8192
    for bad in (tabs.shape(1000), skv.make_shape(skv.BF16, skv.RESIDUAL, 1, 2, 1024, 1000),
                skv.make_shape(skv.INT16, skv.RESIDUAL, 1, 2, 1024, 1024)):
        assert L.skv_encode(tabs.ptr, ctypes.byref(bad), None, None, None, 0, ctypes.byref(ob), None,
                            ctypes.byref(wb), None) == skv.ERR_SHAPE
    other = skv.make_shape(skv.BF16, skv.RESIDUAL, 2, 2, 1024, 1024)           # blob is for 1 layer
    assert L.skv_encode(tabs.ptr, ctypes.byref(other), None, None, None, 0, ctypes.byref(ob), None,
                        ctypes.byref(wb), None) == skv.ERR_TABLES
    dummy = ctypes.c_void_p(12345)
    assert L.skv_encode(dummy, ctypes.byref(s), None, None, None, 0, ctypes.byref(ob), None,
                        ctypes.byref(wb), None) == skv.ERR_ARG                  # not a library blob
    s.abi_version = 2
    assert L.skv_encode(tabs.ptr, ctypes.byref(s), None, None, None, 0, ctypes.byref(ob), None,
                        ctypes.byref(wb), None) == skv.ERR_SHAPE
    # decode workspace size queries (no device memory is touched)
    wd, wr = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.skv_decode(tabs.ptr, None, 0, None, None, 0, None, ctypes.byref(wd), None) == 0
    assert L.skv_decode_range(tabs.ptr, None, 0, 0, 128, None, None, 0, None, ctypes.byref(wr), None) == 0
    assert wr.value == wd.value > 0
    assert L.skv_decode_range(dummy, None, 0, 0, 128, None, None, 0, None, ctypes.byref(wr), None) == skv.ERR_ARG


def test_transfer_size_queries_and_argument_errors(skv):
    """skv_transfer's two-phase sizing: the wire bound is the sum of the
    chunk containers' bounds (every stream raw), and the workspace holds two
    container buffers per side; no device memory is touched."""
    L = skv.lib()
    cfg = gen.CONFIGS[0].with_tokens(256, layers=3, channels=64)
    ct, cp = _residual_calib(cfg)
    tabs = skv.fit_tables(skv.BF16, skv.RESIDUAL, 3, 2, 64, ct, cp, 256)
    s = tabs.shape(1024)
    wire, work = ctypes.c_size_t(), ctypes.c_size_t()

    def query(lpc, shape=s, t=tabs):
        return L.skv_transfer(t.ptr, ctypes.byref(shape), lpc, None, None, None, 0, ctypes.byref(wire), None, None,
                              None, 0, None, ctypes.byref(work), None)

    def bound(layers):
        n = layers * 2 * (1024 // 128) * (64 // 32)
        return 64 + 8 * (n + 1) + n * 4096 * 2

    for lpc, chunks in ((1, [1, 1, 1]), (2, [2, 1]), (3, [3])):
        assert query(lpc) == 0
        assert wire.value == sum(bound(c) for c in chunks)
        assert work.value >= 4 * bound(lpc) + 256
    assert query(0) == skv.ERR_ARG and query(4) == skv.ERR_ARG
    dummy = ctypes.c_void_p(12345)
    assert L.skv_transfer(dummy, ctypes.byref(s), 1, None, None, None, 0, ctypes.byref(wire), None, None, None, 0,
                          None, ctypes.byref(work), None) == skv.ERR_ARG
    other = skv.make_shape(skv.BF16, skv.RESIDUAL, 2, 2, 1024, 64)
    assert query(1, other) == skv.ERR_TABLES
    ragged = skv.make_shape(skv.BF16, skv.RESIDUAL, 3, 2, 1000, 64)
    assert query(1, ragged) == skv.ERR_SHAPE
    cb_cfg = gen.CONFIGS[4].with_tokens(256, channels=64)
    cc, cg = gen.dckv_draw(cb_cfg, gen.CALIB, tokens=256)
    cb = skv.fit_tables(skv.INT16, skv.CHECKERBOARD, 1, 1, 64, cc.numpy(), cg.numpy(), 256)
    assert query(1, cb.shape(1024), cb) == skv.ERR_SHAPE


def _small_tables(skv, dtype, mode, layers=1, kv=2, channels=64):
    if mode == skv.CHECKERBOARD:
        cfg = gen.CONFIGS[4].with_tokens(256, channels=channels)
        cc, cg = gen.dckv_draw(cfg, gen.CALIB, tokens=256)
        return skv.fit_tables(skv.INT16, skv.CHECKERBOARD, 1, 1, channels, cc.numpy(), cg.numpy(), 256)
    cfg = gen.CONFIGS[0 if dtype == skv.BF16 else 2].with_tokens(256, layers=layers, channels=channels)
    ct, cp = _residual_calib(cfg)
    return skv.fit_tables(dtype, mode, layers, kv, channels, ct, cp, 256)


def test_binding_refuses_mis_sized_device_inputs(skv):
    """The binding checks every array the kernels read or write against the
    tables' layout before calling the library: wrong shapes and element
    widths raise ValueError, and the decode capacity passed to the library is
    the smaller of the output's and the predictor's sizes.  (Host tensors of
    the right layout are refused as not device tensors; nothing is launched.)"""
    import torch

    tabs = _small_tables(skv, skv.E4M3, skv.RESIDUAL)
    good = torch.zeros((1, 2, 256, 64), dtype=torch.uint8)
    for bad, what in [(torch.zeros((1, 2, 256, 32), dtype=torch.uint8), "shape"),
                      (torch.zeros((2, 2, 256, 64), dtype=torch.uint8), "shape"),
                      (torch.zeros((1, 2, 128, 64), dtype=torch.uint8), "shape"),
                      (torch.zeros((1, 2, 256, 64), dtype=torch.int16), "byte elements"),
                      (np.zeros((1, 2, 256, 64), dtype=np.uint8), "device tensor")]:
        with pytest.raises(ValueError, match=what):
            skv._check_cache(bad, "target", tabs, 256)
    with pytest.raises(ValueError, match="device tensor"):
        skv._check_cache(good, "target", tabs, 256)
    # decode: out of another element width, and an aux of the wrong rank
    with pytest.raises(ValueError, match="byte elements"):
        skv._decode_buffers(good, torch.zeros(good.shape, dtype=torch.int16), tabs)
    with pytest.raises(ValueError, match="4-D"):
        skv._decode_buffers(good.view(-1), good, tabs)
    with pytest.raises(ValueError, match="shape"):
        skv._decode_buffers(good, good, tabs, tokens=128)
    # the public entry points refuse before reaching the library
    with pytest.raises(ValueError):
        skv.decode_into(tabs, torch.zeros(100, dtype=torch.uint8), good, good)
    with pytest.raises(skv.SkvError) as e:
        skv.decode_range_into(tabs, torch.zeros(100, dtype=torch.uint8), 0, 100, good, good)
    assert e.value.status == skv.ERR_SHAPE
    # bf16 tables take 2-byte elements; checkerboard arrays are [tokens][channels]
    tb = _small_tables(skv, skv.BF16, skv.RESIDUAL)
    with pytest.raises(ValueError, match="byte elements"):
        skv._check_cache(good, "aux", tb, 256)
    tc = _small_tables(skv, skv.INT16, skv.CHECKERBOARD)
    with pytest.raises(ValueError, match="shape"):
        skv._check_cache(torch.zeros((1, 1, 256, 64), dtype=torch.int16), "target", tc, 256)
    with pytest.raises(ValueError, match="device tensor"):
        skv._check_cache(torch.zeros((256, 64), dtype=torch.int16), "target", tc, 256)


def test_noalloc_size_limits_on_host(skv):
    """skv_encode_noalloc's size checks need no device: any residual shape
    reports the same bound as skv_encode (larger ones are coded in passes); a
    checkerboard shape past the fixed array is refused with SKV_ERR_SHAPE."""
    tabs = _small_tables(skv, skv.E4M3, skv.RESIDUAL, layers=1, channels=1024)
    for tokens in (128, 1024, 4096):
        s = tabs.shape(tokens)
        ob, wb = ctypes.c_size_t(), ctypes.c_size_t()
        assert skv.lib().skv_encode(tabs.ptr, ctypes.byref(s), None, None, None, 0, ctypes.byref(ob), None,
                                    ctypes.byref(wb), None) == 0
        assert wb.value <= skv.NOALLOC_WORK_BYTES
        assert skv.encode_noalloc_bound(tabs, tokens) == ob.value
    # 32768 tokens x 1024 channels x K,V: 16384 streams of 8 KiB scratch each, coded in passes
    s = tabs.shape(32768)
    ob = ctypes.c_size_t()
    assert skv.lib().skv_encode(tabs.ptr, ctypes.byref(s), None, None, None, 0, ctypes.byref(ob), None,
                                ctypes.byref(ctypes.c_size_t()), None) == 0
    assert skv.encode_noalloc_bound(tabs, 32768) == ob.value
    assert skv.encode_workspace(tabs, 32768, skv.NOALLOC_WORK_BYTES)[1] == 4
    # a checkerboard shape takes one pass: past the array it is refused
    tc = _small_tables(skv, skv.INT16, skv.CHECKERBOARD, channels=2048)
    with pytest.raises(skv.SkvError) as e:
        skv.encode_noalloc_bound(tc, 32768)
    assert e.value.status == skv.ERR_SHAPE


@pytest.mark.parametrize("rank,channels", [(16, 64), (64, 256), (256, 32)])
def test_fit_matches_oracle_neighbour_map(skv, orc, rank, channels):
    """The decoded-neighbour-map fit (the library's own host map applied to
    the calibration rows, then the checkerboard fit, then the map section)
    equals the oracle's blob byte for byte; the plain fit refuses the mode and
    the map fit refuses ranks that are not powers of two from 16 to 256."""
    cfg = gen.CONFIGS[4].with_tokens(512, channels=channels)
    V, U, sh1, sh2 = gen.dckv_map_weights(cfg, rank)
    cc, cg = (a.numpy() for a in gen.dckv_draw(cfg, gen.CALIB, tokens=256, nbr_map=(V, U, sh1, sh2)))
    tabs = skv.fit_tables_map(channels, cc, cg, 256, V, U, sh1, sh2)
    shape = orc.make_shape(orc.INT16, orc.CHECKERBOARD_MAP, 1, 1, 512, channels)
    want = orc.fit_tables_map(shape, cc, cg, 256, V, U, sh1, sh2)
    assert tabs.bytes() == want
    assert tabs.mode == skv.CHECKERBOARD_MAP
    # the blob loads back (validation of the map section)
    assert skv.load_tables(want).bytes() == want
    with pytest.raises(skv.SkvError) as e:
        skv.fit_tables(skv.INT16, skv.CHECKERBOARD_MAP, 1, 1, channels, cc, cg, 256)
    assert e.value.status == skv.ERR_SHAPE
    with pytest.raises(skv.SkvError) as e:
        skv.fit_tables_map(channels, cc, cg, 256, np.zeros((24, 2 * channels), np.int8),
                           np.zeros((channels, 24), np.int8), sh1, sh2)
    assert e.value.status == skv.ERR_ARG
    # a damaged map header is refused on load
    bad = bytearray(want)
    bad[64 + 514 * 16 * channels] = 48                     # rank 48
    with pytest.raises(skv.SkvError) as e:
        skv.load_tables(bytes(bad))
    assert e.value.status == skv.ERR_TABLES


def test_range_workspace_sizing_on_host(skv):
    """The workspace a range decode asks for needs no device: the status word,
    plus for a checkerboard blob one 256-token block of rows (the even tokens
    after the range); a whole decode needs only the status word."""
    for dtype, mode, channels, extra in [(skv.E4M3, skv.RESIDUAL, 64, 0), (skv.BF16, skv.RESIDUAL_EXP, 64, 0),
                                         (skv.INT16, skv.CHECKERBOARD, 64, 512 * 64)]:
        tabs = _small_tables(skv, dtype, mode, channels=channels)
        wb = ctypes.c_size_t()
        assert skv.lib().skv_decode_range(tabs.ptr, None, 0, 0, 256, None, None, 0, None, ctypes.byref(wb), None) == 0
        assert wb.value == 256 + extra
        assert skv.lib().skv_decode(tabs.ptr, None, 0, None, None, 0, None, ctypes.byref(wb), None) == 0
        assert wb.value == 256
        assert skv.range_aux_tokens(tabs, 1024, 256, 512) == (512 if extra else 256)
        assert skv.range_aux_tokens(tabs, 1024, 512, 1024) == 512


def test_encode_workspace_plans(skv):
    """Workspace budgets (host only): at or above the single-pass need, one
    pass of that size; below it, passes of whole slabs, then of token blocks
    of one slab, each within the budget and more of them as it shrinks;
    below one token block (or, for checkerboard shapes, below one pass)
    SKV_ERR_CAPACITY with the smallest workable size."""
    tabs = _small_tables(skv, skv.E4M3, skv.RESIDUAL, layers=2, channels=256)   # 4 slabs of 16 blocks x 8 groups
    T = 2048
    full, p1 = skv.encode_workspace(tabs, T)
    assert p1 == 1 and skv.encode_workspace(tabs, T, full) == (full, 1)
    raw = 4096
    per_stream = 2 * raw + 4                              # scratch and size word per stream
    seen = []
    for budget in (full - 1, full // 2, full // 4 + 4096, full // 5, full // 16, full // 40, 9 * per_stream):
        wb, passes = skv.encode_workspace(tabs, T, budget)
        assert wb <= budget and passes > 1, budget
        seen.append(passes)
    assert seen == sorted(seen)
    assert skv.encode_workspace(tabs, T, full // 4 + 4096)[1] == 4          # one slab per pass
    assert skv.encode_workspace(tabs, T, full // 5)[1] == 4 * 2             # 12 + 4 token blocks
    smallest = skv.encode_workspace(tabs, T, 1 << 30)[0]
    with pytest.raises(skv.SkvError) as e:
        skv.encode_workspace(tabs, T, 8 * per_stream - 1)
    assert e.value.status == skv.ERR_CAPACITY
    wb, passes = skv.encode_workspace(tabs, T, 8 * per_stream + 2048)
    assert passes == 4 * 16 and wb <= 8 * per_stream + 2048                # one token block per pass
    assert smallest == full
    tc = _small_tables(skv, skv.INT16, skv.CHECKERBOARD, channels=64)
    cfull, _ = skv.encode_workspace(tc, 2048)
    with pytest.raises(skv.SkvError) as e:
        skv.encode_workspace(tc, 2048, cfull - 1)
    assert e.value.status == skv.ERR_CAPACITY
