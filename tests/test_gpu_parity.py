"""GPU parity: containers and reconstructions from libskv's HIP kernels are
bit-identical to the CPU oracle's.

The coding path is integer end to end, so there is no tolerance: container
bytes must equal the oracle's byte for byte and the decode must return the
target exactly (lossless reconstruction, Speculative KV coding summary,
'Core idea'; checkerboard decoding in two passes, DCKV page, 'How it
differs').  Every case, the full-size workloads included, compares the
whole container (header, index, payload) with the oracle's, byte for byte,
and checks the exact GPU round trip.
"""
import ctypes
import os
import struct
import sys

import numpy as np
import pytest
import torch

from workloads import gen

pytestmark = pytest.mark.gpu

# host threads for the oracle: the CPU share of one GPU on the test machines
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def skv():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from lossless_kv_cache_amd import skv as m
    m.lib()
    return m


def _dt(cfg, skv):
    return {"bf16": skv.BF16, "e4m3": skv.E4M3, "int16": skv.INT16}[cfg.dtype]


def _parse(c: bytes):
    n = struct.unpack_from("<Q", c, 32)[0]
    idx = np.frombuffer(c[64:64 + 8 * (n + 1)], dtype=np.uint64)
    return n, idx, 64 + 8 * (n + 1)


def host_u8(x: torch.Tensor) -> np.ndarray:
    return x.cpu().numpy().reshape(-1).view(np.uint8)


def assert_same_container(got: np.ndarray, want: np.ndarray, what: str):
    """Byte-for-byte equality of two containers; a mismatch names the first
    differing part (header, index entry or stream)."""
    if got.size == want.size and np.array_equal(got, want):
        return
    m = min(got.size, want.size)
    diff = np.nonzero(got[:m] != want[:m])[0]
    first = int(diff[0]) if diff.size else m
    n = int(want[32:40].view(np.uint64)[0])
    head = 64 + 8 * (n + 1)
    if first < 64:
        where = f"header byte {first}"
    elif first < head:
        where = f"index entry {(first - 64) // 8}"
    else:
        offs = want[64:head].view(np.uint64) & np.uint64((1 << 63) - 1)
        where = f"stream {int(np.searchsorted(offs, np.uint64(first - head), side='right')) - 1}"
    raise AssertionError(f"{what}: container differs from the oracle's (sizes {got.size} / {want.size}; "
                         f"first difference at byte {first}, {where})")


def residual_case(skv, orc, cfg, device="cuda"):
    t, p = gen.residual_array(cfg, device=device)
    ct, cp = gen.residual_array(cfg, gen.CALIB, tokens=256, device=device)
    ct, cp = ct.cpu().numpy(), cp.cpu().numpy()
    dt = _dt(cfg, skv)
    tabs = skv.fit_tables(dt, skv.RESIDUAL, cfg.layers, cfg.kv, cfg.channels, ct, cp, 256)
    oshape = orc.make_shape(dt, orc.RESIDUAL, cfg.layers, cfg.kv, cfg.tokens, cfg.channels)
    return t, p, tabs, oshape


def full_compare(skv, orc, t, p, tabs, oshape, what):
    say(f"[parity] {what}: encode on GPU")
    cont = skv.encode(tabs, t, p)
    torch.cuda.synchronize()
    tn, pn = t.cpu().numpy(), p.cpu().numpy()
    say(f"[parity] {what}: encode with oracle")
    want_a = orc.encode_array(tabs.bytes(), oshape, tn, pn, threads=ORACLE_THREADS)
    assert_same_container(host_u8(cont), want_a, what)
    want = want_a.tobytes()
    say(f"[parity] {what}: decode on GPU")
    back = skv.decode(tabs, cont, p)
    assert torch.equal(back, t)
    # the GPU decodes the oracle's container as well
    back2 = skv.decode(tabs, torch.from_numpy(want_a.copy()).cuda(), p)
    assert torch.equal(back2, t)
    return want


def test_cfg0_full_container(skv, orc):
    cfg = gen.CONFIGS[0]
    t, p, tabs, oshape = residual_case(skv, orc, cfg)
    c = full_compare(skv, orc, t, p, tabs, oshape, "cfg0 bf16 1x2x1024x1024")
    say(f"[parity] cfg0 ratio {t.numel() * 2 / len(c):.3f}")


def test_ragged_grid_bf16(skv, orc):
    """1188 streams: several scan blocks with a partial last one, and a
    partial last workgroup of the encoder and decoder grids."""
    cfg = gen.Config(90, "ragged-bf16", "bf16", 6, 2, 1152, 352)
    t, p, tabs, oshape = residual_case(skv, orc, cfg)
    assert orc.n_streams(oshape) == 1188
    full_compare(skv, orc, t, p, tabs, oshape, "ragged bf16 6x2x1152x352")


@pytest.mark.parametrize("channels", [160, 256])
def test_e4m3_small(skv, orc, channels):
    """160 channels (5 channel groups) take the one-group encoder, 256 (a
    multiple of 4 groups) the two-group one; 640 tokens leave a partial
    round of token blocks."""
    cfg = gen.CONFIGS[2].with_tokens(640, layers=3, channels=channels)
    t, p, tabs, oshape = residual_case(skv, orc, cfg)
    full_compare(skv, orc, t, p, tabs, oshape, f"e4m3 3x2x640x{channels}")


def test_checkerboard_small(skv, orc):
    cfg = gen.CONFIGS[4].with_tokens(1280, channels=192)
    coef, G = gen.dckv_draw(cfg, device="cuda")
    cc, cg = gen.dckv_draw(cfg, gen.CALIB, tokens=256, device="cuda")
    tabs = skv.fit_tables(skv.INT16, skv.CHECKERBOARD, 1, 1, 192, cc.cpu().numpy(), cg.cpu().numpy(), 256)
    oshape = orc.make_shape(orc.INT16, orc.CHECKERBOARD, 1, 1, 1280, 192)
    full_compare(skv, orc, coef, G, tabs, oshape, "checkerboard 1280x192")


def test_checkerboard_escape_bursts_and_raw(skv, orc):
    """Checkerboard streams whose escaped values come in bursts (a run of
    coded steps where every lane escapes: more escaped values in 8 steps than
    the encoder keeps in LDS), one whose every value escapes (stored raw), and
    near-uniform values (a word from every lane at most steps); containers
    equal the oracle's, both decode exactly."""
    cfg = gen.CONFIGS[4].with_tokens(1280, channels=192)
    coef, G = gen.dckv_draw(cfg, device="cuda")
    cc, cg = gen.dckv_draw(cfg, gen.CALIB, tokens=256)
    tabs = skv.fit_tables(skv.INT16, skv.CHECKERBOARD, 1, 1, 192, cc.numpy(), cg.numpy(), 256)
    c = coef.cpu().numpy().copy()
    rng = np.random.default_rng(31)
    # even pass, token block 1, channel group 2: steps 16..39 all escaped (24 x 32 values)
    for k in range(16, 40):
        c[2 * (128 + k), 64:96] = rng.choice([30000, -30000, 29000, -29001], size=32)
    # odd pass, token block 0, channel group 1: steps 100..102 (96 escapes in one 8-step batch)
    for k in range(100, 103):
        c[2 * k + 1, 32:64] = rng.integers(-32768, 32768, size=32)
    # odd pass, token block 2, channel group 4: every value escapes -> stored raw
    for k in range(128):
        c[2 * (256 + k) + 1, 128:160] = rng.integers(-32768, 32768, size=32)
    # even pass, token block 3, channel group 5: values spread over 81 more cells (6,288 bytes, coded)
    for k in range(128):
        c[2 * (384 + k), 160:192] = np.clip(c[2 * (384 + k), 160:192].astype(np.int64)
                                            + rng.integers(-40, 41, size=32), -32768, 32767)
    coef = torch.from_numpy(c).cuda()
    oshape = orc.make_shape(orc.INT16, orc.CHECKERBOARD, 1, 1, 1280, 192)
    want = full_compare(skv, orc, coef, G, tabs, oshape, "checkerboard escape bursts and raw")
    n = orc.n_streams(oshape)
    idx = np.frombuffer(want, dtype=np.uint64, count=n + 1, offset=64)
    raw = idx >> np.uint64(63)
    assert raw[(1 * 5 + 2) * 6 + 4] == 1, "the all-escaped stream is stored raw"
    assert raw[(0 * 5 + 1) * 6 + 2] == 0 and raw[(1 * 5 + 0) * 6 + 1] == 0 and raw[(0 * 5 + 3) * 6 + 5] == 0


@pytest.mark.parametrize("tokens,channels", [(16384, 64), (32768, 160), (16640, 64)])
def test_checkerboard_block_orders(skv, orc, tokens, channels):
    """The checkerboard kernels' block orders: channel groups paired on an XCD
    (an even group count, 8 or more blocks per XCD), one group after another
    (an odd group count), and dispatch order (a block count that the 8 XCDs do
    not divide); whole containers equal the oracle's, both decode exactly."""
    cfg = gen.CONFIGS[4].with_tokens(tokens, channels=channels)
    coef, G = gen.dckv_draw(cfg, device="cuda")
    cc, cg = gen.dckv_draw(cfg, gen.CALIB, tokens=256)
    tabs = skv.fit_tables(skv.INT16, skv.CHECKERBOARD, 1, 1, channels, cc.numpy(), cg.numpy(), 256)
    oshape = orc.make_shape(orc.INT16, orc.CHECKERBOARD, 1, 1, tokens, channels)
    full_compare(skv, orc, coef, G, tabs, oshape, f"checkerboard {tokens}x{channels}")


def map_case(skv, orc, T, C, rank, device="cuda"):
    """Checkerboard data with a decoded-neighbour map of the given rank, its
    tables (fitted by the library) and the oracle's shape."""
    cfg = gen.CONFIGS[4].with_tokens(T, channels=C)
    V, U, sh1, sh2 = gen.dckv_map_weights(cfg, rank)
    coef, G = gen.dckv_draw(cfg, device=device, nbr_map=(V, U, sh1, sh2))
    cc, cg = gen.dckv_draw(cfg, gen.CALIB, tokens=256, nbr_map=(V, U, sh1, sh2))
    tabs = skv.fit_tables_map(C, cc.numpy(), cg.numpy(), 256, V, U, sh1, sh2)
    oshape = orc.make_shape(orc.INT16, orc.CHECKERBOARD_MAP, 1, 1, T, C)
    return coef, G, tabs, oshape, (V, U, sh1, sh2)


@pytest.mark.parametrize("rank", [16, 32, 64, 128, 256])
def test_checkerboard_map_small(skv, orc, rank):
    """The decoded-neighbour map on the int8 matrix units (every rank the blob
    allows): containers equal the oracle's, both decode exactly."""
    coef, G, tabs, oshape, _ = map_case(skv, orc, 1280, 192, rank)
    full_compare(skv, orc, coef, G, tabs, oshape, f"checkerboard map rank {rank}")


def test_checkerboard_map_extremes_and_unaligned(skv, orc):
    """Coefficients at the ends of int16 (the map's input saturation and both
    halves of the int8 split at their limits), side inputs at the ends of
    int16 (the clamp of G'), escapes; then the same through unaligned buffers
    (the map's element-load path)."""
    coef, G, tabs, oshape, _ = map_case(skv, orc, 768, 128, 64)
    c, g = coef.cpu().numpy().copy(), G.cpu().numpy().copy()
    rng = np.random.default_rng(23)
    for v in (32767, 32640, 32639, -32768, -32767, 255, -129):
        pos = rng.choice(c.size // 2, size=40, replace=False)
        rows, cols = np.divmod(pos, c.shape[1])
        c[2 * rows, cols] = v                              # even rows: the map's inputs
    pos = rng.choice(g.size // 2, size=60, replace=False)
    rows, cols = np.divmod(pos, g.shape[1])
    g[2 * rows + 1, cols] = rng.choice([32767, -32768, 32700, -32700], size=60)
    coef, G = torch.from_numpy(c).cuda(), torch.from_numpy(g).cuda()
    want = full_compare(skv, orc, coef, G, tabs, oshape, "checkerboard map extremes")
    cu, gu = _offset_copy(coef, 1), _offset_copy(G, 3)
    cont = skv.encode(tabs, cu, gu)
    torch.cuda.synchronize()
    assert cont.cpu().numpy().tobytes() == want
    out = _offset_copy(torch.zeros_like(coef), 1)
    skv.decode_into(tabs, cont, gu, out)
    assert torch.equal(out, coef)


def test_checkerboard_map_zero_equals_checkerboard(skv, orc):
    """U = 0 on the GPU: the map mode's index and payload equal the plain
    checkerboard mode's for the same data."""
    cfg = gen.CONFIGS[4].with_tokens(1024, channels=96)
    V, U, sh1, sh2 = gen.dckv_map_weights(cfg, 32)
    U = np.zeros_like(U)
    coef, G = gen.dckv_draw(cfg, device="cuda")
    cc, cg = gen.dckv_draw(cfg, gen.CALIB, tokens=256)
    tm = skv.fit_tables_map(96, cc.numpy(), cg.numpy(), 256, V, U, sh1, sh2)
    t1 = skv.fit_tables(skv.INT16, skv.CHECKERBOARD, 1, 1, 96, cc.numpy(), cg.numpy(), 256)
    cm, c1 = skv.encode(tm, coef, G), skv.encode(t1, coef, G)
    assert torch.equal(cm[64:], c1[64:])
    assert torch.equal(skv.decode(tm, cm, G), coef)


@pytest.mark.parametrize("kind", ["equal", "random", "maxz", "escapes"])
def test_edge_inputs(skv, orc, kind):
    """Degenerate inputs: target == predictor; incompressible (raw
    fallback); residual -2^15 everywhere (largest escape); every value
    escaping but still coded."""
    cfg = gen.Config(91, "edge-bf16", "bf16", 1, 2, 256, 96)
    t, p, tabs, oshape = residual_case(skv, orc, cfg)
    g = torch.Generator(device="cuda")
    g.manual_seed(17)
    if kind == "equal":
        t = p.clone()
    elif kind == "random":
        t = torch.randint(-32768, 32768, p.shape, generator=g, device="cuda", dtype=torch.int32).to(torch.int16)
    elif kind == "maxz":
        t = (p.to(torch.int32) ^ 0x8000).to(torch.int16)          # sign flip: r = -2^15 or near
    elif kind == "escapes":
        t = (p.to(torch.int32) + 300).to(torch.int16)             # |r| = 300 > every direct range
    full_compare(skv, orc, t, p, tabs, oshape, f"edge {kind}")


@pytest.mark.parametrize("channels", [96, 128])
@pytest.mark.parametrize("kind", ["equal", "random", "maxz", "escapes", "mixed"])
def test_edge_inputs_e4m3(skv, orc, kind, channels):
    """The same degenerate inputs for byte elements, on a grid with an odd
    number of token blocks (in the one-group encoder a wavefront runs one
    stream and idles the other half; 128 channels take the two-group
    encoder); "mixed" alternates compressible and raw token blocks."""
    cfg = gen.Config(92, "edge-e4m3", "e4m3", 2, 2, 640, channels)
    t, p, tabs, oshape = residual_case(skv, orc, cfg)
    g = torch.Generator(device="cuda")
    g.manual_seed(19)
    if kind == "equal":
        t = p.clone()
    elif kind == "random":
        t = torch.randint(0, 256, p.shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
    elif kind == "maxz":
        t = (p.to(torch.int32) ^ 0x80).to(torch.uint8)            # sign flip: residual near -128
    elif kind == "escapes":
        t = ((p.to(torch.int32) + 40) & 0xFF).to(torch.uint8)     # |r| about 40: past every direct range
    elif kind == "mixed":
        r = torch.randint(0, 256, p.shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
        blk = (torch.arange(p.shape[2], device="cuda") // 128) % 2 == 1
        t = torch.where(blk[None, None, :, None], r, t)
    full_compare(skv, orc, t, p, tabs, oshape, f"edge e4m3 {kind} {channels}")


def _ordered_noise(x: torch.Tensor, noise: float, seed: int) -> torch.Tensor:
    """e4m3 codes moved by N(0, noise^2) steps in value order (clamped at the
    ends), so residuals stay near the noise without sign-crossing jumps."""
    g = torch.Generator(device=x.device)
    g.manual_seed(seed)
    u = x.to(torch.int32)
    o = torch.where(u < 128, u ^ 0x80, u ^ 0xFF)
    o = (o + (torch.randn(x.shape, generator=g, device=x.device) * noise).round().to(torch.int32)).clamp(0, 255)
    return torch.where(o >= 128, o ^ 0x80, o ^ 0xFF).to(torch.uint8)


@pytest.mark.parametrize("noise,lo,hi", [(10, 64, 127), (24, 128, 255)])
def test_e4m3_wide_tables(skv, orc, noise, lo, hi):
    """Predictors noisier than the workload's widen the tables: 64 to 127
    direct symbols take the tiled e4m3 decoder with 128-row tables, 128 or
    more the per-table LDS decoder.  Containers equal the oracle's."""
    cfg = gen.Config(98, "wide-e4m3", "e4m3", 2, 2, 640, 128)
    t, _ = gen.residual_array(cfg, device="cuda")
    ct, _ = gen.residual_array(cfg, gen.CALIB, tokens=256)
    p, cp = _ordered_noise(t, noise, 1), _ordered_noise(ct, noise, 2)
    tabs = skv.fit_tables(skv.E4M3, skv.RESIDUAL, 2, 2, 128, ct.numpy(), cp.numpy(), 256)
    blob = tabs.bytes()
    ns = [int.from_bytes(blob[64 + 514 * j:66 + 514 * j], "little") for j in range(2 * 2 * 128)]
    assert lo <= max(ns) <= hi, (min(ns), max(ns))
    oshape = orc.make_shape(orc.E4M3, orc.RESIDUAL, 2, 2, 640, 128)
    full_compare(skv, orc, t, p, tabs, oshape, f"e4m3 tables up to {max(ns)} symbols")


@pytest.mark.parametrize("exp", [False, True])
def test_e4m3_encoders_many_draws(skv, orc, exp):
    """The e4m3 encoders (128 channels: the two-group coders, per-channel or
    exponent-class tables) over twelve seeded draws: three seeds, predictors
    at the workload's noise and moved by 2, 5 and 12 steps in value order, so
    streams range from a few words per step to near-raw.  Every container
    equals the oracle's and decodes exactly."""
    mode, omode = (skv.RESIDUAL_EXP, orc.RESIDUAL_EXP) if exp else (skv.RESIDUAL, orc.RESIDUAL)
    for seed in (90, 91, 92):
        cfg = gen.Config(seed, f"draws-e4m3-{seed}", "e4m3", 2, 2, 640, 128)
        t, p0 = gen.residual_array(cfg, device="cuda")
        ct, cp0 = gen.residual_array(cfg, gen.CALIB, tokens=256)
        for noise in (0, 2, 5, 12):
            p = p0 if noise == 0 else _ordered_noise(t, noise, seed)
            cp = cp0 if noise == 0 else _ordered_noise(ct, noise, seed + 100)
            tabs = skv.fit_tables(skv.E4M3, mode, 2, 2, 128, ct.numpy(), cp.numpy(), 256)
            oshape = orc.make_shape(orc.E4M3, omode, 2, 2, 640, 128)
            full_compare(skv, orc, t, p, tabs, oshape, f"e4m3 seed {seed} noise {noise} exp {exp}")


@pytest.mark.parametrize("exp", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_word_bursts_after_escapes(skv, orc, dtype, exp):
    """Every token block escapes in its first 4 steps and codes rare direct
    symbols (about 12 bits each) in the next 8, then repeats the predictor:
    the tiles after the escapes need more words than the decoder's ring holds,
    so they are decoded again from memory while the escapes of the tile before
    are being resolved.  The streams stay coded (not raw).  Per-channel and
    exponent-class tables."""
    cfg = gen.Config(93, f"burst-{dtype}", dtype, 1, 2, 512, 128 if exp else 96)
    t, p, tabs, oshape = exp_case(skv, orc, cfg) if exp else residual_case(skv, orc, cfg)
    step = (torch.arange(p.shape[2], device="cuda") % 128)[None, None, :, None]
    if dtype == "e4m3":
        far, rare, mask = 40, 20, 0xFF
    else:
        far, rare, mask = 300, 100, 0xFFFF
    pi = p.to(torch.int32)
    t = torch.where(step < 4, pi + far, torch.where(step < 12, pi + rare, pi)) & mask
    t = t.to(torch.uint8) if dtype == "e4m3" else t.to(torch.int16)
    full_compare(skv, orc, t, p, tabs, oshape, f"word bursts {dtype}")


def _offset_copy(x: torch.Tensor, k: int) -> torch.Tensor:
    """A contiguous copy of x whose data starts k elements into a larger buffer."""
    buf = torch.zeros(x.numel() + k, dtype=x.dtype, device=x.device)
    v = buf[k:k + x.numel()].view(x.shape)
    v.copy_(x)
    return v


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_unaligned_buffers(skv, orc, dtype):
    """Target, predictor and output that are not 16-byte aligned take the
    per-step kernels (the tiled ones move 8- and 16-byte pieces); their
    containers and reconstructions are the same."""
    cfg = gen.Config(94, f"unaligned-{dtype}", dtype, 1, 2, 384, 128)
    t, p, tabs, oshape = residual_case(skv, orc, cfg)
    tu, pu = _offset_copy(t, 1), _offset_copy(p, 3)
    assert tu.data_ptr() % 8 != 0 and pu.data_ptr() % 8 != 0
    say(f"[parity] unaligned {dtype}: encode on GPU")
    cont = skv.encode(tabs, tu, pu)
    torch.cuda.synchronize()
    want = orc.encode(tabs.bytes(), oshape, t.cpu().numpy(), p.cpu().numpy(), threads=8)
    assert cont.cpu().numpy().tobytes() == want
    out = _offset_copy(torch.zeros_like(t), 1)
    skv.decode_into(tabs, cont, pu, out)
    assert torch.equal(out, t)


def exp_case(skv, orc, cfg):
    t, p = gen.residual_array(cfg, device="cuda")
    ct, cp = gen.residual_array(cfg, gen.CALIB, tokens=256)
    dt = _dt(cfg, skv)
    tabs = skv.fit_tables(dt, skv.RESIDUAL_EXP, cfg.layers, cfg.kv, cfg.channels, ct.numpy(), cp.numpy(), 256)
    oshape = orc.make_shape(dt, orc.RESIDUAL_EXP, cfg.layers, cfg.kv, cfg.tokens, cfg.channels)
    return t, p, tabs, oshape


@pytest.mark.parametrize("cid", [0, 2])
def test_exponent_mode_small(skv, orc, cid):
    """Exponent-conditioned tables: containers byte-identical to the oracle's,
    exact decode of both, and a range decode."""
    cfg = gen.CONFIGS[cid].with_tokens(640, layers=2, channels=192)
    t, p, tabs, oshape = exp_case(skv, orc, cfg)
    want = full_compare(skv, orc, t, p, tabs, oshape, f"exponent mode {cfg.dtype}")
    assert want[7] == orc.RESIDUAL_EXP
    cont = torch.from_numpy(np.frombuffer(want, dtype=np.uint8).copy()).cuda()
    part = skv.decode_range(tabs, cont, 256, 512, p[:, :, 256:512].contiguous())
    assert torch.equal(part, t[:, :, 256:512])


@pytest.mark.parametrize("dtype", ["e4m3", "bf16"])
def test_exponent_mode_escapes_and_unaligned(skv, orc, dtype):
    """Exponent mode through every kernel path: rare far residuals (escapes in
    every class, with bursts of words), the tiled kernels on aligned buffers and
    the per-step ones on unaligned buffers; all containers equal the oracle's."""
    cfg = gen.Config(99, "exp-escapes", dtype, 1, 2, 512, 128)
    t, p, tabs, oshape = exp_case(skv, orc, cfg)
    rng = np.random.default_rng(21)
    tn = t.cpu().numpy()
    flat = tn.reshape(-1)
    pos = rng.choice(flat.size, size=flat.size // 200, replace=False)
    hi = 256 if dtype == "e4m3" else 65536
    flat[pos] = rng.integers(0, hi, size=pos.size).astype(np.int64).astype(flat.dtype)
    t = torch.from_numpy(tn).cuda()
    want = full_compare(skv, orc, t, p, tabs, oshape, "exponent mode escapes")
    tu, pu = _offset_copy(t, 1), _offset_copy(p, 3)
    cont = skv.encode(tabs, tu, pu)
    torch.cuda.synchronize()
    assert cont.cpu().numpy().tobytes() == want
    out = _offset_copy(torch.zeros_like(t), 1)
    skv.decode_into(tabs, cont, pu, out)
    assert torch.equal(out, t)


@pytest.mark.parametrize("dtype,exp,aligned", [("e4m3", True, True), ("e4m3", False, True), ("bf16", True, True),
                                               ("bf16", False, True), ("e4m3", False, False), ("bf16", True, False)])
def test_corruption_verdicts(skv, orc, dtype, exp, aligned):
    """Damaged containers (either element type, per-channel or exponent-class
    tables; unaligned buffers take the per-table LDS or per-stream decoder):
    the decoder reaches the oracle's verdict on every bit flip in the coded
    part of a stream (a flip can leave a consistent stream, which both then
    decode alike), and refuses an index past the payload and another blob."""
    cfg = gen.Config(100, f"corrupt-{dtype}", dtype, 1, 2, 512, 128)
    t, p, tabs, oshape = exp_case(skv, orc, cfg) if exp else residual_case(skv, orc, cfg)
    cont = skv.encode(tabs, t, p)
    good = cont.cpu().numpy()
    pd = p if aligned else _offset_copy(p, 1)

    def dec(tables, c):
        out = torch.zeros_like(t) if aligned else _offset_copy(torch.zeros_like(t), 1)
        return skv.decode_into(tables, c, pd, out)

    n, idx, head = _parse(good.tobytes())
    rng = np.random.default_rng(8)
    pn, tn = p.cpu().numpy(), t.cpu().numpy()
    trials = refused = 0
    while trials < 24:
        st = int(rng.integers(0, n))
        if idx[st] >> np.uint64(63):
            continue
        a = int(idx[st] & np.uint64((1 << 63) - 1))
        nw = int.from_bytes(good[head + a + 128:head + a + 132].tobytes(), "little")
        bad = good.copy()
        pos = head + int(rng.integers(a, a + 132 + 2 * nw))
        bad[pos] ^= np.uint8(1 << int(rng.integers(0, 8)))
        say(f"[parity] {dtype} corrupt trial {trials} (exponent tables {exp}, aligned {aligned}): stream {st} byte {pos}")
        want = np.zeros_like(tn)
        rc = orc.decode_rc(tabs.bytes(), bad.tobytes(), pn, want)
        if rc == orc.E_CORRUPT:
            with pytest.raises(skv.SkvError) as e:
                dec(tabs, torch.from_numpy(bad).cuda())
            assert e.value.status == skv.ERR_CORRUPT
            refused += 1
        else:
            assert rc == orc.OK
            assert np.array_equal(dec(tabs, torch.from_numpy(bad).cuda()).cpu().numpy(), want)
        trials += 1
    assert refused >= 20
    bad = good.copy()
    bad[64 + 8 * 3:64 + 8 * 4] = np.frombuffer(struct.pack("<Q", 1 << 40), np.uint8)
    with pytest.raises(skv.SkvError) as e:
        dec(tabs, torch.from_numpy(bad).cuda())
    assert e.value.status == skv.ERR_CORRUPT
    ct, cp = gen.residual_array(cfg, gen.CALIB, tokens=256)
    other = skv.fit_tables(_dt(cfg, skv), skv.RESIDUAL if exp else skv.RESIDUAL_EXP, 1, 2, 128, ct.numpy(), cp.numpy(),
                           256)
    with pytest.raises(skv.SkvError) as e:
        dec(other, cont)
    assert e.value.status == skv.ERR_TABLES
    assert torch.equal(dec(tabs, cont), t)


def test_exponent_mode_full_size_e4m3(skv, orc):
    """The Qwen3-8B-shaped e4m3 cache with exponent-conditioned tables: the
    whole container equals the oracle's, the round trip is exact, and the
    container is smaller than with per-channel tables."""
    cfg = gen.CONFIGS[2]
    say(f"[parity] exponent mode cfg2: generating {cfg.values} values on GPU")
    t, p, tabs, oshape = exp_case(skv, orc, cfg)
    big_compare(skv, orc, t, p, tabs, oshape, "exponent mode cfg2", min_ratio=4.5)


@pytest.mark.parametrize("cid", [1, 3])
def test_exponent_mode_full_size_bf16(skv, orc, cid):
    """The Qwen3-0.6B- and Qwen3-32B-shaped bf16 caches with exponent-conditioned
    tables (the tiled bf16 kernels with the slab's 16 class tables): whole
    container equal to the oracle's, exact round trip."""
    cfg = gen.CONFIGS[cid]
    say(f"[parity] exponent mode cfg{cid}: generating {cfg.values} values on GPU")
    t, p, tabs, oshape = exp_case(skv, orc, cfg)
    big_compare(skv, orc, t, p, tabs, oshape, f"exponent mode cfg{cid}", min_ratio=2.5)


RANGES = [(0, 1024), (0, 128), (896, 1024), (256, 640), (128, 1024)]


@pytest.mark.parametrize("dtype,aligned,exp", [("e4m3", True, False), ("e4m3", False, False), ("bf16", True, False),
                                               ("bf16", False, False), ("e4m3", True, True), ("bf16", True, True),
                                               ("e4m3", False, True), ("bf16", False, True)])
def test_decode_range(skv, orc, dtype, aligned, exp):
    """A token range decoded through the offset index equals the same tokens
    of the oracle's decode of the whole container (decode_e4m3 / decode_bf16
    with per-channel or exponent-class tables, or the per-table LDS decoder
    for unaligned buffers)."""
    cfg = gen.Config(95, f"range-{dtype}", dtype, 2, 2, 1024, 256)
    t, p, tabs, oshape = (exp_case if exp else residual_case)(skv, orc, cfg)
    cont = skv.encode(tabs, t, p)
    torch.cuda.synchronize()
    pn = p.cpu().numpy()
    say(f"[parity] range {dtype}: oracle decode of the whole container")
    want = orc.decode(tabs.bytes(), cont.cpu().numpy().tobytes(), pn, pn, threads=8)
    assert np.array_equal(want, t.cpu().numpy())
    for a, b in RANGES:
        say(f"[parity] range {dtype} aligned={aligned} exp={exp}: tokens [{a}, {b})")
        pr = p[:, :, a:b].contiguous()
        out = torch.zeros_like(pr)
        if not aligned:
            pr, out = _offset_copy(pr, 1), _offset_copy(out, 1)
        skv.decode_range_into(tabs, cont, a, b, pr, out)
        assert np.array_equal(out.cpu().numpy(), want[:, :, a:b]), (a, b)


def test_decode_range_errors(skv, orc):
    cfg = gen.Config(96, "range-errors", "e4m3", 1, 2, 512, 64)
    t, p, tabs, oshape = residual_case(skv, orc, cfg)
    cont = skv.encode(tabs, t, p)
    for a, b in [(0, 100), (64, 192), (256, 256), (384, 128), (0, 640)]:
        pr = torch.zeros((1, 2, max(b - a, 128), 64), dtype=p.dtype, device="cuda")
        with pytest.raises(skv.SkvError) as e:
            skv.decode_range(tabs, cont, a, b, pr)
        assert e.value.status == skv.ERR_SHAPE, (a, b)
    with pytest.raises(skv.SkvError) as e:
        skv.decode_range_into(tabs, cont, 128, 384, p[:, :, 128:384].contiguous(),
                              torch.empty(10, dtype=torch.uint8, device="cuda"))
    assert e.value.status == skv.ERR_CAPACITY
    # a predictor shorter than the container's tokens: the capacity passed is
    # the smaller of the two buffers, so the library refuses it
    with pytest.raises(skv.SkvError) as e:
        skv.decode_into(tabs, cont, p[:, :, :256].contiguous(), torch.empty_like(p))
    assert e.value.status == skv.ERR_CAPACITY
    # a damaged stream inside the range is found; one outside it is not read
    good = cont.cpu().numpy()
    n, idx, head = _parse(good.tobytes())
    ntb, ncg = 512 // 128, 64 // 32
    for tb, inside in [(1, True), (3, False)]:
        s = (0 * ntb + tb) * ncg + 1                       # slab 0, channel group 1
        assert not (idx[s] >> np.uint64(63))
        a = int(idx[s] & np.uint64((1 << 63) - 1))
        bad = good.copy()
        bad[head + a + 5] ^= np.uint8(0x40)                # a final state byte
        pr = p[:, :, 128:256].contiguous()
        say(f"[parity] range damage in token block {tb}")
        if inside:
            bad_cont = torch.from_numpy(bad).cuda()
            with pytest.raises(skv.SkvError) as e:
                skv.decode_range(tabs, bad_cont, 128, 256, pr)
            assert e.value.status == skv.ERR_CORRUPT
        else:
            out = skv.decode_range(tabs, torch.from_numpy(bad).cuda(), 128, 256, pr)
            assert torch.equal(out, t[:, :, 128:256])
    # checkerboard ranges: whole 256-token blocks, and the side input of the block after the range
    cb = gen.CONFIGS[4].with_tokens(512, channels=64)
    coef, G = gen.dckv_draw(cb, device="cuda")
    cc, cgl = gen.dckv_draw(cb, gen.CALIB, tokens=256, device="cuda")
    ctabs = skv.fit_tables(skv.INT16, skv.CHECKERBOARD, 1, 1, 64, cc.cpu().numpy(), cgl.cpu().numpy(), 256)
    ccont = skv.encode(ctabs, coef, G)
    for a, b in [(0, 128), (128, 384), (256, 256), (0, 768)]:
        with pytest.raises(skv.SkvError) as e:
            skv.decode_range(ctabs, ccont, a, b, G[:256].contiguous())
        assert e.value.status == skv.ERR_SHAPE, (a, b)
    with pytest.raises(ValueError, match="shape"):
        skv.decode_range(ctabs, ccont, 0, 256, G[:256].contiguous())      # the next block's G is missing
    assert torch.equal(skv.decode_range(ctabs, ccont, 0, 256, G), coef[:256])
    assert torch.equal(skv.decode_range(ctabs, ccont, 256, 512, G[256:].contiguous()), coef[256:])


@pytest.mark.parametrize("mapped", [False, True])
def test_decode_range_checkerboard(skv, orc, mapped):
    """Checkerboard ranges (with and without the decoded-neighbour map) equal
    the same tokens of the oracle's decode of the whole container.  A range
    that stops early decodes the even stream of the next block too: damage
    there is found, damage in that block's odd stream is not read."""
    T, C = 2048, 192
    if mapped:
        coef, G, tabs, oshape, _ = map_case(skv, orc, T, C, 64)
    else:
        cfg = gen.CONFIGS[4].with_tokens(T, channels=C)
        coef, G = gen.dckv_draw(cfg, device="cuda")
        cc, cgl = gen.dckv_draw(cfg, gen.CALIB, tokens=256)
        tabs = skv.fit_tables(skv.INT16, skv.CHECKERBOARD, 1, 1, C, cc.numpy(), cgl.numpy(), 256)
    cont = skv.encode(tabs, coef, G)
    torch.cuda.synchronize()
    Gn = G.cpu().numpy()
    want = orc.decode(tabs.bytes(), cont.cpu().numpy().tobytes(), Gn, Gn, threads=8)
    assert np.array_equal(want, coef.cpu().numpy())
    for a, b in [(0, 256), (0, T), (256, 768), (T - 256, T), (512, 1536), (1536, 1792), (0, T - 256)]:
        say(f"[parity] checkerboard range mapped={mapped}: tokens [{a}, {b})")
        aux = G[a:min(T, b + 256)].contiguous()
        out = skv.decode_range(tabs, cont, a, b, aux)
        assert np.array_equal(out.cpu().numpy(), want[a:b]), (a, b)
    good = cont.cpu().numpy()
    n, idx, head = _parse(good.tobytes())
    ntb, ncg = T // 256, C // 32
    for ps, detected in [(0, True), (1, False)]:
        s_ = (ps * ntb + 3) * ncg + 1                     # block 3 (after the range [256, 768)), group 1
        assert not (idx[s_] >> np.uint64(63))
        off = int(idx[s_] & np.uint64((1 << 63) - 1))
        bad = good.copy()
        bad[head + off + 5] ^= np.uint8(0x40)               # a final state byte
        say(f"[parity] checkerboard range damage in pass {ps} of the next block")
        bad_cont = torch.from_numpy(bad).cuda()
        if detected:
            with pytest.raises(skv.SkvError) as e:
                skv.decode_range(tabs, bad_cont, 256, 768, G[256:1024].contiguous())
            assert e.value.status == skv.ERR_CORRUPT
        else:
            out = skv.decode_range(tabs, bad_cont, 256, 768, G[256:1024].contiguous())
            assert np.array_equal(out.cpu().numpy(), want[256:768])


def test_checkerboard_corruption_verdicts(skv, orc):
    """Damaged checkerboard containers: the decoder reaches the oracle's verdict
    on every bit flip anywhere in a coded stream (states, word count, words,
    escaped values, pad), in even and odd passes; where the stream stays
    consistent both decode alike."""
    cfg = gen.CONFIGS[4].with_tokens(1024, channels=128)
    coef, G = gen.dckv_draw(cfg, device="cuda")
    cc, cg = gen.dckv_draw(cfg, gen.CALIB, tokens=256)
    tabs = skv.fit_tables(skv.INT16, skv.CHECKERBOARD, 1, 1, 128, cc.numpy(), cg.numpy(), 256)
    c = coef.cpu().numpy().copy()
    rng = np.random.default_rng(41)
    for k in range(20, 30):                                # escaped values in an odd-pass stream
        c[2 * k + 1, 0:32] = rng.integers(-32768, 32768, size=32)
    coef = torch.from_numpy(c).cuda()
    cont = skv.encode(tabs, coef, G)
    good = cont.cpu().numpy()
    n, idx, head = _parse(good.tobytes())
    gn = G.cpu().numpy()
    trials = refused = 0
    while trials < 32:
        st = int(rng.integers(0, n))
        if idx[st] >> np.uint64(63):
            continue
        a = int(idx[st] & np.uint64((1 << 63) - 1))
        b = int(idx[st + 1] & np.uint64((1 << 63) - 1))
        bad = good.copy()
        pos = head + int(rng.integers(a, b))
        bad[pos] ^= np.uint8(1 << int(rng.integers(0, 8)))
        say(f"[parity] checkerboard corrupt trial {trials}: stream {st} byte {pos}")
        want = np.zeros_like(c)
        rc = orc.decode_rc(tabs.bytes(), bad.tobytes(), gn, want)
        if rc == orc.E_CORRUPT:
            with pytest.raises(skv.SkvError) as e:
                skv.decode(tabs, torch.from_numpy(bad).cuda(), G)
            assert e.value.status == skv.ERR_CORRUPT
            refused += 1
        else:
            assert rc == orc.OK
            assert np.array_equal(skv.decode(tabs, torch.from_numpy(bad).cuda(), G).cpu().numpy(), want)
        trials += 1
    assert refused >= 16
    assert torch.equal(skv.decode(tabs, cont, G), coef)


def test_corruption_and_wrong_tables(skv, orc):
    cfg = gen.Config(92, "corrupt-bf16", "bf16", 1, 2, 256, 64)
    t, p, tabs, oshape = residual_case(skv, orc, cfg)
    cont = skv.encode(tabs, t, p)
    good = cont.cpu().numpy()
    n, idx, head = _parse(good.tobytes())
    rng = np.random.default_rng(4)
    for trial in range(6):
        bad = good.copy()
        s = int(rng.integers(0, n))
        a = int(idx[s] & np.uint64((1 << 63) - 1))
        b = int(idx[s + 1] & np.uint64((1 << 63) - 1))
        if idx[s] >> np.uint64(63):
            continue
        # the coded part (states, word count, words); escaped raw values and raw
        # streams carry no redundancy, so a flip there is not detectable
        nw = int.from_bytes(good[head + a + 128:head + a + 132].tobytes(), "little")
        pos = head + int(rng.integers(a, a + 132 + 2 * nw))
        bad[pos] ^= np.uint8(1 << int(rng.integers(0, 8)))
        say(f"[parity] corrupt trial {trial}: stream {s} byte {pos}")
        with pytest.raises(skv.SkvError) as e:
            skv.decode(tabs, torch.from_numpy(bad).cuda(), p)
        assert e.value.status == skv.ERR_CORRUPT
    # index pointing past the payload
    bad = good.copy()
    bad[64 + 8 * 3:64 + 8 * 4] = np.frombuffer(struct.pack("<Q", 1 << 40), np.uint8)
    with pytest.raises(skv.SkvError) as e:
        skv.decode(tabs, torch.from_numpy(bad).cuda(), p)
    assert e.value.status == skv.ERR_CORRUPT
    # truncated container
    with pytest.raises(skv.SkvError) as e:
        skv.decode(tabs, cont[:-8].contiguous(), p)
    assert e.value.status == skv.ERR_CORRUPT
    # another blob
    ct2, cp2 = gen.residual_array(cfg.with_tokens(256), gen.EVAL, tokens=256)
    other = skv.fit_tables(skv.BF16, skv.RESIDUAL, 1, 2, 64, ct2.numpy(), cp2.numpy(), 256)
    with pytest.raises(skv.SkvError) as e:
        skv.decode(other, cont, p)
    assert e.value.status == skv.ERR_TABLES
    # output too small
    with pytest.raises(skv.SkvError) as e:
        skv.decode_into(tabs, cont, p, torch.empty(10, dtype=torch.int16, device="cuda"))
    assert e.value.status == skv.ERR_CAPACITY
    assert torch.equal(skv.decode(tabs, cont, p), t)


# ------------------------------------------------------------------ full-size workloads
def big_compare(skv, orc, t, p, tabs, oshape, what, min_ratio=None):
    """Whole-container parity at full size: the GPU container equals the
    oracle's byte for byte (every index entry and stream), then the GPU
    decodes it and the reconstruction is compared with the target in HBM."""
    say(f"[parity] {what}: encode on GPU")
    cont = skv.encode(tabs, t, p)
    torch.cuda.synchronize()
    raw_bytes = t.numel() * t.element_size()
    say(f"[parity] {what}: container {cont.numel()} B, ratio {raw_bytes / cont.numel():.4f}")
    if min_ratio is not None:
        assert raw_bytes / cont.numel() > min_ratio
    got = host_u8(cont)
    tn, pn = t.cpu().numpy(), p.cpu().numpy()
    say(f"[parity] {what}: oracle encode on {ORACLE_THREADS} threads")
    want = orc.encode_array(tabs.bytes(), oshape, tn, pn, threads=ORACLE_THREADS)
    del tn, pn
    assert_same_container(got, want, what)
    del got, want
    say(f"[parity] {what}: containers identical; decoding on GPU")
    back = skv.decode(tabs, cont, p)
    assert torch.equal(back, t)
    say(f"[parity] {what}: round trip exact")
    return cont


@pytest.mark.parametrize("cid", [1, 2, 3])
def test_full_size_residual(skv, orc, cid):
    cfg = gen.CONFIGS[cid]
    say(f"[parity] cfg{cid} {cfg.name}: generating {cfg.values} values on GPU")
    t, p, tabs, oshape = residual_case(skv, orc, cfg)
    big_compare(skv, orc, t, p, tabs, oshape, f"cfg{cid}")


def test_slab_over_2gib(skv, orc):
    """A (layer, K|V) slab of 2 GiB (2^21 tokens x 1024 e4m3 channels) is past
    the tiled kernels' 32-bit row offsets, so it takes the per-step encoder and
    decoder; the whole container equals the oracle's, the round trip is exact,
    and a range at the slab's end decodes through the tiled decoder."""
    cfg = gen.Config(97, "slab-2gib-e4m3", "e4m3", 1, 1, 1 << 21, 1024, outliers=False)
    say(f"[parity] 2 GiB slab: generating {cfg.values} values on GPU")
    t, p, tabs, oshape = residual_case(skv, orc, cfg)
    cont = big_compare(skv, orc, t, p, tabs, oshape, "2 GiB slab")
    a = cfg.tokens - 256
    part = skv.decode_range(tabs, cont, a, cfg.tokens, p[:, :, a:].contiguous())
    assert torch.equal(part, t[:, :, a:])
    say("[parity] 2 GiB slab: end range exact")


def test_full_size_checkerboard(skv, orc):
    cfg = gen.CONFIGS[4]
    say("[parity] cfg4: generating")
    coef, G = gen.dckv_draw(cfg, device="cuda")
    cc, cg = gen.dckv_draw(cfg, gen.CALIB, tokens=256, device="cuda")
    tabs = skv.fit_tables(skv.INT16, skv.CHECKERBOARD, 1, 1, cfg.channels, cc.cpu().numpy(), cg.cpu().numpy(), 256)
    oshape = orc.make_shape(orc.INT16, orc.CHECKERBOARD, 1, 1, cfg.tokens, cfg.channels)
    big_compare(skv, orc, coef, G, tabs, oshape, "cfg4 checkerboard")


def test_full_size_checkerboard_map(skv, orc):
    """The DCKV coefficient workload (131072 tokens x 2048 coefficients) with a
    rank-64 decoded-neighbour map: whole container equal to the oracle's,
    exact round trip, smaller than the plain checkerboard container."""
    cfg = gen.CONFIGS[4]
    say("[parity] cfg4 with the neighbour map: generating")
    coef, G, tabs, oshape, _ = map_case(skv, orc, cfg.tokens, cfg.channels, 64)
    cont = big_compare(skv, orc, coef, G, tabs, oshape, "cfg4 neighbour map")
    cc, cg = gen.dckv_draw(cfg, gen.CALIB, tokens=256, nbr_map=gen.dckv_map_weights(cfg, 64))
    plain = skv.fit_tables(skv.INT16, skv.CHECKERBOARD, 1, 1, cfg.channels, cc.numpy(), cg.numpy(), 256)
    c1 = skv.encode(plain, coef, G)
    say(f"[parity] cfg4 neighbour map: {cont.numel()} B against {c1.numel()} B without the map")
    assert cont.numel() < c1.numel()


@pytest.mark.parametrize("cid,exp,layers,lpc", [(0, False, 5, 2), (2, True, 3, 1), (2, False, 4, 4)])
def test_transfer_pipeline(skv, orc, cid, exp, layers, lpc):
    """Chunked encode -> host -> decode: every chunk on the wire is
    byte-identical to the oracle's container of those layers, with tables the
    oracle fits on those layers' calibration alone; the reconstruction is
    exact; a chunk container decodes on its own."""
    cfg = gen.CONFIGS[cid].with_tokens(384, layers=layers, channels=160)
    dt = _dt(cfg, skv)
    mode, omode = (skv.RESIDUAL_EXP, orc.RESIDUAL_EXP) if exp else (skv.RESIDUAL, orc.RESIDUAL)
    t, p = gen.residual_array(cfg, device="cuda")
    ct, cp = [a.numpy() for a in gen.residual_array(cfg, gen.CALIB, tokens=256)]
    tabs = skv.fit_tables(dt, mode, layers, cfg.kv, cfg.channels, ct, cp, 256)
    say(f"[parity] transfer {cfg.dtype} exp={exp} layers={layers} per chunk={lpc}")
    recv_p = p.clone()
    out, wire, offs = skv.transfer(tabs, t, p, recv_p, lpc)
    assert torch.equal(out, t)
    wire = wire.numpy().tobytes()
    nc = -(-layers // lpc)
    assert len(offs) == nc + 1 and offs[0] == 0 and offs[-1] == len(wire)
    tn, pn = t.cpu().numpy(), p.cpu().numpy()
    for c in range(nc):
        l0, l1 = c * lpc, min(layers, (c + 1) * lpc)
        oshape = orc.make_shape(dt, omode, l1 - l0, cfg.kv, cfg.tokens, cfg.channels)
        blob = orc.fit_tables(oshape, np.ascontiguousarray(ct[l0:l1]), np.ascontiguousarray(cp[l0:l1]), 256)
        want = orc.encode(blob, oshape, np.ascontiguousarray(tn[l0:l1]), np.ascontiguousarray(pn[l0:l1]), threads=8)
        assert wire[offs[c]:offs[c + 1]] == want, c
        if c == nc - 1:
            part = skv.load_tables(blob)
            chunk = torch.from_numpy(np.frombuffer(want, dtype=np.uint8).copy()).cuda()
            assert torch.equal(skv.decode(part, chunk, p[l0:l1].contiguous()), t[l0:l1])


def test_transfer_wire_too_small(skv, orc):
    """A wire buffer that cannot hold the first chunk stops the pipeline with
    SKV_ERR_CAPACITY; the same object then runs with a buffer of the bound."""
    cfg = gen.CONFIGS[0].with_tokens(256, layers=3, channels=64)
    t, p = gen.residual_array(cfg, device="cuda")
    ct, cp = [a.numpy() for a in gen.residual_array(cfg, gen.CALIB, tokens=256)]
    tabs = skv.fit_tables(skv.BF16, skv.RESIDUAL, 3, cfg.kv, cfg.channels, ct, cp, 256)
    tr = skv.Transfer(tabs, cfg.tokens, 1)
    full = tr.wire
    tr.wire = full[:1000]
    out = torch.zeros_like(t)
    with pytest.raises(skv.SkvError) as e:
        tr(t, p, p, out)
    assert e.value.status == skv.ERR_CAPACITY
    tr.wire = full
    tr(t, p, p, out)
    assert torch.equal(out, t)


def test_transfer_full_size_e4m3(skv, orc):
    """The Qwen3-8B-shaped e4m3 cache in chunks of 4 layers: exact
    reconstruction, and every chunk container on the wire equals the oracle's
    container of those layers, coded with tables the oracle fits on those
    layers' calibration alone."""
    cfg = gen.CONFIGS[2]
    say(f"[parity] transfer cfg2: generating {cfg.values} values on GPU")
    t, p = gen.residual_array(cfg, device="cuda")
    ct, cp = [a.numpy() for a in gen.residual_array(cfg, gen.CALIB, tokens=256)]
    tabs = skv.fit_tables(skv.E4M3, skv.RESIDUAL, cfg.layers, cfg.kv, cfg.channels, ct, cp, 256)
    tr = skv.Transfer(tabs, cfg.tokens, 4)
    out = torch.empty_like(t)
    wire, offs = tr(t, p, p, out)
    assert torch.equal(out, t)
    ratio = cfg.raw_bytes / wire.numel()
    say(f"[parity] transfer cfg2: {len(offs) - 1} chunks, ratio {ratio:.4f}")
    assert ratio > 3.5
    w = wire.numpy()
    tn, pn = t.cpu().numpy(), p.cpu().numpy()
    for c in range(len(offs) - 1):
        l0, l1 = 4 * c, min(cfg.layers, 4 * c + 4)
        oshape = orc.make_shape(orc.E4M3, orc.RESIDUAL, l1 - l0, cfg.kv, cfg.tokens, cfg.channels)
        blob = orc.fit_tables(oshape, np.ascontiguousarray(ct[l0:l1]), np.ascontiguousarray(cp[l0:l1]), 256)
        want = orc.encode_array(blob, oshape, tn[l0:l1], pn[l0:l1], threads=ORACLE_THREADS)
        assert_same_container(w[offs[c]:offs[c + 1]], want, f"transfer chunk {c}")
        say(f"[parity] transfer cfg2: chunk {c} identical to the oracle's")


@pytest.mark.parametrize("dtype,mode", [("e4m3", 0), ("bf16", 0), ("e4m3", 2), ("bf16", 2)])
def test_encode_in_passes(skv, orc, dtype, mode):
    """A workspace below the single-pass need codes the cache in passes (whole
    slabs, with a ragged last pass; token blocks of one slab; one block per
    pass), each into the same workspace: every container equals the oracle's
    byte for byte, and an output too small is refused with the size needed."""
    cfg = gen.Config(98, f"passes-{dtype}", dtype, 3, 2, 2048, 256, outliers=dtype == "bf16")
    t, p = gen.residual_array(cfg, device="cuda")
    ct, cp = gen.residual_array(cfg, gen.CALIB, tokens=256)
    dt = _dt(cfg, skv)
    tabs = skv.fit_tables(dt, mode, cfg.layers, cfg.kv, cfg.channels, ct.numpy(), cp.numpy(), 256)
    oshape = orc.make_shape(dt, mode, cfg.layers, cfg.kv, cfg.tokens, cfg.channels)
    want = orc.encode_array(tabs.bytes(), oshape, t.cpu().numpy(), p.cpu().numpy(), threads=ORACLE_THREADS)
    T = cfg.tokens
    full, _ = skv.encode_workspace(tabs, T)
    per_block = 8 * 2 * 4096 * cfg.elem_bytes + 4096       # 8 channel groups of scratch, with room for the rest
    seen = set()
    for budget in (0, full * 2 // 3 + 4096, full // 2, full // 4, full // 7, full // 20, per_block):
        wb, passes = skv.encode_workspace(tabs, T, budget)
        enc = skv.Encoder(tabs, T, max_work_bytes=budget)
        assert enc.passes == passes and enc.work.numel() == wb
        say(f"[parity] {dtype} mode {mode}: {passes} passes in {wb} B of workspace")
        got = enc(t, p)
        assert_same_container(host_u8(got), want, f"{dtype} mode {mode}, {passes} passes")
        seen.add(passes)
        if passes > 1:
            with pytest.raises(skv.SkvError) as e:
                lib_out = torch.empty(1000, dtype=torch.uint8, device="cuda")
                ob, wbuf = ctypes.c_size_t(), ctypes.c_size_t(enc.work.numel())
                shape = tabs.shape(T)
                skv._check(skv.lib().skv_encode(tabs.ptr, ctypes.byref(shape), t.data_ptr(), p.data_ptr(),
                                                lib_out.data_ptr(), lib_out.numel(), ctypes.byref(ob),
                                                enc.work.data_ptr(), ctypes.byref(wbuf), skv._stream()), "skv_encode")
            assert e.value.status == skv.ERR_CAPACITY and ob.value == want.size
    assert len(seen) >= 6, seen
    assert torch.equal(skv.decode(tabs, got, p), t)


@pytest.mark.parametrize("dtype", ["e4m3", "bf16"])
def test_encode_in_passes_raw_and_escapes(skv, orc, dtype):
    """Passes over a cache whose token blocks alternate between incompressible
    values (stored raw: the compaction copies them from the pass's own part of
    the target), values that all escape, and ordinary ones: whole-slab and
    token-block passes give the oracle's container."""
    cfg = gen.Config(99, f"passes-mixed-{dtype}", dtype, 2, 2, 1536, 128, outliers=False)
    t, p, tabs, oshape = residual_case(skv, orc, cfg)
    g = torch.Generator(device="cuda")
    g.manual_seed(23)
    t = t.clone()
    bits = 8 if dtype == "e4m3" else 16
    for b in range(cfg.tokens // 128):
        sl = slice(128 * b, 128 * b + 128)
        if b % 3 == 0:
            hi = 1 << bits
            r = torch.randint(0, hi, t[:, :, sl].shape, generator=g, device="cuda", dtype=torch.int32)
            t[:, :, sl] = (r - (hi // 2 if dtype == "bf16" else 0)).to(t.dtype)
        elif b % 3 == 1:
            off = 100 if dtype == "e4m3" else 300
            t[:, :, sl] = (p[:, :, sl].to(torch.int32) + off).to(t.dtype)
    want = orc.encode_array(tabs.bytes(), oshape, t.cpu().numpy(), p.cpu().numpy(), threads=ORACLE_THREADS)
    n, idx, _ = _parse(want.tobytes())
    assert (idx[:-1] >> np.uint64(63)).any(), "some streams are stored raw"
    full, _ = skv.encode_workspace(tabs, cfg.tokens)
    for budget in (0, full // 3, full // 9):
        wb, passes = skv.encode_workspace(tabs, cfg.tokens, budget)
        enc = skv.Encoder(tabs, cfg.tokens, max_work_bytes=budget)
        say(f"[parity] mixed {dtype}: {passes} passes")
        got = enc(t, p)
        assert_same_container(host_u8(got), want, f"mixed {dtype}, {passes} passes")
    assert torch.equal(skv.decode(tabs, got, p), t)
