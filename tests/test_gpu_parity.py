"""GPU parity: containers and reconstructions from libskv's HIP kernels are
bit-identical to the CPU oracle's.

The coding path is integer end to end, so there is no tolerance: container
bytes must equal the oracle's byte for byte and the decode must return the
target exactly (lossless reconstruction, Speculative KV coding summary,
'Core idea'; checkerboard decoding in two passes, DCKV page, 'How it
differs').  Small cases compare whole containers; full-size workloads
compare sampled streams (the oracle encodes them one by one from the
gathered tiles) plus the exact GPU round trip.
"""
import struct
import sys

import numpy as np
import pytest
import torch

from workloads import gen

pytestmark = pytest.mark.gpu


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
    want = orc.encode(tabs.bytes(), oshape, tn, pn, threads=8)
    got = cont.cpu().numpy().tobytes()
    assert len(got) == len(want), (len(got), len(want))
    if got != want:
        n, idx, head = _parse(want)
        gi = np.frombuffer(got[64:head], dtype=np.uint64)
        bad = np.nonzero(gi != idx)[0]
        raise AssertionError(f"container differs; first index mismatch {bad[:5]}")
    say(f"[parity] {what}: decode on GPU")
    back = skv.decode(tabs, cont, p)
    assert torch.equal(back, t)
    # the GPU decodes the oracle's container as well
    back2 = skv.decode(tabs, torch.from_numpy(np.frombuffer(want, dtype=np.uint8).copy()).cuda(), p)
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


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_word_bursts_after_escapes(skv, orc, dtype):
    """Every token block escapes in its first 4 steps and codes rare direct
    symbols (about 12 bits each) in the next 8, then repeats the predictor:
    the tiles after the escapes need more words than the decoder's ring holds,
    so they are decoded again from memory while the escapes of the tile before
    are being resolved.  The streams stay coded (not raw)."""
    cfg = gen.Config(93, f"burst-{dtype}", dtype, 1, 2, 512, 96)
    t, p, tabs, oshape = residual_case(skv, orc, cfg)
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


def test_exponent_mode_escapes_and_unaligned(skv, orc):
    """Exponent mode through every kernel path: rare far residuals (escapes in
    every class, with bursts of words), the tiled kernels on aligned buffers and
    the per-step ones on unaligned buffers; all containers equal the oracle's."""
    cfg = gen.Config(99, "exp-escapes", "e4m3", 1, 2, 512, 128)
    t, p, tabs, oshape = exp_case(skv, orc, cfg)
    rng = np.random.default_rng(21)
    tn = t.cpu().numpy()
    flat = tn.reshape(-1)
    pos = rng.choice(flat.size, size=flat.size // 200, replace=False)
    flat[pos] = rng.integers(0, 256, size=pos.size, dtype=np.uint8)
    t = torch.from_numpy(tn).cuda()
    want = full_compare(skv, orc, t, p, tabs, oshape, "exponent mode escapes")
    tu, pu = _offset_copy(t, 1), _offset_copy(p, 3)
    cont = skv.encode(tabs, tu, pu)
    torch.cuda.synchronize()
    assert cont.cpu().numpy().tobytes() == want
    out = _offset_copy(torch.zeros_like(t), 1)
    skv.decode_into(tabs, cont, pu, out)
    assert torch.equal(out, t)


@pytest.mark.parametrize("exp", [True, False])
def test_e4m3_corruption_verdicts(skv, orc, exp):
    """Damaged e4m3 containers (per-channel or exponent-class tables): the
    decoder reaches the oracle's verdict on every bit flip in the coded part of
    a stream (a flip can leave a consistent stream, which both then decode
    alike), and refuses an index past the payload and another blob."""
    cfg = gen.Config(100, "exp-corrupt", "e4m3", 1, 2, 512, 128)
    t, p, tabs, oshape = exp_case(skv, orc, cfg) if exp else residual_case(skv, orc, cfg)
    cont = skv.encode(tabs, t, p)
    good = cont.cpu().numpy()
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
        say(f"[parity] e4m3 corrupt trial {trials} (exponent tables {exp}): stream {st} byte {pos}")
        want = np.zeros_like(tn)
        rc = orc.decode_rc(tabs.bytes(), bad.tobytes(), pn, want)
        if rc == orc.E_CORRUPT:
            with pytest.raises(skv.SkvError) as e:
                skv.decode(tabs, torch.from_numpy(bad).cuda(), p)
            assert e.value.status == skv.ERR_CORRUPT
            refused += 1
        else:
            assert rc == orc.OK
            assert np.array_equal(skv.decode(tabs, torch.from_numpy(bad).cuda(), p).cpu().numpy(), want)
        trials += 1
    assert refused >= 20
    bad = good.copy()
    bad[64 + 8 * 3:64 + 8 * 4] = np.frombuffer(struct.pack("<Q", 1 << 40), np.uint8)
    with pytest.raises(skv.SkvError) as e:
        skv.decode(tabs, torch.from_numpy(bad).cuda(), p)
    assert e.value.status == skv.ERR_CORRUPT
    ct, cp = gen.residual_array(cfg, gen.CALIB, tokens=256)
    other = skv.fit_tables(skv.E4M3, skv.RESIDUAL if exp else skv.RESIDUAL_EXP, 1, 2, 128, ct.numpy(), cp.numpy(), 256)
    with pytest.raises(skv.SkvError) as e:
        skv.decode(other, cont, p)
    assert e.value.status == skv.ERR_TABLES
    assert torch.equal(skv.decode(tabs, cont, p), t)


def test_exponent_mode_full_size_e4m3(skv, orc):
    """The Qwen3-8B-shaped e4m3 cache with exponent-conditioned tables: sampled
    streams equal the oracle's, the round trip is exact, and the container is
    smaller than with per-channel tables."""
    cfg = gen.CONFIGS[2]
    say(f"[parity] exponent mode cfg2: generating {cfg.values} values on GPU")
    t, p, tabs, oshape = exp_case(skv, orc, cfg)
    cont = skv.encode(tabs, t, p)
    torch.cuda.synchronize()
    n = orc.n_streams(oshape)
    head = 64 + 8 * (n + 1)
    host_head = cont[:head].cpu().numpy().tobytes()
    idx = np.frombuffer(host_head[64:], dtype=np.uint64)
    offs = idx & np.uint64((1 << 63) - 1)
    assert int(offs[-1]) == cont.numel() - head
    ratio = cfg.raw_bytes / cont.numel()
    say(f"[parity] exponent mode cfg2: ratio {ratio:.4f}")
    assert ratio > 4.5
    ncg, ntb, blob = cfg.channels // 32, cfg.tokens // 128, tabs.bytes()
    for s in _sample_ids(n, 32, 2):
        cg, rest = s % ncg, s // ncg
        tb, slab = rest % ntb, rest // ntb
        l, k = divmod(slab, cfg.kv)
        sl = (l, k, slice(tb * 128, tb * 128 + 128), slice(cg * 32, cg * 32 + 32))
        lanes = np.full(32, slab, dtype=np.uint32)            # exponent mode: the stream's slab
        data, raw = orc.encode_tile(blob, oshape, t[sl].cpu().numpy(), p[sl].cpu().numpy(), lanes)
        assert bool(int(idx[s]) >> 63) == raw, s
        assert cont[head + int(offs[s]):head + int(offs[s + 1])].cpu().numpy().tobytes() == data, s
    say("[parity] exponent mode cfg2: sampled streams identical; decoding")
    back = skv.decode(tabs, cont, p)
    assert torch.equal(back, t)


RANGES = [(0, 1024), (0, 128), (896, 1024), (256, 640), (128, 1024)]


@pytest.mark.parametrize("dtype,aligned", [("e4m3", True), ("bf16", True), ("bf16", False)])
def test_decode_range(skv, orc, dtype, aligned):
    """A token range decoded through the offset index equals the same tokens
    of the oracle's decode of the whole container (e4m3: decode_e4m3; bf16:
    decode_bf16, or the per-table LDS decoder for unaligned buffers)."""
    cfg = gen.Config(95, f"range-{dtype}", dtype, 2, 2, 1024, 256)
    t, p, tabs, oshape = residual_case(skv, orc, cfg)
    cont = skv.encode(tabs, t, p)
    torch.cuda.synchronize()
    pn = p.cpu().numpy()
    say(f"[parity] range {dtype}: oracle decode of the whole container")
    want = orc.decode(tabs.bytes(), cont.cpu().numpy().tobytes(), pn, pn, threads=8)
    assert np.array_equal(want, t.cpu().numpy())
    for a, b in RANGES:
        say(f"[parity] range {dtype} aligned={aligned}: tokens [{a}, {b})")
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
        with pytest.raises(skv.SkvError) as e:
            skv.decode_range(tabs, cont, a, b, p[:, :, :128].contiguous())
        assert e.value.status == skv.ERR_SHAPE, (a, b)
    with pytest.raises(skv.SkvError) as e:
        skv.decode_range_into(tabs, cont, 128, 384, p, torch.empty(10, dtype=torch.uint8, device="cuda"))
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
    # checkerboard containers have no range decode
    cb = gen.CONFIGS[4].with_tokens(512, channels=64)
    coef, G = gen.dckv_draw(cb, device="cuda")
    cc, cgl = gen.dckv_draw(cb, gen.CALIB, tokens=256, device="cuda")
    ctabs = skv.fit_tables(skv.INT16, skv.CHECKERBOARD, 1, 1, 64, cc.cpu().numpy(), cgl.cpu().numpy(), 256)
    ccont = skv.encode(ctabs, coef, G)
    with pytest.raises(skv.SkvError) as e:
        skv.decode_range(ctabs, ccont, 0, 256, G[:256].contiguous())
    assert e.value.status == skv.ERR_SHAPE


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
def _sample_ids(n, k, seed):
    rng = np.random.default_rng(seed)
    ids = set(rng.choice(n, size=min(k, n), replace=False).tolist())
    ids.update({0, n - 1})
    return sorted(ids)


def _check_sampled_streams(orc, blob, oshape, cont_host, tile_fn, lane_fn, n, ids, what):
    head = 64 + 8 * (n + 1)
    idx = np.frombuffer(cont_host[64:head], dtype=np.uint64)
    mask = np.uint64((1 << 63) - 1)
    offs = idx & mask
    assert offs[0] == 0 and np.all(offs[1:] >= offs[:-1])
    assert int(offs[-1]) == len(cont_host) - head
    for s in ids:
        tt, ta, nl, nr = tile_fn(s)
        data, raw = orc.encode_tile(blob, oshape, tt, ta, lane_fn(s), nl, nr)
        a, b = int(offs[s]), int(offs[s + 1])
        assert bool(int(idx[s]) >> 63) == raw, (what, s)
        assert cont_host[head + a:head + b] == data, (what, s)


@pytest.mark.parametrize("cid", [1, 2, 3])
def test_full_size_residual(skv, orc, cid):
    cfg = gen.CONFIGS[cid]
    say(f"[parity] cfg{cid} {cfg.name}: generating {cfg.values} values on GPU")
    t, p, tabs, oshape = residual_case(skv, orc, cfg)
    say(f"[parity] cfg{cid}: encode")
    cont = skv.encode(tabs, t, p)
    torch.cuda.synchronize()
    n = orc.n_streams(oshape)
    ratio = cfg.raw_bytes / cont.numel()
    say(f"[parity] cfg{cid}: {n} streams, container {cont.numel()} B, ratio {ratio:.3f}")
    head = 64 + 8 * (n + 1)
    ids = _sample_ids(n, 48, cid)
    # copy back only the header+index and the sampled streams' bytes
    host_head = cont[:head].cpu().numpy().tobytes()
    idx = np.frombuffer(host_head[64:], dtype=np.uint64) & np.uint64((1 << 63) - 1)
    assert int(idx[-1]) == cont.numel() - head
    ncg, ntb = cfg.channels // 32, cfg.tokens // 128
    blob = tabs.bytes()

    def tile(s):
        cg, rest = s % ncg, s // ncg
        tb, slab = rest % ntb, rest // ntb
        l, k = divmod(slab, cfg.kv)
        sl = (l, k, slice(tb * 128, tb * 128 + 128), slice(cg * 32, cg * 32 + 32))
        return t[sl].cpu().numpy(), p[sl].cpu().numpy(), None, None

    def lanes(s):
        cg, slab = s % ncg, s // (ncg * ntb)
        return np.arange(32, dtype=np.uint32) + slab * cfg.channels + cg * 32

    head_raw = np.frombuffer(host_head[64:], dtype=np.uint64)
    for s in ids:
        tt, ta, _, _ = tile(s)
        data, raw = orc.encode_tile(blob, oshape, tt, ta, lanes(s))
        a, b = int(idx[s]), int(idx[s + 1])
        assert bool(int(head_raw[s]) >> 63) == raw, s
        got = cont[head + a:head + b].cpu().numpy().tobytes()
        assert got == data, (cid, s)
    say(f"[parity] cfg{cid}: {len(ids)} sampled streams identical; decoding")
    del cont
    back = skv.decode(tabs, skv.encode(tabs, t, p), p)
    assert torch.equal(back, t)
    say(f"[parity] cfg{cid}: round trip exact")


def test_slab_over_2gib(skv, orc):
    """A (layer, K|V) slab of 2 GiB (2^21 tokens x 1024 e4m3 channels) is past
    the tiled kernels' 32-bit row offsets, so it takes the per-step encoder and
    decoder; sampled streams match the oracle, the round trip is exact, and a
    range at the slab's end decodes through the tiled decoder."""
    cfg = gen.Config(97, "slab-2gib-e4m3", "e4m3", 1, 1, 1 << 21, 1024, outliers=False)
    say(f"[parity] 2 GiB slab: generating {cfg.values} values on GPU")
    t, p, tabs, oshape = residual_case(skv, orc, cfg)
    say("[parity] 2 GiB slab: encode")
    cont = skv.encode(tabs, t, p)
    torch.cuda.synchronize()
    n = orc.n_streams(oshape)
    head = 64 + 8 * (n + 1)
    host_head = cont[:head].cpu().numpy().tobytes()
    idx = np.frombuffer(host_head[64:], dtype=np.uint64)
    offs = idx & np.uint64((1 << 63) - 1)
    assert int(offs[-1]) == cont.numel() - head
    ncg, blob = cfg.channels // 32, tabs.bytes()
    for s in _sample_ids(n, 24, 97):
        cg, tb = s % ncg, s // ncg
        sl = (0, 0, slice(tb * 128, tb * 128 + 128), slice(cg * 32, cg * 32 + 32))
        lanes = np.arange(32, dtype=np.uint32) + cg * 32
        data, raw = orc.encode_tile(blob, oshape, t[sl].cpu().numpy(), p[sl].cpu().numpy(), lanes)
        assert bool(int(idx[s]) >> 63) == raw, s
        assert cont[head + int(offs[s]):head + int(offs[s + 1])].cpu().numpy().tobytes() == data, s
    say("[parity] 2 GiB slab: sampled streams identical; decoding")
    back = skv.decode(tabs, cont, p)
    assert torch.equal(back, t)
    del back
    a = cfg.tokens - 256
    part = skv.decode_range(tabs, cont, a, cfg.tokens, p[:, :, a:].contiguous())
    assert torch.equal(part, t[:, :, a:])
    say("[parity] 2 GiB slab: round trip and end range exact")


def test_full_size_checkerboard(skv, orc):
    cfg = gen.CONFIGS[4]
    say("[parity] cfg4: generating")
    coef, G = gen.dckv_draw(cfg, device="cuda")
    cc, cg = gen.dckv_draw(cfg, gen.CALIB, tokens=256, device="cuda")
    tabs = skv.fit_tables(skv.INT16, skv.CHECKERBOARD, 1, 1, cfg.channels, cc.cpu().numpy(), cg.cpu().numpy(), 256)
    oshape = orc.make_shape(orc.INT16, orc.CHECKERBOARD, 1, 1, cfg.tokens, cfg.channels)
    cont = skv.encode(tabs, coef, G)
    torch.cuda.synchronize()
    n = orc.n_streams(oshape)
    head = 64 + 8 * (n + 1)
    say(f"[parity] cfg4: {n} streams, ratio {cfg.raw_bytes / cont.numel():.3f}")
    idx_raw = np.frombuffer(cont[:head].cpu().numpy().tobytes()[64:], dtype=np.uint64)
    idx = idx_raw & np.uint64((1 << 63) - 1)
    ncg, ntb = cfg.channels // 32, cfg.tokens // 2 // 128
    T = cfg.tokens
    blob = tabs.bytes()
    for s in _sample_ids(n, 48, 4):
        cgi, rest = s % ncg, s // ncg
        tb, ps = rest % ntb, rest // ntb
        toks = torch.arange(128, device="cuda") * 2 + 2 * 128 * tb + ps
        cols = slice(cgi * 32, cgi * 32 + 32)
        tt = coef[toks, cols].cpu().numpy()
        ta = G[toks, cols].cpu().numpy()
        nl = nr = None
        if ps == 1:
            nl = coef[toks - 1, cols].cpu().numpy()
            right = torch.where(toks + 1 < T, toks + 1, toks - 1)
            nr = coef[right, cols].cpu().numpy()
        data, raw = orc.encode_tile(blob, oshape, tt, ta, np.arange(32, dtype=np.uint32) + cgi * 32, nl, nr)
        a, b = int(idx[s]), int(idx[s + 1])
        assert bool(int(idx_raw[s]) >> 63) == raw
        assert cont[head + a:head + b].cpu().numpy().tobytes() == data, s
    back = skv.decode(tabs, cont, G)
    assert torch.equal(back, coef)
    say("[parity] cfg4: sampled streams identical, round trip exact")


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
    reconstruction, and the first and last chunk containers equal the
    one-shot encoder's containers of those layers."""
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
    for c in (0, len(offs) - 2):
        l0, l1 = 4 * c, min(cfg.layers, 4 * c + 4)
        part = skv.fit_tables(skv.E4M3, skv.RESIDUAL, l1 - l0, cfg.kv, cfg.channels,
                              np.ascontiguousarray(ct[l0:l1]), np.ascontiguousarray(cp[l0:l1]), 256)
        want = skv.encode(part, t[l0:l1].contiguous(), p[l0:l1].contiguous())
        assert torch.equal(wire[offs[c]:offs[c + 1]], want.cpu()), c
