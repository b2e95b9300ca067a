"""The encode entry point that allocates nothing (skv_encode_noalloc), for
callers that cannot allocate device memory.  Called through the C ABI, its
container equals skv_encode's byte for byte and decodes exactly, on two
calls in a row with the second input smaller and different (the fixed
workspace keeps the first call's contents, which the second must not
read); shapes larger than one pass of the fixed workspace are coded in
several passes; a checkerboard shape past it and tables not yet on the
device are refused before anything is launched.
"""
import sys

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


def _residual(skv, cid, mode, layers, channels, tokens, purpose):
    cfg = gen.CONFIGS[cid].with_tokens(tokens, layers=layers, channels=channels)
    t, p = gen.residual_array(cfg, purpose, device="cuda")
    return cfg, t, p


def _tables(skv, kind):
    if kind == "checkerboard":
        cfg = gen.CONFIGS[4].with_tokens(256, channels=2048)
        cc, cg = gen.dckv_draw(cfg, gen.CALIB, tokens=256)
        return skv.fit_tables(skv.INT16, skv.CHECKERBOARD, 1, 1, 2048, cc.numpy(), cg.numpy(), 256)
    cid, dt = (0, skv.BF16) if kind == "bf16" else (2, skv.E4M3)
    mode = skv.RESIDUAL_EXP if kind == "exp-e4m3" else skv.RESIDUAL
    layers = 1 if kind == "bf16" else 2
    cfg = gen.CONFIGS[cid].with_tokens(256, layers=layers, channels=1024)
    ct, cp = gen.residual_array(cfg, gen.CALIB, tokens=256)
    return skv.fit_tables(dt, mode, layers, 2, 1024, ct.numpy(), cp.numpy(), 256)


def _inputs(skv, kind, tokens, purpose):
    if kind == "checkerboard":
        cfg = gen.CONFIGS[4].with_tokens(tokens, channels=2048)
        return gen.dckv_draw(cfg, purpose, device="cuda")
    cid = 0 if kind == "bf16" else 2
    layers = 1 if kind == "bf16" else 2
    cfg = gen.CONFIGS[cid].with_tokens(tokens, layers=layers, channels=1024)
    return gen.residual_array(cfg, purpose, device="cuda")


# (kind, tokens of the first call, tokens of the second, smaller call).  The
# first calls of the last two exceed one pass of the fixed array: 8192 bf16
# tokens take one whole slab per pass, 32768 e4m3 tokens 255 + 1 token blocks
# of each slab.
CASES = [("bf16", 1024, 256), ("e4m3", 1024, 384), ("exp-e4m3", 896, 128), ("checkerboard", 4096, 1024),
         ("bf16", 8192, 1024), ("e4m3", 32768, 512)]


@pytest.mark.parametrize("kind,big,small", CASES)
def test_noalloc_equals_encode(skv, kind, big, small):
    tabs = _tables(skv, kind)
    for tokens, purpose in ((big, gen.EVAL), (small, gen.CALIB)):
        say(f"[noalloc] {kind}: {tokens} tokens")
        t, p = _inputs(skv, kind, tokens, purpose)
        want = skv.encode(tabs, t, p)             # the existing entry point (puts the tables on the device)
        bound = skv.encode_noalloc_bound(tabs, tokens)
        out = torch.full((bound,), 0xA5, dtype=torch.uint8, device="cuda")
        got = skv.encode_noalloc(tabs, t, p, out)
        torch.cuda.synchronize()
        assert got.numel() == want.numel()
        assert torch.equal(got, want), (kind, tokens)
        assert torch.equal(skv.decode(tabs, got, p), t)
        # the output buffer too small: refused, with the size needed
        with pytest.raises(skv.SkvError) as e:
            skv.encode_noalloc(tabs, t, p, out[:100])
        assert e.value.status == skv.ERR_CAPACITY


def test_noalloc_refusals(skv):
    # a checkerboard shape (one pass) whose workspace exceeds the fixed array
    tabs = _tables(skv, "checkerboard")
    with pytest.raises(skv.SkvError) as e:
        skv.encode_noalloc_bound(tabs, 32768)
    assert e.value.status == skv.ERR_SHAPE
    # tables never used on this device: building them would allocate
    fresh = _tables(skv, "bf16")
    t, p = _inputs(skv, "bf16", 256, gen.EVAL)
    out = torch.empty(skv.encode_noalloc_bound(fresh, 256), dtype=torch.uint8, device="cuda")
    with pytest.raises(skv.SkvError) as e:
        skv.encode_noalloc(fresh, t, p, out)
    assert e.value.status == skv.ERR_ARG
    # once another call has put them there, the same call succeeds
    want = skv.encode(fresh, t, p)
    assert torch.equal(skv.encode_noalloc(fresh, t, p, out), want)
