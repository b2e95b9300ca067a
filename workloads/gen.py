"""Seeded synthetic inputs shaped like the workloads on the pages.

Real caches of the models the pages measured are not available, so every
input here is synthetic.  Shapes follow the pages:

* Speculative KV coding summary ("Initial results"): Qwen3 family caches, bf16
  and fp8.  Configurations 0-3 use 8 KV heads x 128 dims per layer and the
  layer counts of Qwen3-0.6B (28), Qwen3-8B (36) and Qwen3-32B (64).
* DCKV page ("What it is", "How it works"): 6 full-attention layers x K,V x
  512 dims per token, reduced to 2048 transform coefficients; configuration 4
  codes 131072 tokens of 2048 int16 coefficients.

Layout of every residual-mode array: ``[layers][kv][tokens][channels]`` with
channel = head * 128 + dim fastest.  Elements are returned as integer bit
patterns (uint16 views of bf16, uint8 e4m3 codes, int16 coefficients).

Seeding: every (config, purpose, layer, kv) gets its own child seed, so slabs
can be generated independently and streamed.  Purposes: 0 channel
parameters, 1 evaluation draw, 2 calibration draw.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

PARAMS, EVAL, CALIB = 0, 1, 2
CALIB_TOKENS = 256


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    dtype: str          # "bf16" | "e4m3" | "int16"
    layers: int
    kv: int
    tokens: int
    channels: int
    outliers: bool = True
    layer_scaling: bool = False

    @property
    def elem_bytes(self) -> int:
        return 1 if self.dtype == "e4m3" else 2

    @property
    def values(self) -> int:
        return self.layers * self.kv * self.tokens * self.channels

    @property
    def raw_bytes(self) -> int:
        return self.values * self.elem_bytes

    def with_tokens(self, tokens: int, layers: int | None = None, channels: int | None = None) -> "Config":
        return dataclasses.replace(self, tokens=tokens, layers=self.layers if layers is None else layers,
                                   channels=self.channels if channels is None else channels)


CONFIGS = {
    0: Config(0, "single-layer-bf16", "bf16", 1, 2, 1024, 1024),
    1: Config(1, "qwen3-0.6b-shaped-bf16", "bf16", 28, 2, 8192, 1024, layer_scaling=True),
    2: Config(2, "qwen3-8b-shaped-e4m3", "e4m3", 36, 2, 32768, 1024, outliers=False),
    3: Config(3, "qwen3-32b-shaped-bf16", "bf16", 64, 2, 32768, 1024, layer_scaling=True),
    4: Config(4, "dckv-coefficients-int16", "int16", 1, 1, 131072, 2048, outliers=False),
}


def _seed(cid: int, purpose: int, layer: int = 0, kv: int = 0) -> int:
    ss = np.random.SeedSequence((20261202, cid, purpose, layer, kv))
    return int(ss.generate_state(1, dtype=np.uint64)[0] >> 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def channel_sigma(cfg: Config, layer: int, kv: int) -> np.ndarray:
    """Per-channel standard deviation: log-normal(0, 0.5); with outliers, 4
    dims per 128-dim head (drawn without replacement) scaled x10; with layer
    scaling, x(1 + layer / layers)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence((20261202, cfg.cid, PARAMS, layer, kv))))
    sigma = np.exp(rng.normal(0.0, 0.5, size=cfg.channels))
    if cfg.outliers:
        for h in range(cfg.channels // 128):
            dims = rng.choice(128, size=4, replace=False)
            sigma[h * 128 + dims] *= 10.0
    if cfg.layer_scaling:
        sigma *= 1.0 + layer / cfg.layers
    return sigma.astype(np.float32)


def residual_slab(cfg: Config, layer: int, kv: int, purpose: int, tokens: int, device="cpu"):
    """One (layer, K|V) plane: returns (target, predictor) as integer tensors
    of shape [tokens][channels] on `device`.

    bf16 configs: target = bf16(N(0, sigma_c)); predictor = target scaled by
    the channel's amax / 448, rounded to e4m3, scaled back, plus
    N(0, (0.01 sigma_c)^2) noise, rounded to bf16.
    e4m3 config: target = e4m3(N(0, sigma_c)); predictor =
    e4m3(target + N(0, (0.02 sigma_c)^2)).
    """
    sig = torch.from_numpy(channel_sigma(cfg, layer, kv)).to(device)
    g = _gen(device, _seed(cfg.cid, purpose, layer, kv))
    x = torch.randn((tokens, cfg.channels), generator=g, device=device, dtype=torch.float32) * sig
    noise = torch.randn((tokens, cfg.channels), generator=g, device=device, dtype=torch.float32)
    if cfg.dtype == "bf16":
        t = x.to(torch.bfloat16)
        tf = t.to(torch.float32)
        scale = tf.abs().amax(dim=0).clamp_min(1e-30) / 448.0
        q = (tf / scale).to(torch.float8_e4m3fn).to(torch.float32) * scale
        p = (q + noise * (0.01 * sig)).to(torch.bfloat16)
        return t.view(torch.int16), p.view(torch.int16)
    if cfg.dtype == "e4m3":
        t = x.to(torch.float8_e4m3fn)
        p = (t.to(torch.float32) + noise * (0.02 * sig)).to(torch.float8_e4m3fn)
        return t.view(torch.uint8), p.view(torch.uint8)
    raise ValueError(cfg.dtype)


def residual_array(cfg: Config, purpose: int = EVAL, tokens: int | None = None, device="cpu"):
    """Full [layers][kv][tokens][channels] target and predictor arrays."""
    T = cfg.tokens if tokens is None else tokens
    dt = torch.uint8 if cfg.dtype == "e4m3" else torch.int16
    tgt = torch.empty((cfg.layers, cfg.kv, T, cfg.channels), dtype=dt, device=device)
    prd = torch.empty_like(tgt)
    for l in range(cfg.layers):
        for k in range(cfg.kv):
            a, b = residual_slab(cfg, l, k, purpose, T, device)
            tgt[l, k].copy_(a)
            prd[l, k].copy_(b)
            del a, b
    return tgt, prd


# ------------------------------------------------------------------ DCKV
VOCAB, EMB, RANK = 4096, 256, 64


def dckv_params(cfg: Config, device="cpu"):
    """Scale b_c log-uniform in [0.5, 20] cells; token embeddings N(0, 1/256);
    E rows N(0, (3 b_c)^2); rank-64 map U (rows N(0, b_c^2 / 64)) times V (N(0, 1))."""
    g = _gen("cpu", _seed(cfg.cid, PARAMS))
    C = cfg.channels
    b = torch.exp(torch.empty(C, dtype=torch.float64).uniform_(math.log(0.5), math.log(20.0), generator=g))
    emb = torch.randn((VOCAB, EMB), generator=g, dtype=torch.float64) / math.sqrt(EMB)
    E = torch.randn((C, EMB), generator=g, dtype=torch.float64) * (3.0 * b)[:, None]
    U = torch.randn((C, RANK), generator=g, dtype=torch.float64) * (b / math.sqrt(RANK))[:, None]
    V = torch.randn((RANK, EMB), generator=g, dtype=torch.float64)
    f32 = dict(dtype=torch.float32, device=device)
    return b.to(**f32), emb.to(**f32), E.to(**f32), (U @ V).to(**f32)


MAP_RANK, MAP_SH1, MAP_SH2 = 64, 11, 4


def dckv_map_weights(cfg: Config, rank: int = MAP_RANK):
    """Seeded weights of a rank-`rank` linear map over an odd token's two
    even neighbour rows: V int8 [rank][2C] (entries N(0, 40^2), clipped),
    U int8 [C][rank] (row c ~ N(0, (2 b_c)^2), clipped), and the two shifts
    (MAP_SH1, MAP_SH2) that scale them.  These are inputs of the workload,
    like the codec weights of a trained model."""
    g = _gen("cpu", _seed(cfg.cid, PARAMS, 1))
    b, _, _, _ = dckv_params(cfg)
    C = cfg.channels
    V = (torch.randn((rank, 2 * C), generator=g, dtype=torch.float64) * 40.0).round().clamp(-127, 127)
    U = (torch.randn((C, rank), generator=g, dtype=torch.float64) * (2.0 * b.double())[:, None]).round()
    U = U.clamp(-127, 127)
    return V.to(torch.int8).numpy(), U.to(torch.int8).numpy(), MAP_SH1, MAP_SH2


def dckv_draw(cfg: Config, purpose: int = EVAL, tokens: int | None = None, device="cpu", nbr_map=None):
    """Coefficients and side input for the checkerboard configuration.

    Returns (coef, G): int16 tensors [tokens][channels].  G holds each
    token's conditioning mean in sixteenths of a cell, rounded half-to-even:
    even tokens E*emb(token); odd tokens the rank-64 map UV*emb(token).  The
    coefficient of an even token is round(E*emb + Laplace(b_c)); of an odd
    token round(mean of its two even neighbours + UV*emb + Laplace(b_c)) (the
    last odd token repeats its left neighbour).  With nbr_map = (V, U, sh1,
    sh2) the odd mean also adds the real-valued map of the two neighbour
    rows n, (U (V n) / 2^sh1) / 2^sh2 / 16 cells.
    """
    T = cfg.tokens if tokens is None else tokens
    assert T % 2 == 0
    b, emb, E, UV = dckv_params(cfg, device)
    g = _gen(device, _seed(cfg.cid, purpose))
    tok = torch.randint(0, VOCAB, (T,), generator=g, device=device)
    e = emb[tok]                                  # [T, 256]
    mean = torch.empty((T, cfg.channels), dtype=torch.float32, device=device)
    mean[0::2] = e[0::2] @ E.T
    mean[1::2] = e[1::2] @ UV.T
    G = torch.round(mean * 16.0).clamp(-32768, 32767)
    u1 = torch.rand((T, cfg.channels), generator=g, device=device, dtype=torch.float32)
    u2 = torch.rand((T, cfg.channels), generator=g, device=device, dtype=torch.float32)
    lap = (torch.log1p(-u1) - torch.log1p(-u2)) * b        # Laplace(0, b_c)
    coef = torch.empty((T, cfg.channels), dtype=torch.float32, device=device)
    coef[0::2] = torch.round(G[0::2] / 16.0 + lap[0::2]).clamp(-32768, 32767)
    left = coef[0::2]
    right = torch.cat([coef[2::2], coef[-2:-1]], dim=0)
    odd = (left + right) * 0.5 + G[1::2] / 16.0 + lap[1::2]
    if nbr_map is not None:
        V, U, sh1, sh2 = nbr_map
        C = cfg.channels
        Vf = torch.as_tensor(V, dtype=torch.float32, device=device)
        Uf = torch.as_tensor(U, dtype=torch.float32, device=device)
        h = left @ Vf[:, :C].T.contiguous() + right @ Vf[:, C:].T.contiguous()
        odd = odd + (h / 2.0 ** sh1) @ Uf.T.contiguous() / (2.0 ** sh2 * 16.0)
    coef[1::2] = torch.round(odd).clamp(-32768, 32767)
    return coef.to(torch.int16), G.to(torch.int16)
