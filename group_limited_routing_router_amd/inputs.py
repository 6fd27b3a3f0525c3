"""Seeded synthetic inputs for the MoE block: shapes and random draws only.

This module holds none of the method's arithmetic.  It is the one piece of code
that both the HIP path's tests and the CPU oracle's tests use: it names the
workload shapes and draws the tensors; nothing here scores, selects, sorts,
multiplies or combines.

Shapes follow the Beam MoE block ("Welcome Beam: a 501B open model you can own,
customize, and scale", section "Mixture of Experts": hidden 5120, 256 experts
in 8 groups of 32, 4 groups kept, 8 experts per token, intermediate 2560,
output scale 2.5).  Trained weights are not available, so seeded Gaussians
stand in for them: activations ~ N(0, 1), router and expert weights
~ N(0, 0.02), all cast to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    H: int
    I: int
    E: int
    G: int
    TG: int
    k: int
    scale: float
    hot_groups: int = 0      # skew: number of groups holding biased experts
    hot_per_group: int = 0   # skew: biased experts per hot group
    hot_bias: float = 0.0    # skew: logit bias on each hot expert

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)

    @property
    def pairs(self) -> int:
        return self.T * self.k


_BEAM = dict(H=5120, I=2560, E=256, G=8, TG=4, k=8, scale=2.5)

CONFIGS = {
    # small case the oracle finishes in well under a second
    "tiny": MoEConfig("tiny", T=64, H=256, I=128, E=16, G=4, TG=2, k=4, scale=1.0),
    # decode batch: weight-streaming (HBM-bound) regime
    "decode": MoEConfig("decode", T=128, **_BEAM),
    # prefill chunk: ~256 rows per expert
    "prefill": MoEConfig("prefill", T=8192, **_BEAM),
    # skewed routing: +3.0 logit bias on 8 experts in each of 2 seeded groups
    "skew": MoEConfig("skew", T=4096, hot_groups=2, hot_per_group=8, hot_bias=3.0, **_BEAM),
    # long prefill processed as one call
    "long": MoEConfig("long", T=65536, **_BEAM),
    # dense SwiGLU MLP of the first layers on the expert kernels (one expert
    # takes every token); the pages do not give its intermediate size, so it is
    # taken as the width of the eight experts a token runs, 8 * 2560
    "dense": MoEConfig("dense", T=8192, H=5120, I=20480, E=1, G=1, TG=1, k=1, scale=1.0),
}

ACT_STD = 1.0
W_STD = 0.02


def _randn_bf16(shape, std, gen, device, chunk_rows=None):
    """N(0, std^2) drawn in fp32 and rounded to bf16; big tensors are drawn in
    chunks along dim 0 to bound the fp32 temporary."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    n0 = shape[0]
    step = n0 if chunk_rows is None else max(1, chunk_rows)
    for a in range(0, n0, step):
        b = min(n0, a + step)
        t = torch.randn((b - a, *shape[1:]), generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        out[a:b].copy_(t)
        del t
    return out


WEIGHT_SEED_OFFSET = 1_000_003


def make_tokens(cfg: MoEConfig, seed: int = 0, device="cpu"):
    """Draw the activations x [T,H] (bf16) and the router bias [E] (fp32).

    The bias is zero except for the skewed workload: ``hot_per_group`` experts
    in each of ``hot_groups`` seeded groups get ``hot_bias``.  Draw order: x,
    then the hot-group choice, then the hot experts inside each group."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = _randn_bf16((cfg.T, cfg.H), ACT_STD, gen, device, chunk_rows=8192)
    bias = torch.zeros(cfg.E, dtype=torch.float32, device=device)
    if cfg.hot_groups > 0:
        gsize = cfg.E // cfg.G
        groups = torch.randperm(cfg.G, generator=gen, device=device)[: cfg.hot_groups]
        for g in groups.tolist():
            members = torch.randperm(gsize, generator=gen, device=device)[: cfg.hot_per_group]
            bias[g * gsize + members] = cfg.hot_bias
    return dict(x=x, bias=bias)


def make_weights(cfg: MoEConfig, seed: int = 0, device="cpu"):
    """Draw the router weight [E,H] and the expert stacks w_gate, w_up
    [E,I,H] and w_down [E,H,I] (bf16), in that order, from a generator seeded
    with seed + WEIGHT_SEED_OFFSET."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + WEIGHT_SEED_OFFSET)
    E, H, I = cfg.E, cfg.H, cfg.I
    per = 8 if E >= 64 else E
    w_router = _randn_bf16((E, H), W_STD, gen, device)
    w_gate = _randn_bf16((E, I, H), W_STD, gen, device, chunk_rows=per)
    w_up = _randn_bf16((E, I, H), W_STD, gen, device, chunk_rows=per)
    w_down = _randn_bf16((E, H, I), W_STD, gen, device, chunk_rows=per)
    return dict(w_router=w_router, w_gate=w_gate, w_up=w_up, w_down=w_down)


E4M3_MAX = 448.0  # largest finite FP8 E4M3 (OCP e4m3fn) value


def quantize_rows_e4m3(w: torch.Tensor, chunk: int = 8):
    """An FP8 copy of a stack of weight matrices [E, rows, cols]: one fp32 scale
    per row (its largest magnitude over 448, 1 for an all-zero row) and the E4M3
    codes of w / scale as uint8, both from torch's own float8_e4m3fn cast
    (round to nearest even).  Done in chunks of `chunk` matrices."""
    E, R, C = w.shape
    codes = torch.empty((E, R, C), dtype=torch.uint8, device=w.device)
    scales = torch.empty((E, R), dtype=torch.float32, device=w.device)
    for a in range(0, E, chunk):
        b = min(E, a + chunk)
        wf = w[a:b].float()
        amax = wf.abs().amax(dim=2)
        sc = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
        codes[a:b] = (wf / sc[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
        scales[a:b] = sc
        del wf
    return codes, scales


def make_weights_fp8(cfg: MoEConfig, seed: int = 0, device="cpu"):
    """The router weight of make_weights and an FP8 copy of its expert stacks
    (quantize_rows_e4m3): q_gate/q_up [E,I,H], q_down [E,H,I] uint8 codes with
    s_gate/s_up [E,I] and s_down [E,H] fp32 scales.  The bf16 expert weights are
    drawn exactly as make_weights draws them and then dropped."""
    w = make_weights(cfg, seed, device)
    out = dict(w_router=w.pop("w_router"))
    for name in ("gate", "up", "down"):
        q, s = quantize_rows_e4m3(w.pop("w_" + name))
        out["q_" + name], out["s_" + name] = q, s
    return out


def make_inputs(cfg: MoEConfig, seed: int = 0, device="cpu"):
    """Tokens and weights of one workload: x, bias, w_router, w_gate, w_up,
    w_down (see make_tokens and make_weights)."""
    d = make_tokens(cfg, seed, device)
    d.update(make_weights(cfg, seed, device))
    return d


def bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    import numpy as np
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
