"""GPU parity of the dense SwiGLU MLP (moe_dense_mlp: one expert that takes
every token, on the expert kernels) against the oracle's SwiGLU expert.

Small shapes are compared on every output; wide ones on seeded sampled tokens
that the oracle computes one by one.  The shapes reach the 16-row, 64-row and
large-tile kernels and a ragged last row tile."""
import numpy as np
import pytest
import torch

import oracle
from group_limited_routing_router_amd.inputs import MoEConfig, bits, make_inputs

from _parity import OUT_TOL, out_error, stratified_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from group_limited_routing_router_amd import moe as m
    m.load_library()
    return m


CASES = [
    # (T, H, I, sampled tokens or 0 for all)
    (12, 256, 128, 0),        # 16-row tiles
    (64, 512, 256, 0),        # large tiles, one partly filled row tile
    (64, 384, 192, 0),        # I and H off the large tile's multiples: 64-row tiles
    (300, 512, 384, 0),       # large tiles with a ragged second row tile
    (1000, 256, 1024, 0),
    (2048, 5120, 2048, 24),   # Beam width, large tiles, sampled
    (8192, 5120, 20480, 256), # the benchmarked shape (intermediate 8 x 2560), sampled
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d_H%d_I%d" % c[:3])
def test_dense_mlp(moe, case):
    T, H, I, nsample = case
    print(f"[case] dense_mlp T={T} H={H} I={I}", flush=True)
    cfg = MoEConfig("dense", T=T, H=H, I=I, E=1, G=1, TG=1, k=1, scale=1.0)
    # the wide shapes are drawn on the GPU (a CPU draw of 0.3G values is slow)
    g = make_inputs(cfg, seed=5, device="cuda" if T * I > (1 << 24) else "cpu")
    g = {kk: v.cuda() for kk, v in g.items()}
    p = moe.MoEProblem.from_config(cfg)
    # sentinels: a skipped row tile leaves NaN in out (0xFF bytes are a bf16
    # NaN in the workspace's SwiGLU product)
    ws = torch.full((moe.moe_workspace_bytes(p),), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_dense_mlp(p, g["x"], g["w_gate"], g["w_up"], g["w_down"], out, ws)
    out2 = torch.full_like(out, float("nan"))
    moe.moe_dense_mlp(p, g["x"], g["w_gate"], g["w_up"], g["w_down"], out2, ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "unwritten element of out"
    assert torch.equal(out, out2), "dense MLP is not deterministic"
    if nsample:
        # the rows at every 256-row tile edge, the first and last, then random
        rng = np.random.default_rng(7)
        tok = stratified_tokens(np.array([0, T]), np.arange(T), 1, T, nsample, rng,
                                always=[0, T - 1]).astype(np.int32)
    else:
        tok = np.arange(T, dtype=np.int32)
    got = out[torch.from_numpy(tok.astype(np.int64)).cuda()].cpu().numpy()
    want, _ = oracle.ffn_pairs(tok, np.zeros_like(tok), bits(g["x"]), bits(g["w_gate"]),
                               bits(g["w_up"]), bits(g["w_down"]))
    err, rms = out_error(got, want)
    print(f"    err/rms={err:.2e} (rms {rms:.3f}) on {len(tok)} tokens", flush=True)
    assert err <= OUT_TOL
