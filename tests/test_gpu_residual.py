"""GPU parity of the combine fused with the sublayer epilogue
(moe_combine_residual) against the oracle.

Two checks per case: (1) on the GPU's own expert outputs, the fused call must
match the oracle's epilogue applied to what moe_combine writes, to fp32
rounding (only the order of the sum of squares differs); (2) end to end
against the oracle's block output on the same routing, within the output
tolerance of the block.  Shapes cover one, two, four (with a ragged tail),
eight and sixteen float4 chunks per thread."""
import numpy as np
import pytest
import torch

import oracle
from group_limited_routing_router_amd.inputs import CONFIGS, MoEConfig, bits, make_inputs

from _parity import OUT_TOL, assert_forward_written, out_error, sentinel_buffers

pytestmark = pytest.mark.gpu

EPS = 1e-6


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from group_limited_routing_router_amd import moe as m
    m.load_library()
    return m


CASES = [
    # (T, H, I, E, G, TG, k, scale, step)
    (64, 256, 128, 16, 4, 2, 4, 1.0, 1),
    (64, 256, 128, 16, 4, 2, 4, 2.5, 2),
    (37, 512, 64, 8, 2, 1, 2, 2.5, 7),
    (50, 2176, 64, 16, 4, 2, 4, 2.5, 3),      # 544 float4 chunks: one pass of 9 waves
    (300, 2176, 64, 16, 4, 2, 4, 2.5, 9),     # the same row with 256 threads: three chunks each, ragged
    (40, 5120, 128, 16, 4, 2, 4, 2.5, 104),   # Beam width
    (16, 16384, 64, 8, 2, 1, 2, 2.5, 5),      # the widest row the fused call takes
    (2048, 5120, 64, 16, 4, 2, 8, 2.5, 3),    # y of 335 MB: read past the caches (nontemporal)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d_H%d_k%d_s%d" % (c[0], c[1], c[6], c[8]))
def test_combine_residual(moe, case):
    T, H, I, E, G, TG, k, scale, step = case
    print(f"[case] combine_residual T={T} H={H} k={k} step={step}", flush=True)
    cfg = MoEConfig("res", T=T, H=H, I=I, E=E, G=G, TG=TG, k=k, scale=scale)
    d = make_inputs(cfg, seed=3)
    g = {kk: v.cuda() for kk, v in d.items()}
    p = moe.MoEProblem.from_config(cfg)
    b = sentinel_buffers(moe, p)
    moe.moe_forward(p, g["x"], g["w_router"], g["bias"], g["w_gate"], g["w_up"], g["w_down"],
                    b["out"], b["topk_ids"], b["topk_weights"], b["y"], b["ws"])
    moe.moe_permute(p, b["topk_ids"], b["expert_offsets"], b["sorted_pairs"], b["pair_rows"],
                    b["ws"])
    rng = np.random.default_rng(11)
    gain = torch.from_numpy((rng.normal(size=H) * 0.1 + 1.0).astype(np.float32)).cuda()
    stream0 = torch.from_numpy(rng.normal(size=(T, H)).astype(np.float32)).cuda()
    res = stream0.clone()
    moe.moe_combine_residual(p, b["y"], b["pair_rows"], b["topk_weights"], gain, EPS, step, res)
    res2 = stream0.clone()
    moe.moe_combine_residual(p, b["y"], b["pair_rows"], b["topk_weights"], gain, EPS, step, res2)
    torch.cuda.synchronize()
    assert_forward_written(b, T * k, E)
    assert bool(torch.isfinite(res).all()), "residual row not updated"
    assert torch.equal(res, res2), "fused epilogue is not deterministic"
    got = res.cpu().numpy()
    gain_np, s0 = gain.cpu().numpy(), stream0.cpu().numpy()
    # (1) against the oracle's epilogue on the GPU's own combined output
    want = oracle.residual_norm(b["out"].cpu().numpy(), gain_np, EPS, step, s0)
    e1, rms = out_error(got, want)
    assert e1 <= 1e-5, f"epilogue err {e1} (rms {rms})"
    # (2) end to end on the GPU's routing
    ref_out, _, _ = oracle.forward_with_routing(bits(d["x"]), b["topk_ids"].cpu().numpy(),
                                                b["topk_weights"].cpu().numpy(), bits(d["w_gate"]),
                                                bits(d["w_up"]), bits(d["w_down"]), scale)
    want2 = oracle.residual_norm(ref_out, gain_np, EPS, step, s0)
    e2, _ = out_error(got, want2)
    print(f"    epilogue err/rms={e1:.2e} end-to-end err/rms={e2:.2e}", flush=True)
    assert e2 <= OUT_TOL
