"""GPU parity of the FP8-weight expert path (moe_forward_fp8,
moe_expert_ffn_fp8) against the oracle's FP8 expert (ffn_pairs_fp8) on the
GPU's own routing.

Small shapes are compared on every output; the Beam decode and prefill
shapes on seeded sampled (token, slot) pairs the oracle computes one by one.
Shapes reach the 16-row, 64-row and large tiles, ragged row tails and several
column tiles."""
import numpy as np
import pytest
import torch

import oracle
from group_limited_routing_router_amd.inputs import (CONFIGS, MoEConfig, bits, make_tokens,
                                                    make_weights_fp8)

from _parity import OUT_TOL, out_error

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from group_limited_routing_router_amd import moe as m
    m.load_library()
    return m


def _run(moe, cfg, d, w):
    p = moe.MoEProblem.from_config(cfg)
    b = moe.alloc_buffers(p)
    moe.moe_forward_fp8(p, d["x"], w["w_router"], d["bias"], w["q_gate"], w["s_gate"], w["q_up"],
                        w["s_up"], w["q_down"], w["s_down"], b["out"], b["topk_ids"],
                        b["topk_weights"], b["y"], b["ws"])
    moe.moe_permute(p, b["topk_ids"], b["expert_offsets"], b["sorted_pairs"], b["pair_rows"],
                    b["ws"])
    y2 = torch.empty_like(b["y"])
    moe.moe_expert_ffn_fp8(p, d["x"], b["sorted_pairs"], b["expert_offsets"], w["q_gate"],
                           w["s_gate"], w["q_up"], w["s_up"], w["q_down"], w["s_down"], y2, b["ws"])
    torch.cuda.synchronize()
    assert torch.equal(y2, b["y"]), "moe_expert_ffn_fp8 differs from the forward's expert step"
    return b


SMALL = [
    # (T, H, I, E, G, TG, k)
    (40, 256, 128, 16, 4, 2, 4),      # ~10 rows per expert: 16-row tiles
    (64, 256, 128, 16, 4, 2, 4),      # ~16 rows per expert: 64-row tiles
    (600, 512, 256, 16, 4, 2, 4),     # ~150 rows per expert: large tiles, ragged tails
    (33, 384, 192, 32, 4, 2, 6),
    (300, 256, 192, 8, 2, 1, 2),      # ~75 rows per expert, I not a multiple of 128: 64-row tiles
    (160, 256, 256, 8, 2, 1, 2),      # ~40 rows per expert: 64-row tiles, both reductions in stages of 128
    (300, 256, 256, 8, 2, 1, 2),      # ~75 rows per expert: large tiles
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "T%d_H%d_I%d_E%d_k%d" % (s[0], s[1], s[2], s[3], s[6]))
def test_fp8_small(moe, shape):
    T, H, I, E, G, TG, k = shape
    print(f"[case] fp8 T={T} H={H} I={I} E={E} k={k}", flush=True)
    cfg = MoEConfig("fp8", T=T, H=H, I=I, E=E, G=G, TG=TG, k=k, scale=2.5)
    d = {kk: v.cuda() for kk, v in make_tokens(cfg, seed=2).items()}
    w = {kk: v.cuda() for kk, v in make_weights_fp8(cfg, seed=2).items()}
    b = _run(moe, cfg, d, w)
    ids = b["topk_ids"].cpu().numpy()
    wts = b["topk_weights"].cpu().numpy()
    sp = b["sorted_pairs"].cpu().numpy()
    wc = {kk: v.cpu().numpy() for kk, v in w.items() if kk != "w_router"}
    xb = bits(d["x"].cpu())
    # y in sorted order on the GPU's routing
    tok = (sp // k).astype(np.int32)
    exp = ids.ravel()[sp].astype(np.int32)
    y_ref, _ = oracle.ffn_pairs_fp8(tok, exp, xb, wc["q_gate"], wc["s_gate"], wc["q_up"],
                                    wc["s_up"], wc["q_down"], wc["s_down"])
    ey, _ = out_error(b["y"].cpu().numpy(), y_ref)
    out_ref, _, _ = oracle.forward_with_routing_fp8(xb, ids, wts, wc["q_gate"], wc["s_gate"],
                                                    wc["q_up"], wc["s_up"], wc["q_down"],
                                                    wc["s_down"], cfg.scale)
    eo, rms = out_error(b["out"].cpu().numpy(), out_ref)
    print(f"    y_err/rms={ey:.2e} out_err/rms={eo:.2e} (rms {rms:.3f})", flush=True)
    assert ey <= OUT_TOL and eo <= OUT_TOL


@pytest.fixture(scope="module")
def beam_fp8():
    return make_weights_fp8(CONFIGS["decode"], seed=0, device="cuda")


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_fp8_beam_sampled(moe, beam_fp8, name):
    cfg = CONFIGS[name]
    print(f"[case] fp8 beam {name} T={cfg.T}", flush=True)
    d = make_tokens(cfg, seed=0, device="cuda")
    w = beam_fp8
    b = _run(moe, cfg, d, w)
    ids = b["topk_ids"].cpu().numpy()
    sp = b["sorted_pairs"].cpu().numpy()
    rng = np.random.default_rng(1)
    qsel = np.sort(rng.choice(sp.size, 16, replace=False))
    pairs = sp[qsel]
    tok = (pairs // cfg.k).astype(np.int32)
    exp_full = ids.ravel()[pairs].astype(np.int32)
    used = np.unique(exp_full)
    remap = {int(e): i for i, e in enumerate(used)}
    sel = torch.from_numpy(used).long().cuda()
    wc = {kk: w[kk].index_select(0, sel).cpu().numpy() for kk in
          ("q_gate", "s_gate", "q_up", "s_up", "q_down", "s_down")}
    y_ref, _ = oracle.ffn_pairs_fp8(tok, np.array([remap[int(e)] for e in exp_full], np.int32),
                                    bits(d["x"].cpu()), wc["q_gate"], wc["s_gate"], wc["q_up"],
                                    wc["s_up"], wc["q_down"], wc["s_down"])
    ey, rms = out_error(b["y"][torch.from_numpy(qsel).long().cuda()].cpu().numpy(), y_ref)
    print(f"    y_err/rms={ey:.2e} (rms {rms:.3f}) on {len(qsel)} sampled pairs", flush=True)
    assert ey <= OUT_TOL
