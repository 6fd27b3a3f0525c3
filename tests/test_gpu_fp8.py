"""GPU parity of the FP8-weight expert path (moe_forward_fp8,
moe_expert_ffn_fp8) against the oracle's FP8 expert (ffn_pairs_fp8) on the
GPU's own routing.

Small shapes are compared on every output; the Beam decode, prefill, skew,
long and 212992-token shapes on a seeded, stratified sample of tokens the
oracle computes one by one (y and the block output).  Outputs start filled
with sentinels, so an element no kernel writes fails the test.
Shapes reach the 16-row, 64-row and large tiles, ragged row tails and several
column tiles."""
import numpy as np
import pytest
import torch

import oracle
from group_limited_routing_router_amd.inputs import (CONFIGS, MoEConfig, bits, make_tokens,
                                                    make_weights_fp8)

from _parity import (OUT_TOL, assert_forward_written, out_error, sentinel_buffers,
                     stratified_tokens)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from group_limited_routing_router_amd import moe as m
    m.load_library()
    return m


def _run(moe, cfg, d, w):
    """moe_forward_fp8 into sentinel-filled buffers, then the permutation into
    caller buffers and moe_expert_ffn_fp8 into a NaN-filled y: it must equal
    the forward's expert step bit for bit."""
    p = moe.MoEProblem.from_config(cfg)
    b = sentinel_buffers(moe, p)
    moe.moe_forward_fp8(p, d["x"], w["w_router"], d["bias"], w["q_gate"], w["s_gate"], w["q_up"],
                        w["s_up"], w["q_down"], w["s_down"], b["out"], b["topk_ids"],
                        b["topk_weights"], b["y"], b["ws"])
    torch.cuda.synchronize()
    assert_forward_written(b, cfg.T * cfg.k, cfg.E)
    moe.moe_permute(p, b["topk_ids"], b["expert_offsets"], b["sorted_pairs"], b["pair_rows"],
                    b["ws"])
    y2 = torch.full_like(b["y"], float("nan"))
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
    (300, 65536, 128, 8, 2, 1, 2),    # the largest H: large tiles over K = 65536
    (24, 128, 65536, 8, 2, 1, 2),     # the largest I: 16-row tiles, down over K = 65536
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
    """FP8 copies of the Beam-shaped expert weights on the GPU (10 GB) and on
    the host, drawn once for the module."""
    print("[setup] Beam FP8 weights: draw and quantise on the GPU, copy to the host", flush=True)
    w = make_weights_fp8(CONFIGS["decode"], seed=0, device="cuda")
    host = {kk: v.cpu().numpy() for kk, v in w.items() if kk != "w_router"}
    yield w, host
    del w, host
    torch.cuda.empty_cache()


# first token whose x row starts at or past byte 2^31 (H = 5120, bf16)
HUGE_FIRST_PAST = -(-(2 ** 31) // (5120 * 2))


@pytest.mark.parametrize("name,nsample", [("decode", 128), ("prefill", 256), ("skew", 256),
                                          ("long", 512), ("huge", 32)])
def test_fp8_beam_sampled(moe, beam_fp8, name, nsample):
    """moe_forward_fp8 at Beam sizes: no sentinel survives in out, y, ids or
    weights; y and out of a stratified token sample (the tokens at the edges
    of the row tiles, then random ones) against the oracle's FP8 expert on the
    GPU's routing.  "huge" (212992 tokens) puts x above 2 GiB, where the large
    tile's 32-bit buffer offsets into x pass 2^31."""
    cfg = CONFIGS["long"].with_(name="huge", T=212992) if name == "huge" else CONFIGS[name]
    T, k = cfg.T, cfg.k
    print(f"[case] fp8 beam {name} T={T}", flush=True)
    d = make_tokens(cfg, seed=0, device="cuda")
    w, wh = beam_fp8
    b = _run(moe, cfg, d, w)
    ids = b["topk_ids"].cpu().numpy()
    wts = b["topk_weights"].cpu().numpy()
    off = b["expert_offsets"].cpu().numpy()
    sp = b["sorted_pairs"].cpu().numpy()
    pr = b["pair_rows"].cpu().numpy()
    rng = np.random.default_rng(1)
    always = [0, T - 1]
    if name == "huge":
        assert T * cfg.H * 2 >= 2 ** 31
        always += list(rng.choice(np.arange(HUGE_FIRST_PAST, T), 7, replace=False))
    ft = stratified_tokens(off, sp, k, T, nsample, rng, always=always)
    xf = bits(d["x"][torch.from_numpy(ft).cuda()])
    out_ref, y_ref, _ = oracle.forward_with_routing_fp8(
        xf, ids[ft], wts[ft], wh["q_gate"], wh["s_gate"], wh["q_up"], wh["s_up"], wh["q_down"],
        wh["s_down"], cfg.scale)
    rows = torch.from_numpy(pr.reshape(T, k)[ft].ravel().astype(np.int64)).cuda()
    ey, _ = out_error(b["y"][rows].cpu().numpy(), y_ref)
    eo, rms = out_error(b["out"][torch.from_numpy(ft).cuda()].cpu().numpy(), out_ref)
    print(f"    y_err/rms={ey:.2e} out_err/rms={eo:.2e} (rms {rms:.3f}) on {ft.size} tokens",
          flush=True)
    assert ey <= OUT_TOL and eo <= OUT_TOL
    del b, d
    torch.cuda.empty_cache()
