"""GPU parity at Beam's full sizes (hidden 5120, 256 experts in 8 groups of
32, 4 groups kept, k=8, intermediate 2560, scale 2.5) for the decode, prefill,
skew and long workloads, in the launch configuration the benchmark times
(moe_forward on one stream).

Every output buffer starts filled with a sentinel (NaN, -1, 0xFF bytes), so an
element no kernel writes fails the test.  The oracle routes every token (a
sample that covers every token past the 2 GiB mark of x for the 212992-token
case), checks the permutation of all pairs bit for bit, and recomputes the
SwiGLU product h, the expert outputs y and the block output for a seeded,
stratified sample of tokens one by one: the tokens whose rows sit at the edges
of the expert GEMMs' row tiles (first and last row of every expert, the rows
around the split of experts with more than 256 rows, every 256-row boundary
of the hot experts of the skewed workload) and random tokens for the rest."""
import numpy as np
import pytest
import torch

import oracle
from group_limited_routing_router_amd.inputs import CONFIGS, bits, make_tokens, make_weights

from _parity import (OUT_TOL, all_finite, assert_forward_written, compare_routing, h_error,
                     out_error, sentinel_buffers, stratified_tokens)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from group_limited_routing_router_amd import moe as m
    m.load_library()
    return m


@pytest.fixture(scope="module")
def beam_weights():
    """Beam-shaped weights on the GPU (20 GB) and their bf16 bits on the host,
    drawn once for the module and shared by the workloads."""
    print("[setup] Beam weights: draw on the GPU, copy to the host", flush=True)
    w = make_weights(CONFIGS["decode"], seed=0, device="cuda")
    host = {k: bits(v) for k, v in w.items()}
    yield w, host
    del w, host
    torch.cuda.empty_cache()


# "mid": 1536 tokens, about 48 rows per expert, a serving-size batch on the
# large tile with mostly partly filled row tiles.
# "huge": 212992 tokens, x above 2 GiB: the large tile's 32-bit buffer
# offsets into x pass 2^31 (unsigned) for the later tokens
# "t512": 512 tokens, 16 rows per expert: gate/up on 64-row tiles with the
# weights streamed past the caches, down on the large tile
EXTRA = {"mid": ("prefill", 1536), "t512": ("prefill", 512), "huge": ("long", 212992)}
# first token whose x row starts at or past byte 2^31 (H = 5120, bf16)
HUGE_FIRST_PAST = -(-(2 ** 31) // (5120 * 2))


def _cfg(name):
    if name in EXTRA:
        base, T = EXTRA[name]
        return CONFIGS[base].with_(name=name, T=T)
    return CONFIGS[name]


@pytest.mark.parametrize("name,ffn_sample,seed",
                         [("decode", 128, 0), ("decode", 128, 1), ("decode", 128, 2),
                          ("t512", 256, 0), ("mid", 256, 0), ("prefill", 1024, 0),
                          ("skew", 1024, 0),
                          ("long", 2048, 0), ("huge", 64, 0)])
def test_beam_config(moe, beam_weights, name, ffn_sample, seed):
    cfg = _cfg(name)
    T, k, E, H = cfg.T, cfg.k, cfg.E, cfg.H
    P = T * k
    w, wh = beam_weights
    print(f"[case] beam {name} T={T} token seed {seed}", flush=True)
    g = make_tokens(cfg, seed=seed, device="cuda")
    g.update(w)
    p = moe.MoEProblem.from_config(cfg)
    b = sentinel_buffers(moe, p)
    moe.moe_forward(p, g["x"], g["w_router"], g["bias"], g["w_gate"], g["w_up"], g["w_down"],
                    b["out"], b["topk_ids"], b["topk_weights"], b["y"], b["ws"])
    torch.cuda.synchronize()
    assert_forward_written(b, P, E)
    ids = b["topk_ids"].cpu().numpy()
    wts = b["topk_weights"].cpu().numpy()
    rng = np.random.default_rng(T + seed)

    # ---- routing: every token (huge: a sample holding every token past 2 GiB) ----
    if name == "huge":
        assert T * H * 2 >= 2 ** 31 and HUGE_FIRST_PAST < T
        past = np.arange(HUGE_FIRST_PAST, T)
        rt = np.union1d(past, rng.choice(HUGE_FIRST_PAST, 16384 - past.size, replace=False))
    else:
        rt = np.arange(T)
    xr = bits(g["x"]) if rt.size == T else bits(g["x"][torch.from_numpy(rt).cuda()])
    o_ids, o_w, s, gs = oracle.route(xr, wh["w_router"], g["bias"].cpu().numpy(), cfg.G, cfg.TG,
                                     k, want_scores=True)
    exempt, st = compare_routing(ids[rt], wts[rt], o_ids, o_w, s, gs, E, cfg.G, cfg.TG, k)
    print(f"    routed {rt.size} tokens, exempt {st['exempt']}", flush=True)
    del xr, s, gs
    if T <= 512:
        # the forward routes small batches with the experts split over
        # workgroups (scores through the workspace); moe_route keeps them in
        # one workgroup: the same ids and weights, bit for bit
        ids2 = torch.full_like(b["topk_ids"], -1)
        wts2 = torch.full_like(b["topk_weights"], float("nan"))
        moe.moe_route(p, g["x"], g["w_router"], g["bias"], ids2, wts2)
        torch.cuda.synchronize()
        assert torch.equal(ids2, b["topk_ids"]) and torch.equal(wts2, b["topk_weights"])

    # ---- permutation of all pairs, bit-exact against the oracle's sort ----
    off, sp, pr = oracle.permute(ids, E)
    # moe_forward keeps its permutation in the workspace; rerun the permute
    # call into caller buffers (still holding -1) to compare it
    moe.moe_permute(p, b["topk_ids"], b["expert_offsets"], b["sorted_pairs"], b["pair_rows"],
                    b["ws"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(b["expert_offsets"].cpu().numpy(), off)
    np.testing.assert_array_equal(b["sorted_pairs"].cpu().numpy(), sp)
    np.testing.assert_array_equal(b["pair_rows"].cpu().numpy(), pr)

    # ---- h from the same gate/up kernel into a NaN-filled buffer ----
    moe.moe_expert_gate_up(p, g["x"], b["sorted_pairs"], b["expert_offsets"], g["w_gate"],
                           g["w_up"], b["h"])
    torch.cuda.synchronize()
    assert all_finite(b["h"]), "unwritten row of h"

    if name == "prefill":
        # bf16 output with y streamed past the caches: exactly the nearest-even
        # cast of the fp32 output
        out16 = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        moe.moe_forward(p, g["x"], g["w_router"], g["bias"], g["w_gate"], g["w_up"], g["w_down"],
                        out16, None, None, b["y"], b["ws"])
        torch.cuda.synchronize()
        assert torch.equal(out16.view(torch.int16), b["out"].to(torch.bfloat16).view(torch.int16))
        del out16
    if name == "skew":
        hot = np.nonzero(g["bias"].cpu().numpy() > 0)[0]
        share = np.isin(ids, hot).mean()
        print(f"    hot-expert share of pairs: {share:.3f}", flush=True)
        assert share > 0.5

    # ---- h, y and out on a stratified sample of tokens ----
    always = [0, T - 1]
    if name == "huge":
        always += list(rng.choice(np.arange(HUGE_FIRST_PAST, T), 15, replace=False))
    ft = stratified_tokens(off, sp, k, T, ffn_sample, rng, always=always)
    if name == "huge":
        assert (ft >= HUGE_FIRST_PAST).sum() >= 16
    xf = bits(g["x"][torch.from_numpy(ft).cuda()])
    out_ref, y_ref, h_ref = oracle.forward_with_routing(xf, ids[ft], wts[ft], wh["w_gate"],
                                                        wh["w_up"], wh["w_down"], cfg.scale,
                                                        want_h=True)
    # gather the sampled rows on the GPU before the copy (y is 1-35 GB here)
    rows = torch.from_numpy(pr.reshape(T, k)[ft].ravel().astype(np.int64)).cuda()
    y_rows = b["y"][rows].cpu().numpy()
    h_rows = b["h"][rows].float().cpu().numpy()
    out_rows = b["out"][torch.from_numpy(ft).cuda()].cpu().numpy()
    eh = h_error(h_rows, oracle.bf16_to_f32(h_ref))
    ey, _ = out_error(y_rows, y_ref)
    eo, rms = out_error(out_rows, out_ref)
    print(f"    h_err/bound={eh:.2f} y_err/rms={ey:.2e} out_err/rms={eo:.2e} (rms {rms:.3f}) "
          f"on {ft.size} tokens", flush=True)
    assert eh <= 1.0 and ey <= OUT_TOL and eo <= OUT_TOL
    del b, g
    torch.cuda.empty_cache()
