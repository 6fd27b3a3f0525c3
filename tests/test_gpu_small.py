"""GPU parity on small shapes: every C-ABI call against the oracle, element by
element, on seeded inputs that span several tiles and ragged tails, plus the
degenerate cases of the method (k=1, k=E with one group, groups of one
expert, every token on the same experts, exact ties)."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, Phase, given, settings
from hypothesis import strategies as hst

import oracle
from group_limited_routing_router_amd.inputs import CONFIGS, MoEConfig, bits, make_inputs

from _parity import (OUT_TOL, assert_forward_written, compare_routing, out_error,
                     sentinel_buffers)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from group_limited_routing_router_amd import moe as m
    m.load_library()
    return m


def _to_gpu(d):
    return {k: v.cuda() for k, v in d.items()}


def _run_steps(moe, cfg, g, bias=True):
    """The four steps into sentinel-filled buffers (NaN, -1, 0xFF): every
    output element must be written."""
    p = moe.MoEProblem.from_config(cfg)
    b = sentinel_buffers(moe, p)
    moe.moe_route(p, g["x"], g["w_router"], g["bias"] if bias else None, b["topk_ids"],
                  b["topk_weights"])
    moe.moe_permute(p, b["topk_ids"], b["expert_offsets"], b["sorted_pairs"], b["pair_rows"],
                    b["ws"])
    moe.moe_expert_ffn(p, g["x"], b["sorted_pairs"], b["expert_offsets"], g["w_gate"], g["w_up"],
                       g["w_down"], b["y"], b["ws"])
    moe.moe_combine(p, b["y"], b["pair_rows"], b["topk_weights"], b["out"])
    torch.cuda.synchronize()
    assert_forward_written(b, cfg.T * cfg.k, cfg.E)
    assert int(b["sorted_pairs"].min()) >= 0 and int(b["pair_rows"].min()) >= 0
    return p, {k: v.cpu().numpy() if v.dtype != torch.bfloat16 else v.cpu() for k, v in b.items()}


def _check_all(moe, cfg, d, label):
    print(f"[case] {label} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} G={cfg.G} TG={cfg.TG} "
          f"k={cfg.k}", flush=True)
    g = _to_gpu(d)
    p, r = _run_steps(moe, cfg, g)
    xb, wrb = bits(d["x"]), bits(d["w_router"])
    wgb, wub, wdb = bits(d["w_gate"]), bits(d["w_up"]), bits(d["w_down"])
    bias = d["bias"].numpy()
    # 1. routing
    o_ids, o_w, s, gs = oracle.route(xb, wrb, bias, cfg.G, cfg.TG, cfg.k, want_scores=True)
    exempt, st = compare_routing(r["topk_ids"], r["topk_weights"], o_ids, o_w, s, gs,
                                 cfg.E, cfg.G, cfg.TG, cfg.k)
    # 2. permutation of the GPU's own ids: bit-exact
    off, sp, pr = oracle.permute(r["topk_ids"], cfg.E)
    np.testing.assert_array_equal(r["expert_offsets"], off)
    np.testing.assert_array_equal(r["sorted_pairs"], sp)
    np.testing.assert_array_equal(r["pair_rows"], pr)
    # 3. expert FFN on the GPU's routing: y in sorted order
    ids_flat = r["topk_ids"].ravel()
    tok = (sp // cfg.k).astype(np.int32)
    exp = ids_flat[sp].astype(np.int32)
    y_ref, _ = oracle.ffn_pairs(tok, exp, xb, wgb, wub, wdb)
    ey, _ = out_error(r["y"], y_ref)
    assert ey <= OUT_TOL, f"y err {ey}"
    # 4. combine of the GPU's y: tight, only fp32 rounding differs
    y_pairs = r["y"][pr]
    out_c = oracle.combine(y_pairs, r["topk_weights"], cfg.scale)
    ec, _ = out_error(r["out"], out_c)
    assert ec <= 1e-5, f"combine err {ec}"
    # 5. end to end against the oracle's own routing (GPU routing on exempt tokens)
    ref = oracle.forward(xb, wrb, bias, wgb, wub, wdb, cfg.G, cfg.TG, cfg.k, cfg.scale)["out"]
    if exempt.any():
        inj, _, _ = oracle.forward_with_routing(xb, r["topk_ids"], r["topk_weights"], wgb, wub,
                                                wdb, cfg.scale)
        ref[exempt] = inj[exempt]
    eo, rms = out_error(r["out"], ref)
    print(f"    exempt={st['exempt']} y_err/rms={ey:.2e} out_err/rms={eo:.2e}", flush=True)
    assert eo <= OUT_TOL
    return g, r


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_all_steps(moe, seed):
    cfg = CONFIGS["tiny"]
    _check_all(moe, cfg, make_inputs(cfg, seed=seed), f"tiny seed={seed}")


SHAPES = [
    # (T, H, I, E, G, TG, k) -- chosen to hit every tile configuration,
    # ragged row tails and partial token tiles of the router
    (1, 256, 128, 16, 4, 2, 4),
    (17, 384, 192, 32, 4, 2, 6),
    (200, 256, 64, 64, 8, 3, 8),
    (300, 512, 256, 256, 8, 4, 8),
    (1000, 256, 128, 32, 4, 2, 2),
    (3000, 256, 128, 16, 4, 2, 4),
    (5000, 128, 64, 16, 4, 2, 4),
    (2000, 512, 256, 8, 2, 1, 2),       # ~500 rows per expert: two large row tiles
    (1500, 256, 384, 16, 4, 2, 4),      # ~375 rows per expert, I not a power of two
    (2600, 256, 128, 8, 2, 1, 2),       # ~650 rows per expert: 256 + 256 + ragged last row tile
    (2400, 256, 128, 12, 4, 2, 2),      # ~400 rows per expert, 8 does not divide E
    (1200, 256, 128, 256, 8, 4, 16),    # the largest k, MFMA router (more than 512 tokens)
    (200, 256, 128, 256, 8, 8, 16),     # the largest k, every group kept, small-batch router
    (300, 256, 128, 24, 3, 2, 6),       # three groups of eight
    (100, 256, 128, 4, 2, 1, 2),        # fewer experts than router waves
    (8230, 128, 64, 16, 4, 2, 4),       # above 8192 tokens: 64-token router tiles, ragged last tile
    (8300, 256, 64, 256, 8, 4, 8),      # the same with 256 experts
    (600, 512, 256, 64, 8, 4, 4),       # ~38 rows per expert: large tiles of one or two row blocks
    (400, 256, 128, 32, 4, 2, 2),       # ~25 rows per expert: 64-row gate/up tiles, weights streamed
    # the largest H and I the library takes (65536), on the large tile (75
    # rows per expert; gate/up over K = 65536, or K = 128 in two stages) and
    # on 16-row tiles (6 rows per expert)
    (300, 65536, 128, 8, 2, 1, 2),
    (300, 128, 65536, 8, 2, 1, 2),
    (24, 65536, 128, 8, 2, 1, 2),
    (24, 128, 65536, 8, 2, 1, 2),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "T%d_H%d_I%d_E%d_G%d_TG%d_k%d" % s)
def test_shapes(moe, shape):
    T, H, I, E, G, TG, k = shape
    cfg = MoEConfig("sweep", T=T, H=H, I=I, E=E, G=G, TG=TG, k=k, scale=2.5)
    _check_all(moe, cfg, make_inputs(cfg, seed=T), "sweep")


def test_dense_all_experts(moe):
    """k = E with one group: the dense mixture over all experts."""
    cfg = MoEConfig("dense", T=96, H=256, I=128, E=16, G=1, TG=1, k=16, scale=1.0)
    _check_all(moe, cfg, make_inputs(cfg, seed=5), "dense k=E")


def test_k1_and_groups_of_one(moe):
    cfg = MoEConfig("k1", T=130, H=128, I=64, E=8, G=8, TG=8, k=1, scale=2.5)
    _check_all(moe, cfg, make_inputs(cfg, seed=6), "k=1, group size 1")
    cfg = MoEConfig("g1", T=70, H=256, I=128, E=32, G=32, TG=5, k=3, scale=2.5)
    _check_all(moe, cfg, make_inputs(cfg, seed=7), "groups of one expert")


def test_all_tokens_on_same_experts(moe):
    """Extreme skew: a +6 logit bias on 4 experts sends every token there."""
    cfg = MoEConfig("skewed", T=700, H=256, I=128, E=32, G=4, TG=2, k=4, scale=2.5)
    d = make_inputs(cfg, seed=8)
    d["bias"][[5, 6, 9, 12]] = 6.0
    g, r = _check_all(moe, cfg, d, "all tokens on 4 experts")
    counts = np.diff(r["expert_offsets"])
    assert counts[[5, 6, 9, 12]].sum() >= 0.95 * cfg.T * cfg.k


def test_exact_ties_lower_index(moe):
    """Duplicate router rows give identical logits on any summation order; a
    +100 bias saturates the sigmoid to 1.0.  The lower index must win."""
    cfg = CONFIGS["tiny"]
    d = make_inputs(cfg, seed=4)
    d["w_router"][9] = d["w_router"][3]
    d["w_router"][2] = d["w_router"][3]
    d["bias"][[1, 3]] = 100.0
    g, r = _check_all(moe, cfg, d, "ties")
    assert np.all(r["topk_ids"][:, 0] == 1) and np.all(r["topk_ids"][:, 1] == 3)


def test_forward_matches_steps_bf16_and_determinism(moe):
    cfg = CONFIGS["tiny"].with_(T=333, scale=2.5)
    d = make_inputs(cfg, seed=9)
    g = _to_gpu(d)
    p, r = _run_steps(moe, cfg, g)
    outs = []
    for dtype in (torch.float32, torch.float32, torch.bfloat16):
        b = sentinel_buffers(moe, p, out_dtype=dtype)
        moe.moe_forward(p, g["x"], g["w_router"], g["bias"], g["w_gate"], g["w_up"], g["w_down"],
                        b["out"], b["topk_ids"], b["topk_weights"], b["y"], b["ws"])
        torch.cuda.synchronize()
        outs.append(b["out"].cpu())
        np.testing.assert_array_equal(b["topk_ids"].cpu().numpy(), r["topk_ids"])
        np.testing.assert_array_equal(b["topk_weights"].cpu().numpy(), r["topk_weights"])
    # the composed call equals the four steps, bit for bit, and repeats exactly
    np.testing.assert_array_equal(outs[0].numpy(), r["out"])
    assert torch.equal(outs[0], outs[1])
    # bf16 output is the round-to-nearest-even cast of the fp32 output
    assert torch.equal(outs[2].view(torch.int16), outs[0].to(torch.bfloat16).view(torch.int16))
    # forward without routing outputs (kept in the workspace) gives the same out
    b = sentinel_buffers(moe, p)
    moe.moe_forward(p, g["x"], g["w_router"], g["bias"], g["w_gate"], g["w_up"], g["w_down"],
                    b["out"], None, None, b["y"], b["ws"])
    torch.cuda.synchronize()
    assert torch.equal(b["out"].cpu(), outs[0])


def test_zero_tokens_gpu(moe):
    cfg = CONFIGS["tiny"]
    p = moe.MoEProblem.from_config(cfg, T=0)
    b = moe.alloc_buffers(p)
    moe.moe_forward(p, None, None, None, None, None, None, b["out"], None, None, None, None)
    torch.cuda.synchronize()


@pytest.mark.parametrize("T", [700, 1500])
def test_permute_drops_out_of_range_ids(moe, T):
    """moe_permute's documented handling of ids outside [0, E): the pair is
    dropped (pair_rows = -1), expert_offsets count only the kept pairs, the
    kept pairs keep the stable order, and sorted positions past the kept
    pairs are not written.  moe_combine then counts a dropped pair as 0.
    (The oracle rejects such ids -- they are not routing results -- so the
    expected permutation here is numpy's stable sort of the kept pairs.)
    700 tokens use the one-workgroup permutation, 1500 the three launches."""
    cfg = MoEConfig("drop", T=T, H=256, I=128, E=16, G=4, TG=2, k=4, scale=2.5)
    E, k = cfg.E, cfg.k
    print(f"[case] permute drop T={T}", flush=True)
    rng = np.random.default_rng(T)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    bad = rng.random((T, k)) < 0.1
    ids[bad] = rng.choice(np.array([-1, -100, E, E + 5, 2 ** 31 - 1], np.int32), int(bad.sum()))
    p = moe.MoEProblem.from_config(cfg)
    b = sentinel_buffers(moe, p)
    for key in ("sorted_pairs", "pair_rows", "expert_offsets"):
        b[key].fill_(-7)
    gi = torch.from_numpy(ids).cuda()
    moe.moe_permute(p, gi, b["expert_offsets"], b["sorted_pairs"], b["pair_rows"], b["ws"])
    torch.cuda.synchronize()
    flat = ids.ravel()
    keep = (flat >= 0) & (flat < E)
    kept = np.nonzero(keep)[0]
    order = kept[np.argsort(flat[kept], kind="stable")]
    off = np.concatenate([[0], np.cumsum(np.bincount(flat[kept], minlength=E))]).astype(np.int32)
    rows = np.full(T * k, -1, np.int32)
    rows[order] = np.arange(order.size, dtype=np.int32)
    np.testing.assert_array_equal(b["expert_offsets"].cpu().numpy(), off)
    sp = b["sorted_pairs"].cpu().numpy()
    np.testing.assert_array_equal(sp[:order.size], order)
    assert np.all(sp[order.size:] == -7), "sorted positions past the kept pairs were written"
    np.testing.assert_array_equal(b["pair_rows"].cpu().numpy(), rows)
    # combine: dropped pairs contribute 0
    y = torch.randn((T * k, cfg.H), dtype=torch.float32, device="cuda")
    w = torch.rand((T, k), dtype=torch.float32, device="cuda")
    moe.moe_combine(p, y, b["pair_rows"], w, b["out"])
    torch.cuda.synchronize()
    yp = np.zeros((T * k, cfg.H), np.float32)
    yp[kept] = y.cpu().numpy()[rows[kept]]
    want = oracle.combine(yp, w.cpu().numpy(), cfg.scale)
    err, _ = out_error(b["out"].cpu().numpy(), want)
    assert err <= 1e-5


@hst.composite
def _problems(draw):
    G = draw(hst.sampled_from([1, 2, 3, 4, 8]))
    per = draw(hst.sampled_from([1, 2, 4, 8, 16, 32]))
    TG = draw(hst.integers(1, G))
    k = draw(hst.integers(1, min(16, TG * per)))
    H = draw(hst.sampled_from([128, 256, 384, 512]))
    I = draw(hst.sampled_from([64, 128, 192, 256, 384]))
    T = draw(hst.integers(1, 640))
    seed = draw(hst.integers(0, 2 ** 20))
    return (T, H, I, G * per, G, TG, k, seed)


@settings(max_examples=40, deadline=None, derandomize=True, database=None,
          phases=(Phase.explicit, Phase.generate), print_blob=True,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(prob=_problems())
def test_property_random_shapes(moe, prob):
    """Hypothesis over small (T, H, I, E, G, TG, k): every step against the
    oracle (routing, exact permutation, y, combine, end to end) with sentinel
    outputs.  Examples are derived deterministically and not shrunk: the run
    stops at the first failing example, which it prints."""
    T, H, I, E, G, TG, k, seed = prob
    cfg = MoEConfig("prop", T=T, H=H, I=I, E=E, G=G, TG=TG, k=k, scale=2.5)
    _check_all(moe, cfg, make_inputs(cfg, seed=seed), f"property seed={seed}")
