"""Pins for the oracle's FP8-weight expert (ffn_pairs_fp8).

Reading: expert weights stored as FP8 E4M3 codes (OCP e4m3fn) with one fp32
scale per output channel; a channel's dot product is its scale times the dot
product with the decoded codes.  Pinned by torch's float8_e4m3fn decoding of
all 256 codes, and by bit equality with the bf16 expert (ffn_pairs) when every
scale is a power of two: the scaled weights are then exact in bf16 and a
power-of-two scale commutes with every fp32 rounding of the sums."""
import numpy as np
import torch

from group_limited_routing_router_amd.inputs import CONFIGS, bits, make_inputs


def test_decode_matches_torch_e4m3fn(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    got = oracle_mod.e4m3_decode(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    np.testing.assert_array_equal(got[~nan], want[~nan])


def _random_codes(shape, rng):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    return c


def _pow2_case(seed=0, T=24, E=4, H=256, I=128):
    rng = np.random.default_rng(seed)
    cfg = CONFIGS["tiny"].with_(T=T, E=E, G=1, TG=1, k=1, H=H, I=I)
    x = bits(make_inputs(cfg, seed=seed)["x"])
    q = {n: _random_codes(s, rng) for n, s in (("g", (E, I, H)), ("u", (E, I, H)),
                                                ("d", (E, H, I)))}
    s = {n: np.exp2(rng.integers(-12, -5, size=q[n].shape[:2])).astype(np.float32) for n in q}
    tok = np.repeat(np.arange(T, dtype=np.int32), 2)
    exp = rng.integers(0, E, size=2 * T).astype(np.int32)
    return x, q, s, tok, exp


def _as_bf16_weights(oracle_mod, q, s):
    w = oracle_mod.e4m3_decode(q).astype(np.float64) * s[..., None]
    return torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16), w


def test_power_of_two_scales_equal_the_bf16_expert(oracle_mod):
    x, q, s, tok, exp = _pow2_case()
    wb = {}
    for n in q:
        wb[n], w64 = _as_bf16_weights(oracle_mod, q[n], s[n])
        # the scaled weights are exact in bf16
        back = torch.from_numpy(wb[n].view(np.int16)).view(torch.bfloat16).double().numpy()
        np.testing.assert_array_equal(back, w64)
    y8, h8 = oracle_mod.ffn_pairs_fp8(tok, exp, x, q["g"], s["g"], q["u"], s["u"], q["d"], s["d"],
                                      want_h=True)
    y16, h16 = oracle_mod.ffn_pairs(tok, exp, x, wb["g"], wb["u"], wb["d"], want_h=True)
    np.testing.assert_array_equal(h8, h16)
    np.testing.assert_array_equal(y8, y16)


def test_down_scale_is_linear_and_zero_codes_give_zero(oracle_mod):
    x, q, s, tok, exp = _pow2_case(seed=1)
    y1, _ = oracle_mod.ffn_pairs_fp8(tok, exp, x, q["g"], s["g"], q["u"], s["u"], q["d"], s["d"])
    y3, _ = oracle_mod.ffn_pairs_fp8(tok, exp, x, q["g"], s["g"], q["u"], s["u"], q["d"],
                                     s["d"] * np.float32(3.0))
    np.testing.assert_array_equal(y3, np.float32(3.0) * y1)
    zero = np.zeros_like(q["u"])
    y0, h0 = oracle_mod.ffn_pairs_fp8(tok, exp, x, q["g"], s["g"], zero, s["u"], q["d"], s["d"],
                                      want_h=True)
    assert not np.any(h0 & 0x7FFF) and not np.any(y0)
