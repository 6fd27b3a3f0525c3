"""moe_forward_noalloc (the workspace in the library's static device array)
against moe_forward (a caller workspace) through the C ABI: the same ids,
weights, expert outputs and block output, bit for bit, on two calls in a row,
the second with fewer tokens (the array keeps the first call's contents), and
a problem too large for the array refused with nothing written.  Outputs start
filled with sentinels."""
import pytest
import torch

from group_limited_routing_router_amd.inputs import CONFIGS, make_tokens, make_weights

from _parity import assert_forward_written, sentinel_buffers

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from group_limited_routing_router_amd import moe as m
    m.load_library()
    return m


def test_noalloc_forward_matches_forward(moe):
    w = make_weights(CONFIGS["decode"], seed=0, device="cuda")
    for T, out_dtype in ((512, torch.float32), (40, torch.bfloat16)):
        cfg = CONFIGS["decode"].with_(T=T)
        print(f"[case] noalloc T={T} out={out_dtype}", flush=True)
        d = make_tokens(cfg, seed=T, device="cuda")
        p = moe.MoEProblem.from_config(cfg)
        assert moe.moe_workspace_bytes(p) <= moe.NOALLOC_SCRATCH_BYTES
        ref = sentinel_buffers(moe, p, out_dtype=out_dtype)
        moe.moe_forward(p, d["x"], w["w_router"], d["bias"], w["w_gate"], w["w_up"], w["w_down"],
                        ref["out"], ref["topk_ids"], ref["topk_weights"], ref["y"], ref["ws"])
        got = sentinel_buffers(moe, p, out_dtype=out_dtype)
        moe.moe_forward_noalloc(p, d["x"], w["w_router"], d["bias"], w["w_gate"], w["w_up"],
                                w["w_down"], got["out"], got["topk_ids"], got["topk_weights"],
                                got["y"])
        torch.cuda.synchronize()
        assert_forward_written(got, T * cfg.k, cfg.E)
        for name in ("topk_ids", "topk_weights", "y", "out"):
            a, b = got[name], ref[name]
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), f"T={T}: {name} differs from moe_forward"
    # too large for the static array: refused, nothing written
    big = CONFIGS["decode"].with_(T=4096)
    p = moe.MoEProblem.from_config(big)
    assert moe.moe_workspace_bytes(p) > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((big.T, big.H), dtype=torch.bfloat16, device="cuda")
    out = torch.full((big.T, big.H), 7.0, dtype=torch.float32, device="cuda")
    y = torch.empty((big.T * big.k, big.H), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward_noalloc(p, x, w["w_router"], None, w["w_gate"], w["w_up"], w["w_down"],
                                out, None, None, y)
    assert ei.value.status == 2
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
