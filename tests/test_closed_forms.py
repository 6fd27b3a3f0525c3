"""The Beam-shaped configs reproduce the size facts the pages print
(tests/golden/beam_closed_forms.json): three bias-free [I,H] matrices per
expert, 256 experts in each of 49 MoE layers, 8 routed per token."""
import json
import os

from group_limited_routing_router_amd.inputs import CONFIGS

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "beam_closed_forms.json")))


def _near(x, entry):
    step = entry.get("round_to", 1)
    return abs(x - entry["value"]) <= step / 2 + 1e-9


def test_beam_sizes():
    c = CONFIGS["prefill"]
    per_expert = 3 * c.H * c.I
    assert _near(per_expert / 1e6, GOLD["params_per_expert_millions"])
    layers = GOLD["moe_layers"]["value"]
    experts_total = layers * c.E * per_expert
    total = GOLD["total_params_billions"]["value"] * 1e9
    assert _near(100 * experts_total / total, GOLD["expert_share_percent"])
    rest = total - experts_total
    assert abs(rest / 1e9 - GOLD["replicated_params_billions"]["value"]) < 0.1
    active = layers * c.k * per_expert + GOLD["replicated_params_billions"]["value"] * 1e9
    assert _near(active / 1e9, GOLD["active_params_billions"])
    rep_gb = GOLD["replicated_bytes_gb"]["value"]
    assert _near(experts_total * 2 / 16 / 1e9 + rep_gb, GOLD["per_gpu_weights_gb_ep16"])
    assert _near(experts_total * 2 / 8 / 1e9 + rep_gb, GOLD["per_gpu_weights_gb_ep8"])
    # the group structure: 8 groups of 32, 4 kept, 8 routed
    assert (c.E, c.G, c.E // c.G, c.TG, c.k) == (256, 8, 32, 4, 8)
