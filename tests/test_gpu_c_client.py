"""The library driven by a plain C program (tests/c_client/moe_client.c): no
Python and no torch in that process, only include/moe.h and the HIP runtime's
C API.  The program checks the documented host-side errors itself, runs
moe_forward with fp32 and with bf16 output, and writes its seeded inputs and
the outputs to files.  Here they are compared with the oracle on those same
inputs: routing bit-exact outside the 1e-5 boundary gaps, the fp32 output
within 2e-2 x RMS, the bf16 output exactly the nearest-even cast of the fp32
one."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from _parity import OUT_TOL, compare_routing, out_error

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_client", "moe_client")

CASES = [
    # (T, H, I, E, G, TG, k, scale, seed)
    (64, 256, 128, 16, 4, 2, 4, 1.0, 1),      # the tiny layer; small-batch router
    (300, 512, 256, 64, 8, 4, 8, 2.5, 2),     # 8 groups, k = 8
    (1100, 256, 128, 32, 4, 2, 4, 2.5, 3),    # MFMA router, large-tile expert GEMMs
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d_H%d_I%d_E%d_G%d_TG%d_k%d" % c[:7])
def test_c_client_forward(tmp_path, case):
    T, H, I, E, G, TG, k, scale, seed = case
    assert os.path.exists(CLIENT), f"{CLIENT} is missing: run __graft_entry__.build() first"
    print(f"[case] C client T={T} H={H} I={I} E={E} G={G} TG={TG} k={k} seed={seed}", flush=True)
    r = subprocess.run([CLIENT, str(tmp_path), *(str(v) for v in case)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, f"moe_client exited with {r.returncode}:\n{r.stdout}{r.stderr}"
    assert "moe_client ok" in r.stdout

    def load(name, dtype, shape):
        return np.fromfile(tmp_path / name, dtype=dtype).reshape(shape)

    xb = load("x.bin", np.uint16, (T, H))
    wrb = load("w_router.bin", np.uint16, (E, H))
    bias = load("bias.bin", np.float32, (E,))
    wgb = load("w_gate.bin", np.uint16, (E, I, H))
    wub = load("w_up.bin", np.uint16, (E, I, H))
    wdb = load("w_down.bin", np.uint16, (E, H, I))
    out = load("out.bin", np.float32, (T, H))
    out16 = load("out_bf16.bin", np.uint16, (T, H))
    ids = load("ids.bin", np.int32, (T, k))
    w = load("weights.bin", np.float32, (T, k))
    # the generator's draws look like the configured distributions
    x = oracle.bf16_to_f32(xb)
    assert abs(float(x.mean())) < 0.05 and 0.95 < float(x.std()) < 1.05

    ref = oracle.forward(xb, wrb, bias, wgb, wub, wdb, G, TG, k, scale)
    exempt, st = compare_routing(ids, w, ref["ids"], ref["weights"], ref["scores"],
                                 ref["group_scores"], E, G, TG, k)
    out_ref = ref["out"]
    if exempt.any():
        inj, _, _ = oracle.forward_with_routing(xb, ids, w, wgb, wub, wdb, scale)
        out_ref[exempt] = inj[exempt]
    err, _ = out_error(out, out_ref)
    print(f"    exempt={st['exempt']} out_err/rms={err:.2e}", flush=True)
    assert err <= OUT_TOL
    np.testing.assert_array_equal(out16, oracle.f32_to_bf16(out))
