"""Host-side logic of bench.py, on the CPU: the algorithmic work it divides by
(closed forms of the method's FLOPs and bytes), the roofline choice, the
one-GPU guard and the layout of the stored HBM-traffic figures."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from group_limited_routing_router_amd.inputs import CONFIGS  # noqa: E402


def test_layer_work_closed_forms():
    # per token: the router 2*H*E and k experts of three [I, H] matrices,
    # 2 FLOPs per multiply-add: 2.62 + 8 * 78.64 = 631.8 MFLOP at Beam sizes
    c = CONFIGS["prefill"]
    counts, layer = bench.work_counts(c, n_hit=256)
    assert layer["flops"] == c.T * (2 * c.H * c.E + c.k * 6 * c.H * c.I)
    assert abs(layer["flops"] / c.T / 1e6 - 631.8) < 0.1
    # each hit expert streams its three bf16 matrices once (78.64 MB), plus
    # the router weight, x in bf16 and the fp32 output
    per_expert = 3 * c.I * c.H * 2
    assert abs(per_expert / 1e6 - 78.64) < 0.01
    assert layer["bytes"] == 256 * per_expert + c.E * c.H * 2 + c.T * c.H * 2 + c.T * c.H * 4
    # the steps add up to the layer's FLOPs (the combine's 2*k*H per token is
    # not part of the method's matrix work)
    steps = counts["route"]["flops"] + counts["gate_up"]["flops"] + counts["down"]["flops"]
    assert steps == layer["flops"]
    # fewer experts hit, fewer weight bytes (decode: about 252 of 256)
    _, dec = bench.work_counts(CONFIGS["decode"], n_hit=252)
    _, dec_all = bench.work_counts(CONFIGS["decode"], n_hit=256)
    assert dec_all["bytes"] - dec["bytes"] == 4 * per_expert


def test_roofline_bound_choice():
    c = CONFIGS["prefill"]
    counts, layer = bench.work_counts(c, n_hit=256)
    res = dict(cfg=c, counts=counts, kernel_ms={"gate_up": 3.0, "route": 0.1})
    # prefill gate_up: 13.8 GB at 8 TB/s (1.73 ms) outweighs 3.4 TFLOP at
    # 2.5 PFLOP/s (1.37 ms), so its roofline is the HBM one
    r = bench.roofline_for(res, "gate_up")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["achieved"] - counts["gate_up"]["bytes"] / 3e-3 / 1e9) < 0.1
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-4
    # at the long workload the same kernel is MFMA-bound
    cl = CONFIGS["long"]
    cnt_l, _ = bench.work_counts(cl, n_hit=256)
    rl = bench.roofline_for(dict(cfg=cl, counts=cnt_l, kernel_ms={"gate_up": 20.0}), "gate_up")
    assert rl["bound"] == "mfma" and rl["unit"] == "TFLOP/s"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_stored_traffic_layout():
    with open(bench.TRAFFIC_FILE) as f:
        tr = json.load(f)
    assert len(tr["kernel_source_sha"]) == 16
    assert 1.5 < tr["fetch_factor"] < 2.5 and 0.5 < tr["write_factor"] < 1.5
    for wl in ("prefill", "decode"):
        for k in ("route", "gate_up", "down", "combine"):
            e = tr[wl][k]
            assert e["fetch_bytes"] >= 0 and e["write_bytes"] >= 0
    # the measured prefill gate_up reads at least its algorithmic weight bytes
    c = CONFIGS["prefill"]
    assert tr["prefill"]["gate_up"]["fetch_bytes"] >= 256 * 2 * c.I * c.H * 2


def test_kernel_source_sha_is_stable():
    assert bench.kernel_source_sha() == bench.kernel_source_sha()
    assert all(p.endswith((".hip", ".h")) for p in bench.KERNEL_SOURCES)


def test_kernel_names_and_steps():
    n = ("void moe::(anonymous namespace)::ffn_gemm_dma_kernel<true, false>"
         "(moe::(anonymous namespace)::FfnArgs)")
    assert bench.short_kernel_name(n) == "ffn_gemm_dma_kernel<true, false>"
    assert bench.step_of("ffn_gemm_dma_kernel<true, false>") == "gate_up"
    assert bench.step_of("ffn_gemm_dma_kernel<false, true>") == "fp8_down"
    assert bench.step_of("ffn_gemm_kernel<16, 128, 1, 4, true, false, 128>") == "gate_up"
    assert bench.step_of("route_small_kernel<8, 1, 10>") == "route"
    assert bench.step_of("permute_scatter_kernel") == "permute"
    assert bench.step_of("combine_residual_kernel<8, 8>") == "combine_residual"
    assert bench.step_of("combine_kernel<8, false>") == "combine"


def _write_csv(path, header, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_and_counter_summaries(tmp_path, capsys):
    gu = "void moe::(anonymous namespace)::ffn_gemm_dma_kernel<true, false>(FfnArgs)"
    cp = "__amd_rocclr_copyBuffer"
    # kernel trace: 3 launches of gate_up (1000, 2000, 3000 us), skip the first
    hdr = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"]
    rows = [["KERNEL_DISPATCH", i + 1, gu, 10 ** 9 * i, 10 ** 9 * i + 10 ** 6 * (i + 1), 2621440]
            for i in range(3)]
    _write_csv(str(tmp_path / "tr" / "host" / "1" / "t_kernel_trace.csv"), hdr, rows)
    bench.summarize_trace(str(tmp_path / "tr"), skip=1)
    out = capsys.readouterr().out
    line = [ln for ln in out.splitlines() if "ffn_gemm_dma_kernel" in ln][0].split()
    assert line[0] == "gate_up" and line[-5] == "2" and float(line[-4]) == 2500.0
    # counters: the copy reads half its bytes in FETCH_SIZE units (factor 2)
    hdr = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    f_rows = [[1, cp, 1024, "FETCH_SIZE", 524288], [2, gu, 2621440, "FETCH_SIZE", 1000],
              [3, gu, 2621440, "FETCH_SIZE", 3000]]
    w_rows = [[1, cp, 1024, "WRITE_SIZE", 1048576], [2, gu, 2621440, "WRITE_SIZE", 10],
              [3, gu, 2621440, "WRITE_SIZE", 30]]
    _write_csv(str(tmp_path / "f" / "x_counter_collection.csv"), hdr, f_rows)
    _write_csv(str(tmp_path / "w" / "x_counter_collection.csv"), hdr, w_rows)
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), skip=1)
    out = capsys.readouterr().out
    line = [ln for ln in out.splitlines() if "ffn_gemm_dma_kernel" in ln][0].split()
    # 3000 KiB x 2 -> 6.144 MB read; 30 KiB x 1 -> 0.031 MB written
    assert abs(float(line[-2]) - 3000 * 2 * 1024 / 1e9) < 1e-3
    assert "x 2.000 x 1024" in out


def test_kernel_source_sha_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("// a comment\\nint f() { return 1; } /* block */\\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["k.hip"])
    a = bench.kernel_source_sha()
    src.write_text("// another comment\\nint f()  {\\n return 1; }\\n")
    assert bench.kernel_source_sha() == a
    src.write_text("int f() { return 2; }\\n")
    assert bench.kernel_source_sha() != a


def test_power_sampler_parse_and_window():
    text = ("GPU: 0\n    POWER:\n        SOCKET_POWER: 1396 W\n        GFX_VOLTAGE: N/A\n"
            "    CLOCK:\n        GFX_0:\n            CLK: 1600 MHz\n            MIN_CLK: 231 MHz\n"
            "        GFX_1:\n            CLK: 1620 MHz\n            MAX_CLK: 2400 MHz\n"
            "    TEMPERATURE:\n        EDGE: N/A\n        HOTSPOT: 55 °C\n        MEM: 40 °C\n")
    smp = bench._PowerSampler.parse(text)
    assert smp == {"power_w": 1396, "gfx_mhz": 1610.0, "hotspot_c": 55}
    assert bench._PowerSampler.parse("amd-smi: no devices") == {
        "power_w": None, "gfx_mhz": None, "hotspot_c": None}
    s = bench._PowerSampler()
    s.samples = [(1.0, smp), (2.0, dict(smp, power_w=1400, gfx_mhz=1590.0)),
                 (5.0, dict(smp, power_w=300))]
    w = s.window(0.5, 2.5)
    assert w["samples"] == 2 and w["power_w"] == 1398 and w["power_w_max"] == 1400
    assert w["gfx_mhz"] == 1600 and w["gfx_mhz_min"] == 1590 and w["hotspot_c_max"] == 55
    assert s.window(10, 11)["power_w"] is None


def test_ceiling_at_intensity_picks_the_point_below():
    peaks = {"mfma_with_hbm_stream": [
        {"loads_per_step": 0, "bytes_per_kflop": 0.0, "tflops": 1800.0},
        {"loads_per_step": 1, "bytes_per_kflop": 1.953, "tflops": 1500.0},
        {"loads_per_step": 2, "bytes_per_kflop": 3.906, "tflops": 1300.0},
        {"loads_per_step": 4, "bytes_per_kflop": 7.812, "tflops": 750.0}]}
    # 4.03 bytes per kFLOP (prefill gate/up): the 3.906 point, 1300 TFLOP/s
    roof = {"algorithmic_bytes": 4.03e9, "algorithmic_flops": 1e12, "ms": 1.0}
    bench.at_intensity(roof, peaks)
    assert roof["achievable_at_bytes_per_kflop"] == 3.906
    assert roof["achievable_mfma_tflops_at_intensity"] == 1300.0
    assert abs(roof["mfma_frac_of_achievable_at_intensity"] - 1000.0 / 1300.0) < 1e-4
    # an HBM-bound kernel past the largest measured intensity gets nothing
    roof = {"algorithmic_bytes": 250e9, "algorithmic_flops": 1e12, "ms": 1.0}
    bench.at_intensity(roof, peaks)
    assert "achievable_mfma_tflops_at_intensity" not in roof
