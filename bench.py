#!/usr/bin/env python3
"""Benchmark of one Beam-shaped MoE block forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill]

A step is one moe_forward call (router, group-limited top-k, permutation,
gate/up + SwiGLU GEMM, down GEMM, weighted combine) over T tokens that are
already resident in HBM.  The default workload is the prefill chunk: T=8192
tokens, hidden 5120, 256 experts in 8 groups (4 kept), k=8, intermediate
2560, bf16 weights and activations with fp32 accumulation; the decode batch
(T=128) is timed as well because its HBM-bandwidth fraction is the other half
of the headline metric.  Inputs are seeded synthetic Gaussians (no trained
weights exist here).

Prints one JSON line.  `value` is tokens/s of the timed workload; `roofline`
describes the dominant kernel (timed with HIP events on the stream the
library launches on); `cpu_baseline` is the CPU oracle timed on a bounded
sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5166e15   # dense bf16 MFMA, FLOP/s (MI355X published)
PEAK_HBM = 8.0e12       # HBM3E, B/s (MI355X published)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = sorted(
    os.path.join("group_limited_routing_router_amd", "csrc", f)
    for f in os.listdir(os.path.join(ROOT, "group_limited_routing_router_amd", "csrc"))
    if f.endswith((".hip", ".h")))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def work_counts(cfg, n_hit):
    """Algorithmic FLOPs and HBM bytes of each step (what the method must do:
    no padding, no intermediate round trips) -- see the design doc."""
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    P = T * k
    w_expert = 3 * I * H * 2  # bytes of one expert's three bf16 matrices
    c = {
        "route": dict(flops=2 * T * H * E, bytes=T * H * 2 + E * H * 2 + P * 8),
        "permute": dict(flops=0, bytes=P * 4 + (E + 1) * 4 + 2 * P * 4),
        "gate_up": dict(flops=4 * P * H * I, bytes=n_hit * 2 * I * H * 2 + T * H * 2 + P * I * 2),
        "down": dict(flops=2 * P * I * H, bytes=n_hit * I * H * 2 + P * I * 2 + P * H * 4),
        "combine": dict(flops=2 * P * H, bytes=P * H * 4 + P * 8 + T * H * 4),
        # combine fused with the post-norm and residual update: the stream is
        # read and written, the combined output never leaves the chip
        "combine_residual": dict(flops=2 * P * H + 6 * T * H,
                                 bytes=P * H * 4 + P * 8 + 2 * T * H * 4 + H * 4),
    }
    layer = dict(flops=2 * T * H * E + 6 * P * H * I,
                 bytes=n_hit * w_expert + E * H * 2 + T * H * 2 + T * H * 4)
    return c, layer


def run_workload(name, steps, warmup, weights, want_kernels=True):
    import torch

    from group_limited_routing_router_amd import moe
    from group_limited_routing_router_amd.inputs import CONFIGS, make_tokens

    cfg = CONFIGS[name]
    d = make_tokens(cfg, seed=0, device="cuda")
    d.update(weights)
    p = moe.MoEProblem.from_config(cfg)
    b = moe.alloc_buffers(p)

    def step():
        moe.moe_forward(p, d["x"], d["w_router"], d["bias"], d["w_gate"], d["w_up"], d["w_down"],
                        b["out"], b["topk_ids"], b["topk_weights"], b["y"], b["ws"])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / steps

    ids = b["topk_ids"]
    n_hit = int((torch.bincount(ids.flatten().long(), minlength=cfg.E) > 0).sum())
    counts, layer = work_counts(cfg, n_hit)
    res = dict(cfg=cfg, ms=ms, n_hit=n_hit, counts=counts, layer=layer, buffers=b, inputs=d)

    if want_kernels:
        # the same steps as separate calls, each bracketed by events on the
        # current stream (the stream the library launches on)
        names = ["route", "permute", "gate_up", "down", "combine", "combine_residual"]
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
              for _ in range(steps)]
        gain = torch.ones(cfg.H, dtype=torch.float32, device="cuda")
        stream_res = torch.zeros((cfg.T, cfg.H), dtype=torch.float32, device="cuda")
        for it in range(warmup + steps):
            e = ev[it - warmup] if it >= warmup else None
            if e: e[0].record()
            moe.moe_route(p, d["x"], d["w_router"], d["bias"], b["topk_ids"], b["topk_weights"])
            if e: e[1].record()
            moe.moe_permute(p, b["topk_ids"], b["expert_offsets"], b["sorted_pairs"],
                            b["pair_rows"], b["ws"])
            if e: e[2].record()
            moe.moe_expert_gate_up(p, d["x"], b["sorted_pairs"], b["expert_offsets"],
                                   d["w_gate"], d["w_up"], b["h"])
            if e: e[3].record()
            moe.moe_expert_down(p, b["h"], b["expert_offsets"], d["w_down"], b["y"])
            if e: e[4].record()
            moe.moe_combine(p, b["y"], b["pair_rows"], b["topk_weights"], b["out"])
            if e: e[5].record()
            moe.moe_combine_residual(p, b["y"], b["pair_rows"], b["topk_weights"], gain, 1e-6, 2,
                                     stream_res)
            if e: e[6].record()
        torch.cuda.synchronize()
        kt = {}
        for j, nm in enumerate(names):
            kt[nm] = sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)) / steps
        res["kernel_ms"] = kt
    return res


def run_fp8(name, steps, warmup, weights_fp8):
    """The block with FP8 expert weights (moe_forward_fp8) on a workload, timed
    with events on the current stream; algorithmic bytes count one byte per
    weight plus the per-channel scales."""
    import torch

    from group_limited_routing_router_amd import moe
    from group_limited_routing_router_amd.inputs import CONFIGS, make_tokens

    cfg = CONFIGS[name]
    d = make_tokens(cfg, seed=0, device="cuda")
    w = weights_fp8
    p = moe.MoEProblem.from_config(cfg)
    b = moe.alloc_buffers(p)

    def step():
        moe.moe_forward_fp8(p, d["x"], w["w_router"], d["bias"], w["q_gate"], w["s_gate"],
                            w["q_up"], w["s_up"], w["q_down"], w["s_down"], b["out"],
                            b["topk_ids"], b["topk_weights"], b["y"], b["ws"])

    for _ in range(warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    n_hit = int((torch.bincount(b["topk_ids"].flatten().long(), minlength=cfg.E) > 0).sum())
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    flops = 2 * T * H * E + 6 * T * k * H * I
    bytes_ = n_hit * (3 * I * H + (2 * I + H) * 4) + E * H * 2 + T * H * 2 + T * H * 4
    return {"tokens": T, "ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "experts_hit": n_hit, "hbm_gbs": round(bytes_ / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(bytes_ / (ms * 1e-3) / PEAK_HBM, 4),
            "mfma_frac": round(flops / (ms * 1e-3) / PEAK_BF16, 4)}


def run_dense(steps, warmup):
    """The dense SwiGLU MLP (moe_dense_mlp) on its synthetic workload, timed
    with events on the current stream."""
    import torch

    from group_limited_routing_router_amd import moe
    from group_limited_routing_router_amd.inputs import CONFIGS, make_inputs

    cfg = CONFIGS["dense"]
    d = make_inputs(cfg, seed=0, device="cuda")
    p = moe.MoEProblem.from_config(cfg)
    ws = torch.empty(moe.moe_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda")

    def step():
        moe.moe_dense_mlp(p, d["x"], d["w_gate"], d["w_up"], d["w_down"], out, ws)

    for _ in range(warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 6 * cfg.T * cfg.H * cfg.I
    bytes_ = 3 * cfg.I * cfg.H * 2 + cfg.T * cfg.H * 2 + cfg.T * cfg.H * 4
    del d, ws, out
    return {"tokens": cfg.T, "hidden": cfg.H, "intermediate": cfg.I, "ms_per_step": round(ms, 4),
            "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "roofline": {"bound": "mfma", "achieved": round(flops / (ms * 1e-3) / 1e12, 1),
                         "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                         "frac": round(flops / (ms * 1e-3) / PEAK_BF16, 4), "traffic": None,
                         "algorithmic_bytes": bytes_, "algorithmic_flops": flops}}


def gemm_study(weights, steps, warmup):
    """Where the time of the prefill expert GEMMs goes: gate_up and down of
    the prefill workload (T=8192) with the routed row counts and with
    hand-made expert_offsets giving every expert the same R rows (R <= 256,
    one row tile per expert and column tile), next to the library's batched
    GEMM (torch.bmm, hipBLASLt) on the uniform 256-row shapes.  Events on the
    current stream; prints one JSON line."""
    import torch

    from group_limited_routing_router_amd import moe
    from group_limited_routing_router_amd.inputs import CONFIGS, make_tokens

    cfg = CONFIGS["prefill"]
    d = make_tokens(cfg, seed=0, device="cuda")
    d.update(weights)
    p = moe.MoEProblem.from_config(cfg)
    b = moe.alloc_buffers(p)
    moe.moe_route(p, d["x"], d["w_router"], d["bias"], b["topk_ids"], b["topk_weights"])
    moe.moe_permute(p, b["topk_ids"], b["expert_offsets"], b["sorted_pairs"], b["pair_rows"],
                    b["ws"])
    routed = b["expert_offsets"].clone()

    def timed(fn):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    H, I, E = cfg.H, cfg.I, cfg.E
    rows = {}
    for name in ["routed", 32, 64, 128, 192, 256]:
        if name == "routed":
            b["expert_offsets"].copy_(routed)
        else:  # every expert takes R of the sorted pairs (each a valid token)
            b["expert_offsets"].copy_(torch.arange(E + 1, dtype=torch.int32, device="cuda") * name)
        n = int(b["expert_offsets"][-1])
        gu = timed(lambda: moe.moe_expert_gate_up(p, d["x"], b["sorted_pairs"], b["expert_offsets"],
                                                  d["w_gate"], d["w_up"], b["h"]))
        dn = timed(lambda: moe.moe_expert_down(p, b["h"], b["expert_offsets"], d["w_down"], b["y"]))
        rows[str(name)] = {"pairs": n, "gate_up_ms": round(gu, 4), "down_ms": round(dn, 4),
                           "gate_up_mfma_frac": round(4 * n * H * I / (gu * 1e-3) / PEAK_BF16, 4),
                           "down_mfma_frac": round(2 * n * H * I / (dn * 1e-3) / PEAK_BF16, 4)}
        log("[study] rows %s: %s" % (name, rows[str(name)]))
    b["expert_offsets"].copy_(routed)
    del b, d
    torch.cuda.empty_cache()
    # the library on the same uniform shapes: [E, 256, H] x [E, H, 2I] (gate
    # and up side by side) and [E, 256, I] x [E, I, H], bf16 out, contiguous
    M = 256
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.empty(E, M, H, dtype=torch.bfloat16, device="cuda").normal_(generator=g)
    w = torch.empty(E, H, 2 * I, dtype=torch.bfloat16, device="cuda").normal_(0, 0.02, generator=g)
    o = torch.empty(E, M, 2 * I, dtype=torch.bfloat16, device="cuda")
    t_gu = timed(lambda: torch.bmm(a, w, out=o))
    del a, w, o
    a = torch.empty(E, M, I, dtype=torch.bfloat16, device="cuda").normal_(generator=g)
    w = torch.empty(E, I, H, dtype=torch.bfloat16, device="cuda").normal_(0, 0.02, generator=g)
    o = torch.empty(E, M, H, dtype=torch.bfloat16, device="cuda")
    t_dn = timed(lambda: torch.bmm(a, w, out=o))
    del a, w, o
    torch.cuda.empty_cache()
    n = E * M
    lib = {"gate_up_ms": round(t_gu, 4), "down_ms": round(t_dn, 4),
           "gate_up_mfma_frac": round(4 * n * H * I / (t_gu * 1e-3) / PEAK_BF16, 4),
           "down_mfma_frac": round(2 * n * H * I / (t_dn * 1e-3) / PEAK_BF16, 4),
           "note": "torch.bmm bf16 out, contiguous operands, no gather, no SwiGLU"}
    log("[study] library bmm, 256 rows per expert: %s" % lib)
    print(json.dumps({"study": "prefill expert GEMMs by rows per expert",
                      "workload": "beam-moe-prefill", "steps": steps, "warmup": warmup,
                      "rows_per_expert": rows, "library_bmm_256_rows": lib}), flush=True)


def roofline_for(res, kernel):
    c = res["counts"][kernel]
    ms = res["kernel_ms"][kernel]
    t_mfma = c["flops"] / PEAK_BF16
    t_hbm = c["bytes"] / PEAK_HBM
    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        ent = tr.get(res["cfg"].name, {}).get(kernel)
        if ent and tr.get("kernel_source_sha") == kernel_source_sha():
            traffic = int(ent["fetch_bytes"] + ent["write_bytes"])
    except (OSError, ValueError, KeyError):
        traffic = None
    if t_hbm >= t_mfma:
        ach = c["bytes"] / (ms * 1e-3) / 1e9
        r = dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM / 1e9, unit="GB/s",
                 frac=round(ach / (PEAK_HBM / 1e9), 4), traffic=traffic)
    else:
        ach = c["flops"] / (ms * 1e-3) / 1e12
        r = dict(bound="mfma", achieved=round(ach, 1), peak=PEAK_BF16 / 1e12, unit="TFLOP/s",
                 frac=round(ach / (PEAK_BF16 / 1e12), 4), traffic=traffic)
    r["kernel"] = kernel
    r["ms"] = round(ms, 4)
    r["algorithmic_bytes"] = c["bytes"]
    r["algorithmic_flops"] = c["flops"]
    r["mfma_frac"] = round(c["flops"] / (ms * 1e-3) / PEAK_BF16, 4)
    r["hbm_frac"] = round(c["bytes"] / (ms * 1e-3) / PEAK_HBM, 4)
    return r


def cpu_baseline(res, target_s):
    """The oracle, as it stands, on a bounded sample of the timed workload's
    tokens (routing + expert FFN + combine for the first n tokens)."""
    import numpy as np
    import torch

    if "OMP_NUM_THREADS" not in os.environ:
        os.environ["OMP_NUM_THREADS"] = str(len(os.sched_getaffinity(0)))
    os.environ.setdefault("OMP_PROC_BIND", "close")
    import oracle
    from group_limited_routing_router_amd.inputs import bits

    threads = oracle.num_threads()

    cfg, d = res["cfg"], res["inputs"]
    wr = bits(d["w_router"])
    bias = d["bias"].cpu().numpy()

    def run(n):
        xs = bits(d["x"][:n])
        t0 = time.perf_counter()
        ids, w, _, _ = oracle.route(xs, wr, bias, cfg.G, cfg.TG, cfg.k)
        t_route = time.perf_counter() - t0
        used = np.unique(ids)
        sel = torch.from_numpy(used).cuda()
        wg = bits(d["w_gate"].index_select(0, sel))       # host copies: not timed
        wu = bits(d["w_up"].index_select(0, sel))
        wd = bits(d["w_down"].index_select(0, sel))
        remap = np.full(cfg.E, -1, np.int32)
        remap[used] = np.arange(len(used), dtype=np.int32)
        t1 = time.perf_counter()
        oracle.forward_with_routing(xs, remap[ids], w, wg, wu, wd, cfg.scale)
        t_ffn = time.perf_counter() - t1
        return t_route + t_ffn

    # calibrate on enough tokens to keep every thread busy (a handful of
    # tokens gives too few pairs and overstates the per-token time)
    n0 = max(16, threads // 4)
    t0 = run(n0)
    n = int(max(4, min(cfg.T, round(target_s / max(t0 / n0, 1e-6)))))
    t = run(n)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return dict(value=round(n / t, 2), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"first {n} of the {cfg.T} tokens of the {cfg.name} workload: "
                       f"routing, expert FFN and combine ({t:.1f} s)",
                cpu_model=model)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill",
                    choices=["prefill", "decode", "skew", "long"])
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the secondary decode (T=128) measurement")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the secondary FP8-weight measurements")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the secondary dense-MLP measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM counters)")
    ap.add_argument("--gemm-study", action="store_true",
                    help="instead of the benchmark: the prefill expert GEMMs at fixed rows per "
                         "expert next to the library batched GEMM (one JSON line)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    from group_limited_routing_router_amd import moe
    from group_limited_routing_router_amd.inputs import CONFIGS, make_weights

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    moe.load_library()
    weights = make_weights(CONFIGS["decode"], seed=0, device="cuda")
    torch.cuda.synchronize()
    if args.gemm_study:
        gemm_study(weights, args.steps, args.warmup)
        return

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        bb = torch.empty_like(a)
        for _ in range(3):
            bb.copy_(a)
        torch.cuda.synchronize()
        del a, bb

    main_res = run_workload(args.workload, args.steps, args.warmup, weights)
    cfg = main_res["cfg"]
    kms = main_res["kernel_ms"]
    log("[bench] %s T=%d: %.3f ms/step; kernels %s" % (
        cfg.name, cfg.T, main_res["ms"], {k: round(v, 4) for k, v in kms.items()}))
    dominant = max((k for k in kms if k != "combine_residual"), key=kms.get)
    layer = main_res["layer"]
    ms = main_res["ms"]
    out = {
        "metric": "MoE-layer tokens/s + % bf16 MFMA peak (T=8192); % HBM peak BW (T=128)",
        "value": round(cfg.T * args.steps / (ms * 1e-3 * args.steps), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"beam-moe-{cfg.name}", "tokens": cfg.T, "hidden": cfg.H,
                   "intermediate": cfg.I, "experts": cfg.E, "groups": cfg.G,
                   "kept_groups": cfg.TG, "top_k": cfg.k, "scale": cfg.scale,
                   "experts_hit": main_res["n_hit"]},
        "layer": {"tflops": round(layer["flops"] / (ms * 1e-3) / 1e12, 1),
                  "mfma_frac": round(layer["flops"] / (ms * 1e-3) / PEAK_BF16, 4),
                  "hbm_gbs": round(layer["bytes"] / (ms * 1e-3) / 1e9, 1),
                  "hbm_frac": round(layer["bytes"] / (ms * 1e-3) / PEAK_HBM, 4)},
        "kernels_ms": {k: round(v, 4) for k, v in kms.items() if k != "combine_residual"},
        "roofline": roofline_for(main_res, dominant),
        # the combine fused with the post-norm and residual update (not part of
        # the timed step: a separate entry point after the block)
        "combine_residual": roofline_for(main_res, "combine_residual"),
    }
    if not args.no_decode and args.workload != "decode":
        dec = run_workload("decode", args.steps, args.warmup, weights)
        dl = dec["layer"]
        out["decode"] = {
            "tokens": dec["cfg"].T, "ms_per_step": round(dec["ms"], 4),
            "tokens_per_s": round(dec["cfg"].T / (dec["ms"] * 1e-3), 1),
            "experts_hit": dec["n_hit"],
            "hbm_gbs": round(dl["bytes"] / (dec["ms"] * 1e-3) / 1e9, 1),
            "hbm_frac": round(dl["bytes"] / (dec["ms"] * 1e-3) / PEAK_HBM, 4),
            "kernels_ms": {k: round(v, 4) for k, v in dec["kernel_ms"].items()
                           if k != "combine_residual"},
            "roofline": roofline_for(dec, max((k for k in dec["kernel_ms"] if k != "combine_residual"),
                                              key=dec["kernel_ms"].get)),
        }
        log("[bench] decode T=128: %.3f ms/step, %.1f%% of HBM peak" % (
            dec["ms"], 100 * out["decode"]["hbm_frac"]))
        del dec
    if not args.no_fp8:
        from group_limited_routing_router_amd.inputs import make_weights_fp8
        w8 = make_weights_fp8(CONFIGS["decode"], seed=0, device="cuda")
        out["fp8_weights"] = {n: run_fp8(n, args.steps, args.warmup, w8)
                              for n in ("decode", args.workload)}
        log("[bench] fp8 weights: %s" % {n: (v["ms_per_step"], v["hbm_frac"])
                                          for n, v in out["fp8_weights"].items()})
        del w8
        torch.cuda.empty_cache()
    if not args.no_dense:
        out["dense_mlp"] = run_dense(args.steps, args.warmup)
        log("[bench] dense MLP T=%d I=%d: %.3f ms/step, %.1f%% of bf16 MFMA peak" % (
            out["dense_mlp"]["tokens"], out["dense_mlp"]["intermediate"],
            out["dense_mlp"]["ms_per_step"], 100 * out["dense_mlp"]["roofline"]["frac"]))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(main_res, args.cpu_seconds)
        log("[bench] cpu oracle: %s" % out["cpu_baseline"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
