#!/usr/bin/env python3
"""Benchmark of one Beam-shaped MoE block forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill]

A step is one moe_forward call (router, group-limited top-k, permutation,
gate/up + SwiGLU GEMM, down GEMM, weighted combine) over T tokens that are
already resident in HBM.  The default workload is the prefill chunk: T=8192
tokens, hidden 5120, 256 experts in 8 groups (4 kept), k=8, intermediate
2560, bf16 weights and activations with fp32 accumulation.  The decode batch
(T=128, the HBM half of the headline metric), the skewed (T=4096) and long
(T=65536) workloads are timed the same way and reported as secondary objects,
with the FP8-weight layer and the dense MLP; the prefill and decode forward
is also timed as a replayed HIP graph (`graph_replay`).  Inputs are seeded
synthetic Gaussians (no trained weights exist here).

Prints one JSON line.  `value` is tokens/s of the timed workload (mean wall
time of exactly --steps calls between two device synchronisations; the
median and minimum per-step event times are reported beside it); `roofline`
describes the dominant kernel (timed with HIP events on the stream the
library launches on); `achievable_*` are this GPU's measured streaming-read
bandwidth and sustained back-to-back MFMA rate on pseudo-random operands
(the measurement kernels of include/moe_peak.h), and `roofline` adds the
MFMA rate those kernels reach beside an HBM stream of the kernel's own bytes
per FLOP; `cpu_baseline` is the CPU oracle timed on this host's cores (every
decode token, samples of prefill and skew, long extrapolated).

Other modes (one JSON line or a text table each):
  --kernels-only       only the timed workload's separate calls (the kernel
                       trace of such a run holds nothing else)
  --gemm-study         the prefill expert GEMMs at fixed rows per expert
  --power-study        board power and graphics clock (amd-smi samples) while
                       each kernel runs back to back
  --summarize-trace D  per-kernel durations from a rocprofv3 kernel trace
  --summarize-pmc D1 D2  HBM bytes per launch from FETCH_SIZE / WRITE_SIZE runs
  --summarize-counters D per-kernel averages of any counter run
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5166e15   # dense bf16 MFMA, FLOP/s (MI355X published)
PEAK_HBM = 8.0e12       # HBM3E, B/s (MI355X published)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the sources of the MoE block's kernels (the measurement kernels of peak.hip
# are not part of the block and do not invalidate its stored traffic)
KERNEL_SOURCES = sorted(
    os.path.join("group_limited_routing_router_amd", "csrc", f)
    for f in os.listdir(os.path.join(ROOT, "group_limited_routing_router_amd", "csrc"))
    if f.endswith((".hip", ".h")) and f != "peak.hip")
STEPS = ["route", "permute", "gate_up", "down", "combine", "combine_residual"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha():
    """Hash of the block's kernel sources with comments and blank space taken
    out, so that stored counter figures stay keyed to the code itself."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
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


def timed_steps(step, steps, warmup):
    """warmup untimed calls, then exactly `steps` calls bracketed by a device
    synchronisation on both sides (wall clock), with an event on the current
    stream between consecutive calls.  Returns (mean wall ms per step, the
    per-step event times in ms)."""
    import torch

    for _ in range(warmup):
        step()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / steps, [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def step_stats(step_ms):
    """Median and minimum of the per-step event times."""
    return {"ms_median": round(statistics.median(step_ms), 4), "ms_min": round(min(step_ms), 4)}


def run_workload(name, steps, warmup, weights, forward=True, kernels=True):
    """One workload on the bf16 weights: the timed forward (if `forward`) and
    each step as a separate entry-point call bracketed by events on the
    current stream (if `kernels`)."""
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

    res = dict(cfg=cfg, buffers=b, inputs=d)
    if forward:
        res["ms"], res["step_ms"] = timed_steps(step, steps, warmup)
    if kernels:
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STEPS) + 1)]
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
        res["kernel_ms"] = {nm: sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)) / steps
                            for j, nm in enumerate(STEPS)}
        del stream_res
    ids = b["topk_ids"]
    res["n_hit"] = int((torch.bincount(ids.flatten().long(), minlength=cfg.E) > 0).sum())
    res["counts"], res["layer"] = work_counts(cfg, res["n_hit"])
    if cfg.hot_groups:
        hot = torch.nonzero(d["bias"] > 0).flatten()
        res["hot_share"] = round(float(torch.isin(ids.flatten(), hot.to(ids.dtype)).float().mean()), 4)
    return res


def graph_replay_ms(res, steps, warmup):
    """The same moe_forward captured once into a HIP graph (the library's
    calls are capture-safe) and replayed: ms per replay, events on the
    current stream.  Shows what the per-call launch overhead costs."""
    import torch

    from group_limited_routing_router_amd import moe

    cfg, d, b = res["cfg"], res["inputs"], res["buffers"]
    p = moe.MoEProblem.from_config(cfg)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            moe.moe_forward(p, d["x"], d["w_router"], d["bias"], d["w_gate"], d["w_up"],
                            d["w_down"], b["out"], b["topk_ids"], b["topk_weights"], b["y"], b["ws"])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ms, step_ms = timed_steps(g.replay, steps, warmup)
    del g
    return {"ms_per_step": round(ms, 4), **step_stats(step_ms)}


def workload_summary(res, peaks=None):
    """The secondary object of a workload: times, rates, fractions of the
    published (and, if measured, the achievable) peaks, per-step times and
    the roofline of its dominant kernel."""
    cfg, ms, layer = res["cfg"], res["ms"], res["layer"]
    kms = res["kernel_ms"]
    dominant = max((k for k in kms if k != "combine_residual"), key=kms.get)
    out = {"tokens": cfg.T, "ms_per_step": round(ms, 4), **step_stats(res["step_ms"]),
           "tokens_per_s": round(cfg.T / (ms * 1e-3), 1), "experts_hit": res["n_hit"],
           "tflops": round(layer["flops"] / (ms * 1e-3) / 1e12, 1),
           "mfma_frac": round(layer["flops"] / (ms * 1e-3) / PEAK_BF16, 4),
           "hbm_gbs": round(layer["bytes"] / (ms * 1e-3) / 1e9, 1),
           "hbm_frac": round(layer["bytes"] / (ms * 1e-3) / PEAK_HBM, 4)}
    if peaks:
        out["mfma_frac_of_achievable"] = round(
            layer["flops"] / (ms * 1e-3) / 1e12 / peaks["achievable_mfma_tflops"], 4)
        out["hbm_frac_of_achievable"] = round(
            layer["bytes"] / (ms * 1e-3) / 1e9 / peaks["achievable_hbm_gbs"], 4)
    if "hot_share" in res:
        out["hot_expert_share"] = res["hot_share"]
    out["kernels_ms"] = {k: round(v, 4) for k, v in kms.items() if k != "combine_residual"}
    out["roofline"] = roofline_for(res, dominant)
    if peaks:
        at_intensity(out["roofline"], peaks)
    return out


def run_fp8(name, steps, warmup, weights_fp8):
    """The block with FP8 expert weights (moe_forward_fp8) on a workload;
    algorithmic bytes count one byte per weight plus the per-channel scales."""
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

    ms, step_ms = timed_steps(step, steps, warmup)
    n_hit = int((torch.bincount(b["topk_ids"].flatten().long(), minlength=cfg.E) > 0).sum())
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    flops = 2 * T * H * E + 6 * T * k * H * I
    bytes_ = n_hit * (3 * I * H + (2 * I + H) * 4) + E * H * 2 + T * H * 2 + T * H * 4
    del b, d
    torch.cuda.empty_cache()
    return {"tokens": T, "ms_per_step": round(ms, 4), **step_stats(step_ms),
            "tokens_per_s": round(T / (ms * 1e-3), 1),
            "experts_hit": n_hit, "hbm_gbs": round(bytes_ / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(bytes_ / (ms * 1e-3) / PEAK_HBM, 4),
            "mfma_frac": round(flops / (ms * 1e-3) / PEAK_BF16, 4)}


def run_dense(steps, warmup):
    """The dense SwiGLU MLP (moe_dense_mlp) on its synthetic workload."""
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

    ms, step_ms = timed_steps(step, steps, warmup)
    flops = 6 * cfg.T * cfg.H * cfg.I
    bytes_ = 3 * cfg.I * cfg.H * 2 + cfg.T * cfg.H * 2 + cfg.T * cfg.H * 4
    del d, ws, out
    torch.cuda.empty_cache()
    return {"tokens": cfg.T, "hidden": cfg.H, "intermediate": cfg.I, "ms_per_step": round(ms, 4),
            **step_stats(step_ms), "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "roofline": {"bound": "mfma", "achieved": round(flops / (ms * 1e-3) / 1e12, 1),
                         "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                         "frac": round(flops / (ms * 1e-3) / PEAK_BF16, 4), "traffic": None,
                         "ms": round(ms, 4), "algorithmic_bytes": bytes_,
                         "algorithmic_flops": flops}}


def achievable_peaks(repeats=5):
    """What this GPU sustains, measured with the library's measurement kernels
    (include/moe_peak.h): a streaming read of 8 GiB (far larger than the
    256 MB Infinity Cache) over several grid sizes, with and without the
    nontemporal cache policy, and back-to-back bf16 MFMAs on register operands
    over two grid sizes, on pseudo-random operands (the rate reported as
    achievable) and on one fixed operand pattern.  The reads are the best of
    `repeats` calls; the MFMA loops run for about a second each and report the
    mean of the second half, since the board power limit takes effect only
    after the first tens of milliseconds."""
    import torch

    from group_limited_routing_router_amd import moe

    nbytes = 8 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(0x5A)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def best_ms(fn):
        fn()
        times = []
        for _ in range(repeats):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return min(times)

    def sustained_ms(fn, n):
        for _ in range(n):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    reads = {}
    for nt in (False, True):
        for wg in (2048, 8192, 16384, 32768):
            ms = best_ms(lambda: moe.moe_peak_stream_read(buf, sink, wg, nontemporal=nt))
            reads[f"{'nt' if nt else 'cached'}_wg{wg}"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    # LDS-fed MFMAs with an HBM stream of 0, 1, 2 and 4 16-byte loads a lane
    # per 16 MFMAs (one workgroup per compute unit, four rounds); each call
    # reads at most the 8 GiB buffer once
    mixed = []
    wg_mix = 1024
    fsink = torch.empty(4 * wg_mix, dtype=torch.float32, device="cuda")
    for nl in (0, 1, 2, 4):
        steps = 1000 if nl == 0 else (nbytes // (wg_mix * 256 * 16) // nl - 8) // 8 * 8
        flops, nb = moe.moe_peak_mfma_stream(buf, nl, steps, fsink, wg_mix)
        ms = sustained_ms(lambda: moe.moe_peak_mfma_stream(buf, nl, steps, fsink, wg_mix),
                          max(4, int(round(500 / (flops / 1.5e15 * 1e3)))))
        mixed.append({"loads_per_step": nl, "bytes_per_kflop": round(nb / flops * 1e3, 3),
                      "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                      "gbs": round(nb / (ms * 1e-3) / 1e9, 1)})
    del buf, sink, fsink
    torch.cuda.empty_cache()
    mfma = {}
    iters = 20000
    for rnd in (True, False):
        for wg in (1024, 2048):
            out = torch.empty(4 * wg, dtype=torch.float32, device="cuda")
            flops = moe.moe_peak_mfma_bf16(iters, out, wg, random_operands=rnd)
            ms = sustained_ms(lambda: moe.moe_peak_mfma_bf16(iters, out, wg, random_operands=rnd),
                              max(4, int(round(500 / (flops / 2.0e15 * 1e3)))))
            mfma[f"{'random' if rnd else 'fixed'}_wg{wg}"] = round(flops / (ms * 1e-3) / 1e12, 1)
            del out
    hbm = max(reads.values())
    tf = max(v for k, v in mfma.items() if k.startswith("random"))
    tf_fixed = max(v for k, v in mfma.items() if k.startswith("fixed"))
    log("[bench] achievable: read %s GB/s, bf16 MFMA %s TFLOP/s, with a stream %s" % (
        reads, mfma, mixed))
    return {"achievable_hbm_gbs": hbm, "achievable_hbm_frac_of_peak": round(hbm * 1e9 / PEAK_HBM, 4),
            "achievable_mfma_tflops": tf,
            "achievable_mfma_frac_of_peak": round(tf * 1e12 / PEAK_BF16, 4),
            "mfma_fixed_operands_tflops": tf_fixed,
            "read_gbs_by_grid": reads, "mfma_tflops_by_grid": mfma,
            "mfma_with_hbm_stream": mixed,
            "how": "moe_peak_stream_read: one read of 8 GiB, 16-byte loads, 8 in flight per lane, "
                   f"256-thread workgroups, best of {repeats} event-timed calls per grid; "
                   "moe_peak_mfma_bf16: 8 independent 32x32x16 bf16 MFMA chains per wave on "
                   f"register operands, {iters} steps, 4 waves per workgroup, the mean of about "
                   "0.5 s of calls after 0.5 s of the same calls; achievable_mfma_tflops is the "
                   "rate on pseudo-random operands (bits change at every issue, as on real "
                   "data), mfma_fixed_operands_tflops the rate on one fixed pattern; "
                   "moe_peak_mfma_stream: per step and wave 8 LDS fragment reads of random "
                   "bf16 and their 16 MFMAs, with 0-4 nontemporal 16-byte loads a lane of an "
                   "8 GiB buffer, 1024 workgroups, timed like the MFMA loop"}


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


class _PowerSampler:
    """Samples the board's socket power, graphics clocks and temperatures with
    `amd-smi metric` (read-only) in a background thread, about four times a
    second, each sample stamped with the wall time."""

    def __init__(self):
        import shutil
        import threading
        self.samples, self.error = [], None
        self.exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def parse(text):
        pw = re.search(r"SOCKET_POWER:\s*(\d+)", text)
        clk = [int(v) for v in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)", text)]
        hot = re.search(r"HOTSPOT:\s*(\d+)", text)
        return dict(power_w=int(pw.group(1)) if pw else None,
                    gfx_mhz=sum(clk) / len(clk) if clk else None,
                    hotspot_c=int(hot.group(1)) if hot else None)

    def _run(self):
        import subprocess
        while not self._stop.is_set():
            t = time.time()
            try:
                r = subprocess.run([self.exe, "metric", "-g", "0", "-p", "-c", "-t"],
                                   capture_output=True, text=True, timeout=10)
                smp = self.parse(r.stdout)
                if smp["power_w"] is None and smp["gfx_mhz"] is None:
                    self.error = (r.stdout + r.stderr).strip()[-300:]
                else:
                    self.samples.append(((t + time.time()) / 2, smp))
            except (OSError, subprocess.SubprocessError) as e:
                self.error = repr(e)
                return
            self._stop.wait(0.25)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=15)

    def window(self, t0, t1):
        """Mean and extremes over the samples in [t0, t1]."""
        ss = [s for t, s in self.samples if t0 <= t <= t1]

        def col(key):
            return [s[key] for s in ss if s[key] is not None]
        pw, ck, hot = col("power_w"), col("gfx_mhz"), col("hotspot_c")
        return dict(samples=len(ss),
                    power_w=round(sum(pw) / len(pw)) if pw else None,
                    power_w_max=max(pw) if pw else None,
                    gfx_mhz=round(sum(ck) / len(ck)) if ck else None,
                    gfx_mhz_min=round(min(ck)) if ck else None,
                    hotspot_c_max=max(hot) if hot else None)


def power_study(weights, seconds):
    """Board power, graphics clock and rate of the block's kernels and of the
    measurement kernels, each run back to back for `seconds` while
    `amd-smi metric` samples the board (the first half second of a phase is
    left out of its averages).  Prints one line per phase and one JSON line."""
    import torch

    from group_limited_routing_router_amd import moe
    from group_limited_routing_router_amd.inputs import CONFIGS, make_tokens

    def setup(name):
        cfg = CONFIGS[name]
        d = make_tokens(cfg, seed=0, device="cuda")
        d.update(weights)
        p = moe.MoEProblem.from_config(cfg)
        b = moe.alloc_buffers(p)
        moe.moe_route(p, d["x"], d["w_router"], d["bias"], b["topk_ids"], b["topk_weights"])
        moe.moe_permute(p, b["topk_ids"], b["expert_offsets"], b["sorted_pairs"], b["pair_rows"],
                        b["ws"])
        n_hit = int((torch.bincount(b["topk_ids"].flatten().long(), minlength=cfg.E) > 0).sum())
        counts, layer = work_counts(cfg, n_hit)
        torch.cuda.synchronize()
        return cfg, p, d, b, counts, layer

    phases = []

    def phase(label, fn, flops=None, nbytes=None, what=""):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.time()
        e0.record()
        n = 0
        if fn is None:
            time.sleep(seconds)
        else:
            while time.time() - t0 < seconds:
                for _ in range(5):
                    fn()
                n += 5
                torch.cuda.synchronize()
        e1.record()
        torch.cuda.synchronize()
        t1 = time.time()
        ent = dict(phase=label, what=what, calls=n)
        if n:
            ms = e0.elapsed_time(e1) / n
            ent["ms_per_call"] = round(ms, 4)
            if flops:
                ent["tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
                ent["frac_bf16_peak"] = round(flops / (ms * 1e-3) / PEAK_BF16, 4)
            if nbytes:
                ent["gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        ent.update(sampler.window(t0 + 0.5, t1))
        phases.append(ent)
        log("[power] %-22s %s" % (label, {k: v for k, v in ent.items() if k not in ("phase", "what")}))

    with _PowerSampler() as sampler:
        phase("idle", None, what="no kernel")
        iters, wg = 20000, 2048
        sink = torch.empty(4 * wg, dtype=torch.float32, device="cuda")
        fl = moe.moe_peak_mfma_bf16(iters, sink, wg, random_operands=False)
        phase("mfma_fixed_operands", lambda: moe.moe_peak_mfma_bf16(iters, sink, wg, False),
              flops=fl, what="moe_peak_mfma_bf16, one fixed operand pattern")
        phase("mfma_random_operands", lambda: moe.moe_peak_mfma_bf16(iters, sink, wg, True),
              flops=fl, what="moe_peak_mfma_bf16, pseudo-random operands")
        buf = torch.empty(8 << 30, dtype=torch.uint8, device="cuda")
        buf.fill_(0x5A)
        s2 = torch.zeros(4, dtype=torch.int32, device="cuda")
        phase("stream_read_nt", lambda: moe.moe_peak_stream_read(buf, s2, 32768, nontemporal=True),
              nbytes=buf.numel(), what="moe_peak_stream_read, 8 GiB, nontemporal, 32768 workgroups")
        fsink = torch.empty(4 * 1024, dtype=torch.float32, device="cuda")
        for nl in (0, 1, 2, 4):
            steps = 1000 if nl == 0 else (buf.numel() // (1024 * 256 * 16) // nl - 8) // 8 * 8
            fl2, nb2 = moe.moe_peak_mfma_stream(buf, nl, steps, fsink, 1024)
            phase(f"mfma_lds_stream_{nl}", lambda: moe.moe_peak_mfma_stream(buf, nl, steps, fsink, 1024),
                  flops=fl2, nbytes=nb2 or None,
                  what=f"moe_peak_mfma_stream, {nl} loads a lane per 16 MFMAs "
                       f"({nb2 / fl2 * 1e3:.2f} bytes per kFLOP)")
        del buf, s2, sink, fsink
        torch.cuda.empty_cache()
        for name in ("decode", "prefill", "long"):
            cfg, p, d, b, counts, layer = setup(name)

            def gate_up():
                moe.moe_expert_gate_up(p, d["x"], b["sorted_pairs"], b["expert_offsets"],
                                       d["w_gate"], d["w_up"], b["h"])

            def down():
                moe.moe_expert_down(p, b["h"], b["expert_offsets"], d["w_down"], b["y"])

            def forward():
                moe.moe_forward(p, d["x"], d["w_router"], d["bias"], d["w_gate"], d["w_up"],
                                d["w_down"], b["out"], b["topk_ids"], b["topk_weights"], b["y"],
                                b["ws"])
            tag = f"{cfg.name} T={cfg.T}"
            phase(f"{cfg.name}_gate_up", gate_up, flops=counts["gate_up"]["flops"],
                  nbytes=counts["gate_up"]["bytes"], what=f"moe_expert_gate_up, {tag}")
            if name == "prefill":
                phase(f"{cfg.name}_down", down, flops=counts["down"]["flops"],
                      nbytes=counts["down"]["bytes"], what=f"moe_expert_down, {tag}")
            if name != "long":
                phase(f"{cfg.name}_forward", forward, flops=layer["flops"], nbytes=layer["bytes"],
                      what=f"moe_forward, {tag}")
            del b, d
            torch.cuda.empty_cache()
        phase("idle_after", None, what="no kernel")
    if sampler.error and not sampler.samples:
        log("[power] amd-smi gave no samples: %s" % sampler.error)
    print(json.dumps({"study": "board power and graphics clock by kernel",
                      "seconds_per_phase": seconds, "sampler": "amd-smi metric -g 0 -p -c -t",
                      "phases": phases}), flush=True)


def at_intensity(roof, peaks):
    """Add to a roofline object the rate moe_peak_mfma_stream reaches at the
    largest measured intensity not above the kernel's algorithmic bytes per
    thousand FLOPs (a ceiling at least as high as the one at the kernel's own
    intensity), and the kernel's fraction of it."""
    if not roof.get("algorithmic_flops"):
        return
    ai = roof["algorithmic_bytes"] / roof["algorithmic_flops"] * 1e3
    pts = [m for m in peaks.get("mfma_with_hbm_stream", []) if m["bytes_per_kflop"] <= ai]
    if not pts or ai > max(m["bytes_per_kflop"] for m in peaks["mfma_with_hbm_stream"]):
        return
    best = max(pts, key=lambda m: m["bytes_per_kflop"])
    tflops = roof["algorithmic_flops"] / (roof["ms"] * 1e-3) / 1e12
    roof["bytes_per_kflop"] = round(ai, 3)
    roof["achievable_mfma_tflops_at_intensity"] = best["tflops"]
    roof["achievable_at_bytes_per_kflop"] = best["bytes_per_kflop"]
    roof["mfma_frac_of_achievable_at_intensity"] = round(tflops / best["tflops"], 4)


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


def cpu_baseline(weights, main_name, target_s):
    """The oracle, as it stands, timed on this host's cores (the threads of
    the process affinity mask, OMP_PROC_BIND=close): routing, the expert FFN of
    every pair and the combine of the first n tokens of a workload.  Every
    decode token; the first tokens of prefill and skew, sized from the decode
    rate so the whole takes about target_s; long extrapolated from the prefill
    rate (the oracle's cost per token does not depend on the routing: k pairs
    per token).  The weights are copied to the host once, untimed."""
    import torch

    if "OMP_NUM_THREADS" not in os.environ:
        os.environ["OMP_NUM_THREADS"] = str(len(os.sched_getaffinity(0)))
    os.environ.setdefault("OMP_PROC_BIND", "close")
    import oracle
    from group_limited_routing_router_amd.inputs import CONFIGS, bits, make_tokens

    threads = oracle.num_threads()
    wh = {k: bits(v) for k, v in weights.items()}

    def run(cfg, n):
        d = make_tokens(cfg, seed=0, device="cuda")
        xs = bits(d["x"][:n])
        bias = d["bias"].cpu().numpy()
        del d
        torch.cuda.empty_cache()
        t0 = time.perf_counter()
        ids, w, _, _ = oracle.route(xs, wh["w_router"], bias, cfg.G, cfg.TG, cfg.k)
        oracle.forward_with_routing(xs, ids, w, wh["w_gate"], wh["w_up"], wh["w_down"], cfg.scale)
        return time.perf_counter() - t0

    def entry(cfg, n, t):
        flops = n * (2 * cfg.H * cfg.E + cfg.k * 6 * cfg.H * cfg.I)
        return {"tokens": n, "of_tokens": cfg.T, "seconds": round(t, 2),
                "tokens_per_s": round(n / t, 2), "gflops": round(flops / t / 1e9, 1),
                "full_workload_s": round(t * cfg.T / n, 1)}

    out = {}
    dec = CONFIGS["decode"]
    t = run(dec, dec.T)
    out["decode"] = entry(dec, dec.T, t)
    rate = dec.T / t
    for name, share in (("prefill", 0.6), ("skew", 0.25)):
        cfg = CONFIGS[name]
        n = int(max(64, min(cfg.T, round(rate * target_s * share))))
        out[name] = entry(cfg, n, run(cfg, n))
    lg, pre = CONFIGS["long"], out["prefill"]
    out["long"] = {"tokens": 0, "of_tokens": lg.T, "extrapolated": True,
                   "tokens_per_s": pre["tokens_per_s"], "gflops": pre["gflops"],
                   "full_workload_s": round(lg.T / pre["tokens_per_s"], 1),
                   "note": "not run: the prefill sample's rate applied to 65536 tokens"}
    del wh
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    main = out[main_name]
    return dict(value=main["tokens_per_s"], unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{main['tokens']} of the {main['of_tokens']} tokens of the {main_name} "
                       f"workload (routing, expert FFN, combine) in {main['seconds']} s"
                       if not main.get("extrapolated") else
                       f"the {main_name} rate extrapolated from the prefill sample",
                cpu_model=model, workloads=out)


# ---- rocprofv3 output summaries -----------------------------------------

def _csv_files(path, suffix):
    if os.path.isdir(path):
        files = sorted(glob.glob(os.path.join(path, "**", "*" + suffix), recursive=True))
    else:
        files = [path]
    if not files:
        raise SystemExit(f"no *{suffix} under {path}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            rows += list(csv.DictReader(f))
    return rows


def short_kernel_name(name):
    """'void moe::(anonymous namespace)::ffn_gemm_dma_kernel<true, false>(...)'
    -> 'ffn_gemm_dma_kernel<true, false>'."""
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):  # drop the parameter list
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not name[i:].startswith("(anonymous"):
            cut = i
            break
    name = name[:cut]
    name = re.sub(r"\(anonymous namespace\)::", "", name)
    name = re.sub(r"^(\w+::)+", "", name)
    return re.sub(r"\b(moe|std)::", "", name)


def step_of(kname):
    """The block's step a kernel belongs to (fp8_* for the FP8-weight GEMMs)."""
    if kname.startswith("route"):
        return "route"
    if kname.startswith("permute") or kname.startswith("identity_dispatch"):
        return "permute"
    if kname.startswith("combine_residual"):
        return "combine_residual"
    if kname.startswith("combine"):
        return "combine"
    if kname.startswith("ffn_gemm"):
        flags = re.findall(r"\b(true|false)\b", kname)
        gateup = flags[0] == "true"
        fp8 = len(flags) > 1 and flags[1] == "true"
        return ("fp8_" if fp8 else "") + ("gate_up" if gateup else "down")
    return "other"


def _grid(row):
    for k in ("Grid_Size", "Grid_Size_X"):
        if k in row and row[k]:
            return int(row[k])
    return 0


def summarize_trace(path, skip):
    """Per kernel: launches after the first `skip` of each kernel name,
    average / median / min / max duration in microseconds."""
    rows = _csv_files(path, "kernel_trace.csv")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    by = {}
    for r in rows:
        k = short_kernel_name(r["Kernel_Name"])
        by.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), _grid(r)))
    lines = [f"# skipped: the first {skip} launches of each kernel",
             "# step               kernel                                             grid  calls"
             "    avg_us    med_us    min_us    max_us"]
    for k, v in sorted(by.items(), key=lambda kv: STEPS.index(step_of(kv[0]).replace("fp8_", ""))
                       if step_of(kv[0]).replace("fp8_", "") in STEPS else 99):
        if step_of(k) == "other":  # torch's own kernels (input draws, copies)
            continue
        d = [x[0] / 1e3 for x in v[skip:]] or [x[0] / 1e3 for x in v]
        lines.append(f"  {step_of(k):<18} {k:<48} {v[0][1]:>9} {len(d):>6} {sum(d) / len(d):>9.1f} "
                     f"{statistics.median(d):>9.1f} {min(d):>9.1f} {max(d):>9.1f}")
    print("\n".join(lines))


def _per_dispatch(rows, counter):
    """{dispatch id: (short kernel name, grid, counter value summed over its
    rows)} for one counter of a rocprofv3 --pmc run, in dispatch order."""
    out = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        did = int(r["Dispatch_Id"])
        k = short_kernel_name(r["Kernel_Name"])
        prev = out.get(did, (k, _grid(r), 0.0))
        out[did] = (k, prev[1], prev[2] + float(r["Counter_Value"]))
    return dict(sorted(out.items()))


def summarize_pmc(fetch_path, write_path, skip, workload=None, update=False):
    """HBM bytes per launch from a FETCH_SIZE run and a WRITE_SIZE run (KiB per
    dispatch), each scaled by what the same counter reads for the plain 1 GiB
    device copy the runs make (--copy-calibration): bytes = FETCH_SIZE x
    (2^30 / 1024 / copy FETCH_SIZE) x 1024, the same for WRITE_SIZE.  Averaged
    per kernel over the launches after the first `skip`; with --update-traffic
    the per-step sums go to profiles/traffic.json under the workload's name,
    keyed to the hash of the kernel sources."""
    fd = _per_dispatch(_csv_files(fetch_path, "counter_collection.csv"), "FETCH_SIZE")
    wd = _per_dispatch(_csv_files(write_path, "counter_collection.csv"), "WRITE_SIZE")
    copy_f = [v for v in fd.values() if "copyBuffer" in v[0]]
    copy_w = [v for v in wd.values() if "copyBuffer" in v[0]]
    if not copy_f or not copy_w:
        raise SystemExit("no device copy in the runs: profile with --copy-calibration")
    cf, cw = max(c[2] for c in copy_f), max(c[2] for c in copy_w)
    ff, wf = (1 << 30) / 1024 / cf, (1 << 30) / 1024 / cw

    def per_kernel(d):
        by = {}
        for k, g, v in d.values():
            if "copyBuffer" in k or "fill" in k.lower() or k.startswith("at::"):
                continue
            by.setdefault(k, []).append((g, v))
        return {k: (v[0][0], [x[1] for x in v[skip:]] or [x[1] for x in v]) for k, v in by.items()}

    fk, wk = per_kernel(fd), per_kernel(wd)
    lines = [f"# calibration: the 1 GiB device copy reads FETCH_SIZE={cf:.0f} KiB and "
             f"WRITE_SIZE={cw:.0f} KiB;",
             f"#   HBM bytes = FETCH_SIZE x {ff:.3f} x 1024 + WRITE_SIZE x {wf:.3f} x 1024",
             f"# skipped: the first {skip} launches of each kernel",
             "# step               kernel                                             grid"
             "    FETCH_KiB  WRITE_KiB  read_GB write_GB"]
    steps = {}
    for k in sorted(fk, key=lambda n: STEPS.index(step_of(n).replace("fp8_", ""))
                    if step_of(n).replace("fp8_", "") in STEPS else 99):
        fv = sum(fk[k][1]) / len(fk[k][1])
        wv = sum(wk.get(k, (0, [0.0]))[1]) / max(1, len(wk.get(k, (0, [0.0]))[1]))
        rb, wb = fv * ff * 1024, wv * wf * 1024
        st = step_of(k)
        s = steps.setdefault(st, {"fetch_bytes": 0, "write_bytes": 0})
        s["fetch_bytes"] += int(rb)
        s["write_bytes"] += int(wb)
        lines.append(f"  {st:<18} {k:<48} {fk[k][0]:>9} {fv:>12.0f} {wv:>10.0f} {rb / 1e9:>8.3f} "
                     f"{wb / 1e9:>8.3f}")
    print("\n".join(lines))
    if update:
        try:
            with open(TRAFFIC_FILE) as f:
                tr = json.load(f)
        except (OSError, ValueError):
            tr = {}
        sha = kernel_source_sha()
        if tr.get("kernel_source_sha") != sha:
            tr = {"kernel_source_sha": sha}
        tr["fetch_factor"], tr["write_factor"] = ff, wf
        tr.setdefault(workload, {}).update(steps)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(tr, f, indent=1)
        log(f"[bench] traffic of {workload} stored under kernel sources {sha}")


def summarize_counters(path, skip):
    """Per kernel of the block: every counter of a rocprofv3 --pmc run,
    summed over the dispatch's rows and averaged over the launches after the
    first `skip`; with SQ_LDS_BANK_CONFLICT and SQ_LDS_IDX_ACTIVE the share
    of LDS cycles lost to bank conflicts, with SQ_VALU_MFMA_BUSY_CYCLES and
    GRBM_GUI_ACTIVE the MFMA busy fraction per SIMD (1024 SIMDs, 8 XCDs)."""
    rows = _csv_files(path, "counter_collection.csv")
    per, names = {}, {}
    for r in rows:
        k = short_kernel_name(r["Kernel_Name"])
        if step_of(k) == "other":
            continue
        d = int(r["Dispatch_Id"])
        names[d] = k
        per.setdefault(d, {}).setdefault(r["Counter_Name"], 0.0)
        per[d][r["Counter_Name"]] += float(r["Counter_Value"])
    by = {}
    for d in sorted(per):
        by.setdefault(names[d], []).append(per[d])
    lines = [f"# skipped: the first {skip} launches of each kernel"]
    for k, lst in by.items():
        lst = lst[skip:] or lst
        avg = {c: sum(x.get(c, 0.0) for x in lst) / len(lst) for c in lst[0]}
        derived = []
        if "SQ_LDS_BANK_CONFLICT" in avg and avg.get("SQ_LDS_IDX_ACTIVE"):
            derived.append("lds_bank_conflict_share=%.3f" % (avg["SQ_LDS_BANK_CONFLICT"] /
                                                            avg["SQ_LDS_IDX_ACTIVE"]))
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and avg.get("GRBM_GUI_ACTIVE"):
            derived.append("mfma_busy=%.3f" % (avg["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 /
                                               (avg["GRBM_GUI_ACTIVE"] / 8)))
        lines.append(f"  {step_of(k):<18} {k:<48} launches={len(lst)} " + " ".join(
            f"{c}={v:.4g}" for c, v in sorted(avg.items())) + ("  " + " ".join(derived)
                                                              if derived else ""))
    print("\n".join(lines))


def kernels_only(args, weights):
    """The timed workload's steps as separate calls only (warmup + steps
    launches of each kernel, nothing else on the GPU), optionally with the
    FP8 expert FFN, a plain 1 GiB device copy for counter calibration, and
    the event times of this same run."""
    import torch

    from group_limited_routing_router_amd import moe
    from group_limited_routing_router_amd.inputs import CONFIGS, make_weights_fp8

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        bb = torch.empty_like(a)
        for _ in range(3):
            bb.copy_(a)
        torch.cuda.synchronize()
        del a, bb
    if args.workload == "dense":  # the dense MLP's calls only
        weights.clear()
        torch.cuda.empty_cache()
        print(json.dumps({"mode": "kernels-only", "workload": "dense-mlp", "steps": args.steps,
                          "warmup": args.warmup, "dense_mlp": run_dense(args.steps, args.warmup)}),
              flush=True)
        return
    res = run_workload(args.workload, args.steps, args.warmup, weights, forward=False)
    line = {"mode": "kernels-only", "workload": f"beam-moe-{args.workload}", "steps": args.steps,
            "warmup": args.warmup,
            "kernels_ms": {k: round(v, 4) for k, v in res["kernel_ms"].items()},
            "roofline": roofline_for(res, "gate_up")}
    if args.with_fp8:
        cfg, b, d = res["cfg"], res["buffers"], res["inputs"]
        for k in ("w_gate", "w_up", "w_down"):
            d.pop(k, None)
        weights.clear()
        torch.cuda.empty_cache()
        w8 = make_weights_fp8(CONFIGS["decode"], seed=0, device="cuda")
        p = moe.MoEProblem.from_config(cfg)

        def ffn8():
            moe.moe_expert_ffn_fp8(p, d["x"], b["sorted_pairs"], b["expert_offsets"], w8["q_gate"],
                                   w8["s_gate"], w8["q_up"], w8["s_up"], w8["q_down"],
                                   w8["s_down"], b["y"], b["ws"])

        ms, _ = timed_steps(ffn8, args.steps, args.warmup)
        line["fp8_expert_ffn_ms"] = round(ms, 4)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill",
                    choices=["prefill", "decode", "skew", "long", "dense"],
                    help="the timed workload (dense: with --kernels-only only)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary decode, skew and long measurements")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the secondary FP8-weight measurements")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the secondary dense-MLP measurement")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the achievable-peak measurement kernels")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM counters)")
    ap.add_argument("--gemm-study", action="store_true",
                    help="instead of the benchmark: the prefill expert GEMMs at fixed rows per "
                         "expert next to the library batched GEMM (one JSON line)")
    ap.add_argument("--power-study", action="store_true",
                    help="instead of the benchmark: board power and clock while each kernel runs "
                         "back to back (amd-smi samples; one JSON line)")
    ap.add_argument("--seconds", type=float, default=3.0,
                    help="with --power-study: seconds per phase")
    ap.add_argument("--kernels-only", action="store_true",
                    help="instead of the benchmark: the workload's steps as separate calls only")
    ap.add_argument("--with-fp8", action="store_true",
                    help="with --kernels-only: also the FP8-weight expert FFN")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print per-kernel durations of a rocprofv3 kernel trace (no GPU)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print HBM bytes per launch from two rocprofv3 --pmc runs (no GPU)")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print per-kernel averages of any rocprofv3 --pmc run (no GPU)")
    ap.add_argument("--skip", type=int, default=0,
                    help="with --summarize-*: leave out the first N launches of each kernel")
    ap.add_argument("--update-traffic", action="store_true",
                    help="with --summarize-pmc: store the figures for --workload")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.skip)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.skip)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.skip, args.workload, args.update_traffic)
        return

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
    if args.power_study:
        power_study(weights, args.seconds)
        return
    if args.kernels_only:
        kernels_only(args, weights)
        return
    if args.workload == "dense":
        raise SystemExit("--workload dense is a --kernels-only choice (the dense MLP is reported "
                         "in the dense_mlp object of every bench line)")

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        bb = torch.empty_like(a)
        for _ in range(3):
            bb.copy_(a)
        torch.cuda.synchronize()
        del a, bb

    peaks = None if args.no_peaks else achievable_peaks()
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
        "value": round(cfg.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        **step_stats(main_res["step_ms"]),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"beam-moe-{cfg.name}", "tokens": cfg.T, "hidden": cfg.H,
                   "intermediate": cfg.I, "experts": cfg.E, "groups": cfg.G,
                   "kept_groups": cfg.TG, "top_k": cfg.k, "scale": cfg.scale,
                   "experts_hit": main_res["n_hit"]},
        "layer": {k: v for k, v in workload_summary(main_res, peaks).items()
                  if k in ("tflops", "mfma_frac", "hbm_gbs", "hbm_frac", "mfma_frac_of_achievable",
                           "hbm_frac_of_achievable", "hot_expert_share")},
        "kernels_ms": {k: round(v, 4) for k, v in kms.items() if k != "combine_residual"},
        "roofline": roofline_for(main_res, dominant),
        # the combine fused with the post-norm and residual update (not part of
        # the timed step: a separate entry point after the block)
        "combine_residual": roofline_for(main_res, "combine_residual"),
    }
    out["graph_replay"] = graph_replay_ms(main_res, args.steps, args.warmup)
    if peaks:
        at_intensity(out["roofline"], peaks)
        out["achievable_hbm_gbs"] = peaks["achievable_hbm_gbs"]
        out["achievable_mfma_tflops"] = peaks["achievable_mfma_tflops"]
        out["achievable"] = peaks
    del main_res
    torch.cuda.empty_cache()
    if not args.no_secondary:
        for name in ("decode", "skew", "long"):
            if name == args.workload:
                continue
            r = run_workload(name, args.steps, args.warmup, weights)
            out[name] = workload_summary(r, peaks)
            if name == "decode":
                out[name]["graph_replay"] = graph_replay_ms(r, args.steps, args.warmup)
            log("[bench] %s T=%d: %.3f ms/step, %.1f%% of bf16 MFMA peak, %.1f%% of HBM peak" % (
                name, r["cfg"].T, r["ms"], 100 * out[name]["mfma_frac"],
                100 * out[name]["hbm_frac"]))
            del r
            torch.cuda.empty_cache()
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
        if peaks:
            at_intensity(out["dense_mlp"]["roofline"], peaks)
        log("[bench] dense MLP T=%d I=%d: %.3f ms/step, %.1f%% of bf16 MFMA peak" % (
            out["dense_mlp"]["tokens"], out["dense_mlp"]["intermediate"],
            out["dense_mlp"]["ms_per_step"], 100 * out["dense_mlp"]["roofline"]["frac"]))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(weights, args.workload, args.cpu_seconds)
        log("[bench] cpu oracle: %s" % out["cpu_baseline"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
