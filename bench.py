#!/usr/bin/env python3
"""Throughput of one expert-parallel rank's share of the MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--only] [--graph]

A step is one pass of the whole share -- route, dispatch (count, scan,
scatter, pack), grouped gate/up GEMM with the SwiGLU epilogue, grouped down
GEMM, combine -- over one batch of seeded synthetic inputs that are already
resident in HBM.

The headline value times K steps of the fused entry point ``moe_layer`` on
the headline workload (default: the 6000-token prefill shard), with a HIP
event before every step, so the line carries the wall-clock mean and the
median and minimum step.  ``--graph`` captures that step in a HIP graph and
replays it.  A second timed region runs the same K steps through the staged
entry points in the order ``moe_layer`` uses, with HIP events on the launch
stream around every stage, so each kernel's average duration (and the
dominant kernel's roofline) is measured live.

Unless ``--only`` is given, the other full-size workloads (decode shard,
skewed prefill, whole layer) are measured the same way afterwards and
reported under ``configs`` (the decode shard under ``decode``), followed by
the grouped-GEMM micro-benchmark of a decode rank: every local expert
activated by one token, for 32, 16, 8, 4 and 2 local experts
(``gemm_single_token_sweep``), and the prefill and decode shards with MXFP8
expert GEMMs (``mxfp8``: the quantisation the pages deploy).  The
line also carries the MFMA and copy rates measured on this chip next to the
published peaks, and the oracle timed on the host cores (headline workload).
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16/fp16 MFMA (published)
PEAK_FP8_TFLOPS = 5033.2      # MI355X dense fp8 MFMA (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published)
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
METRIC = "MoE-layer tokens/s + % bf16 MFMA peak (prefill) / % HBM GB/s (decode), 1 GPU"
OTHERS = ["decode_ep16_shard", "skewed_prefill", "whole_layer"]
PRECISION = {
    "router": "fp32 fma chain (canonical order) on bf16 x and router weight",
    "gate_up": "bf16 x bf16 MFMA, fp32 accumulation",
    "h": "fp16 (SwiGLU activations)",
    "down": "fp16 x fp16 MFMA, fp32 accumulation (down weights bf16 -> fp16 at pack time)",
    "y": "fp16 (expert outputs)",
    "combine_out": "fp32",
}


def parse():
    from moe_layer_03_amd.workloads import WORKLOAD_ORDER
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the clocks settle only after a few tens of steps: with 5 warm-up steps the first timed region ran
    # 4-7 % slower than with 30
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="prefill_ep4_shard", choices=WORKLOAD_ORDER)
    ap.add_argument("--only", action="store_true", help="measure the headline workload only")
    ap.add_argument("--graph", action="store_true", help="replay the step as a captured HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the MFMA and copy rate probes")
    ap.add_argument("--cpu-tokens", type=int, default=None, help="tokens in the oracle's timed sample")
    ap.add_argument("--mxfp8-only", action="store_true",
                    help="measure the workload's MXFP8 path only and print its result object (for profiling)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before the timed region, run a plain device copy (torch.neg) of this many MiB twice, "
                         "so a counter run can scale FETCH_SIZE/WRITE_SIZE against a kernel of known traffic")
    return ap.parse_args()


def host_cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.lower().startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def measure_peaks(torch, B, dev):
    """Dense bf16 MFMA rate (the library's probe kernel) and plain copy rate (torch), measured here."""
    res = {}
    blocks, iters = 2048, 4000
    sink = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    B.moe_probe_mfma_bf16(blocks, iters, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    flops = 0
    for _ in range(5):
        flops += B.moe_probe_mfma_bf16(blocks, iters, sink)
    e1.record()
    torch.cuda.synchronize()
    res["mfma_bf16_tflops"] = round(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    del sink
    n = (1 << 30) // 4
    src = torch.randn(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    res["copy_gbs"] = round(5 * 2 * n * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    res["copy_note"] = "1 GiB fp32 device copy (read + write bytes)"
    del src, dst
    torch.cuda.empty_cache()
    return res


def copy_probe(torch, dev, mib):
    """A plain device copy (torch.neg over `mib` MiB of float32, twice): a counter run scales FETCH_SIZE and
    WRITE_SIZE by what they read for this kernel of known traffic."""
    if mib <= 0:
        return
    src = torch.randn(mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def measure(wl, steps, warmup, graph, copy_probe_mib=0):
    """Time `steps` fused steps and `steps` staged steps of workload wl; returns (result dict, inputs)."""
    import numpy as np
    import torch

    from moe_layer_03_amd import binding as B
    from moe_layer_03_amd import workloads as W

    dev = torch.device("cuda:0")
    s = B.Shape.of(wl)

    t_gen = time.perf_counter()
    inp = W.make_inputs(wl)

    def dev_t(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).to(dev)

    x = dev_t(inp.x)
    w_router = dev_t(inp.w_router)
    bias = dev_t(inp.bias) if inp.bias is not None else None
    g, u, d = dev_t(inp.w_gate), dev_t(inp.w_up), dev_t(inp.w_down)
    packed = B.moe_pack_weights(s, g, u, d)
    torch.cuda.synchronize()
    del g, u, d
    t_gen = time.perf_counter() - t_gen

    i32, f32 = torch.int32, torch.float32
    cap = s.cap
    buf = dict(
        topk_idx=torch.empty((s.T, s.K), dtype=i32, device=dev),
        topk_w=torch.empty((s.T, s.K), dtype=f32, device=dev),
        counts=torch.empty(s.E_loc, dtype=i32, device=dev),
        offsets=torch.empty(s.E_loc + 1, dtype=i32, device=dev),
        row_token=torch.empty(cap, dtype=i32, device=dev),
        row_slot=torch.empty(cap, dtype=i32, device=dev),
        slot_row=torch.empty((s.T, s.K), dtype=i32, device=dev),
        x_packed=torch.empty((cap if wl.dtype != "bf16" else 1, s.H), dtype=B.operand_dtype(x.dtype), device=dev),
        h=torch.empty((cap, s.I), dtype=torch.float16, device=dev),
        y=torch.empty((cap, s.H), dtype=torch.float16, device=dev),
        out=torch.empty((s.T, s.H), dtype=f32, device=dev),
        ws=torch.empty(max(B.moe_dispatch_workspace_bytes(s), 16), dtype=torch.uint8, device=dev),
        ws_route=torch.empty(max(B.moe_route_workspace_bytes(s), 16), dtype=torch.uint8, device=dev),
    )
    stages = ["route", "dispatch", "gemm_gate_up", "gemm_down", "combine"]
    gather = wl.dtype == "bf16"

    def step(ev=None):
        b = buf
        if ev is not None:
            ev[0].record()
        B.moe_route(s, x, w_router, bias, topk_idx=b["topk_idx"], topk_w=b["topk_w"], ws=b["ws_route"])
        if ev is not None:
            ev[1].record()
        if gather:   # bf16: the gate/up GEMM reads token rows straight from x, as moe_layer does
            B.moe_dispatch(s, b["topk_idx"], None, counts=b["counts"], offsets=b["offsets"],
                           row_token=b["row_token"], row_slot=b["row_slot"], slot_row=b["slot_row"], ws=b["ws"])
        else:
            B.moe_dispatch(s, b["topk_idx"], x, counts=b["counts"], offsets=b["offsets"], row_token=b["row_token"],
                           row_slot=b["row_slot"], slot_row=b["slot_row"], x_packed=b["x_packed"], ws=b["ws"])
        if ev is not None:
            ev[2].record()
        if gather:
            B.moe_grouped_gemm(s, x, b["offsets"], packed, B.MOE_GEMM_GATE_UP, B.MOE_EPI_SWIGLU, c=b["h"],
                               a_rows=b["row_token"])
        else:
            B.moe_grouped_gemm(s, b["x_packed"], b["offsets"], packed, B.MOE_GEMM_GATE_UP, B.MOE_EPI_SWIGLU,
                               c=b["h"])
        if ev is not None:
            ev[3].record()
        B.moe_grouped_gemm(s, b["h"], b["offsets"], packed, B.MOE_GEMM_DOWN, B.MOE_EPI_NONE, c=b["y"])
        if ev is not None:
            ev[4].record()
        B.moe_combine(s, b["y"], b["slot_row"], b["topk_w"], out=b["out"])
        if ev is not None:
            ev[5].record()

    copy_probe(torch, dev, copy_probe_mib)

    # the fused entry point, on buffers of its own (moe_layer carves its scratch from one workspace)
    ws_layer = torch.empty(max(B.moe_layer_workspace_bytes(s), 16), dtype=torch.uint8, device=dev)
    out_fused = torch.empty((s.T, s.H), dtype=f32, device=dev)

    def fused_step():
        B.moe_layer(s, x, w_router, packed, bias, out=out_fused, ws=ws_layer)

    for _ in range(warmup):
        fused_step()
        step()
    torch.cuda.synchronize()

    # timed region: K steps of the fused entry point, an event before each step and after the last
    ev_f = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    if graph:
        cgraph = torch.cuda.CUDAGraph()
        cap_stream = torch.cuda.Stream()
        cap_stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap_stream):
            with torch.cuda.graph(cgraph, stream=cap_stream):
                fused_step()
        torch.cuda.current_stream().wait_stream(cap_stream)
        cgraph.replay()
        torch.cuda.synchronize()
        run = cgraph.replay
    else:
        run = fused_step
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        ev_f[k].record()
        run()
    ev_f[steps].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    per_step = np.array([ev_f[k].elapsed_time(ev_f[k + 1]) for k in range(steps)])

    # second timed region: the same K steps through the staged entry points, with HIP events around every
    # stage on the launch stream (per-stage durations and the dominant kernel's roofline); each step is queued
    # behind a spin, so the events time the GPU's work, not the host's launches
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    prime = queue_primer(torch, step)
    for k in range(steps):
        prime()
        step(events[k])
    torch.cuda.synchronize()
    ms_staged = float(np.mean([events[k][0].elapsed_time(events[k][-1]) for k in range(steps)]))
    stage_ms = {name: float(np.mean([events[k][i].elapsed_time(events[k][i + 1]) for k in range(steps)]))
                for i, name in enumerate(stages)}

    counts = buf["counts"].cpu().numpy()
    n_loc = int(buf["offsets"][-1].item())
    # the staged step and the fused entry point compute the same bits
    fused_equal = bool(torch.equal(buf["out"], out_fused))

    # algorithmic work (route + expert FFN) and bytes (active local experts' weights, router weight,
    # x read once, out written once)
    H, I, E, T = wl.H, wl.I, wl.E, wl.T
    wbytes = 2 if wl.dtype == "bf16" else 4
    active = int((counts > 0).sum())
    flops = 2 * T * H * E + n_loc * (2 * H * 2 * I + 2 * I * H)
    bytes_alg = active * 3 * H * I * 2 + H * E * wbytes + T * H * wbytes + T * H * 4
    sec = ms * 1e-3

    # dominant kernel: the gate/up grouped GEMM (two thirds of the FLOPs and of the weight bytes)
    gu_flops = n_loc * 2 * H * 2 * I
    gu_bytes = active * 2 * H * I * 2 + n_loc * H * 2 + n_loc * I * 2
    skinny = T * wl.K <= 64 * E   # the library's choice: weight streaming when an even expert gets <= 64 rows
    kname = ("grouped_gemm_skinny_kernel<SwiGLU,bf16,fp16,4> (gate/up)" if skinny
             else "grouped_gemm_kernel<4,SwiGLU,bf16,fp16,4> (gate/up)")
    t_gu = stage_ms["gemm_gate_up"] * 1e-3
    if gu_flops / max(gu_bytes, 1) >= RIDGE:
        ach = gu_flops / t_gu / 1e12
        roofline = dict(kernel=kname, bound="mfma", achieved=round(ach, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                        frac=round(ach / PEAK_BF16_TFLOPS, 4), traffic=measured_traffic(wl.name),
                        per_launch=dict(flops=gu_flops, us=round(t_gu * 1e6, 2)))
    else:
        ach = gu_bytes / t_gu / 1e9
        roofline = dict(kernel=kname, bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                        frac=round(ach / PEAK_HBM_GBS, 4), traffic=measured_traffic(wl.name),
                        per_launch=dict(bytes=gu_bytes, us=round(t_gu * 1e6, 2)))

    res = {
        "workload": wl.name,
        "config": {"T": T, "H": H, "E": E, "K": wl.K, "I": I, "local_experts": [wl.e_begin, wl.e_end],
                   "zipf_s": wl.zipf_s, "seed": wl.seed, "mode": "graph" if graph else "eager"},
        "steps": steps,
        "ms_per_step": round(ms, 4),
        "ms_median": round(float(np.median(per_step)), 4),
        "ms_min": round(float(per_step.min()), 4),
        "tokens_s": round(T / sec, 1),
        "tflops": round(flops / sec / 1e12, 2),
        "mfma_frac": round(flops / sec / 1e12 / PEAK_BF16_TFLOPS, 4),
        "gbs": round(bytes_alg / sec / 1e9, 1),
        "hbm_frac": round(bytes_alg / sec / 1e9 / PEAK_HBM_GBS, 4),
        "alg_flops": flops,
        "alg_bytes": bytes_alg,
        "n_loc": n_loc,
        "expert_rows": {"min": int(counts.min()), "mean": round(float(counts.mean()), 2), "max": int(counts.max()),
                        "cv": round(float(counts.std() / counts.mean()), 4) if counts.mean() > 0 else None,
                        "active": active},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "ms_per_step_staged": round(ms_staged, 4),
        "roofline": roofline,
        "fused_entry_bitwise_equal": fused_equal,
        "input_setup_s": round(t_gen, 1),
    }
    del buf, ws_layer, out_fused, packed, x, w_router, bias
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, inp


def queue_primer(torch, step):
    """Returns a function that, called before `step()`, keeps the GPU busy (a torch.cuda._sleep spin) for
    about three times the host time that enqueuing one step takes.  The step's kernels are then all queued
    when the GPU reaches them, so HIP events between its stages time GPU execution, not the host's launch
    latency (staged calls from Python can otherwise leave the GPU idle between stages)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.cuda._sleep(1 << 20)
    e1.record()
    torch.cuda.synchronize()
    cycles_per_us = (1 << 20) / max(e0.elapsed_time(e1) * 1e3, 1e-3)
    host = []
    for _ in range(3):
        t = time.perf_counter()
        step()
        host.append(time.perf_counter() - t)
    torch.cuda.synchronize()
    cycles = int(3 * max(host) * 1e6 * cycles_per_us)
    return lambda: torch.cuda._sleep(cycles)


def measure_mxfp8(wl, steps, warmup, copy_probe_mib=0):
    """The layer share with MXFP8 expert GEMMs (moe_layer_mxfp8): fused steps with a HIP event per step, then
    the staged calls with events around route, activation quantisation, dispatch, gate/up, down and combine."""
    import numpy as np
    import torch

    from moe_layer_03_amd import binding as B
    from moe_layer_03_amd import workloads as W

    dev = torch.device("cuda:0")
    s = B.Shape.of(wl)
    inp = W.make_inputs(wl)

    def dev_t(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).to(dev)

    x, wr = dev_t(inp.x), dev_t(inp.w_router)
    bias = dev_t(inp.bias) if inp.bias is not None else None
    g, u, d = dev_t(inp.w_gate), dev_t(inp.w_up), dev_t(inp.w_down)
    packed = B.moe_pack_weights_mxfp8(s, g, u, d)
    torch.cuda.synchronize()
    del g, u, d, inp
    ws = torch.empty(max(B.moe_layer_workspace_bytes_mxfp8(s), 16), dtype=torch.uint8, device=dev)
    out = torch.empty((s.T, s.H), dtype=torch.float32, device=dev)
    cap = s.cap
    i32 = torch.int32
    b = dict(idx=torch.empty((s.T, s.K), dtype=i32, device=dev), tw=torch.empty((s.T, s.K), dtype=torch.float32,
                                                                               device=dev),
             xc=torch.empty((s.T, s.H), dtype=torch.uint8, device=dev),
             xs=torch.empty((s.T, s.H // 32), dtype=torch.uint8, device=dev),
             hc=torch.empty((cap, s.I), dtype=torch.uint8, device=dev),
             hs=torch.empty((cap, s.I // 32), dtype=torch.uint8, device=dev),
             y=torch.empty((cap, s.H), dtype=torch.float16, device=dev),
             out=torch.empty((s.T, s.H), dtype=torch.float32, device=dev),
             ws_route=torch.empty(max(B.moe_route_workspace_bytes(s), 16), dtype=torch.uint8, device=dev),
             ws_d=torch.empty(max(B.moe_dispatch_workspace_bytes(s), 16), dtype=torch.uint8, device=dev))
    stages = ["route", "quantize_x", "dispatch", "gemm_gate_up", "gemm_down", "combine"]
    dd = {}
    copy_probe(torch, dev, copy_probe_mib)

    def staged(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        B.moe_route(s, x, wr, bias, topk_idx=b["idx"], topk_w=b["tw"], ws=b["ws_route"])
        mark(1)
        B.moe_quantize_mxfp8(x, b["xc"], b["xs"])
        mark(2)
        dd.update(B.moe_dispatch(s, b["idx"], None, ws=b["ws_d"]))
        mark(3)
        B.moe_grouped_gemm_mxfp8(s, b["xc"], b["xs"], dd["offsets"], packed, B.MOE_GEMM_GATE_UP, B.MOE_EPI_SWIGLU,
                                 c=b["hc"], c_dtype=torch.uint8, c_scales=b["hs"], a_rows=dd["row_token"])
        mark(4)
        B.moe_grouped_gemm_mxfp8(s, b["hc"], b["hs"], dd["offsets"], packed, B.MOE_GEMM_DOWN, B.MOE_EPI_NONE,
                                 c=b["y"])
        mark(5)
        B.moe_combine(s, b["y"], dd["slot_row"], b["tw"], out=b["out"])
        mark(6)

    def fused():
        B.moe_layer_mxfp8(s, x, wr, packed, bias, out=out, ws=ws)

    for _ in range(warmup):
        fused()
        staged()
    torch.cuda.synchronize()
    ev_f = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    for k in range(steps):
        ev_f[k].record()
        fused()
    ev_f[steps].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    per = np.array([ev_f[k].elapsed_time(ev_f[k + 1]) for k in range(steps)])
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    prime = queue_primer(torch, staged)
    for k in range(steps):
        prime()
        staged(evs[k])
    torch.cuda.synchronize()
    stage_ms = {nm: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(steps)]))
                for i, nm in enumerate(stages)}
    counts = dd["counts"].cpu().numpy()
    n_loc = int(dd["offsets"][-1].item())
    H, I, E, T = wl.H, wl.I, wl.E, wl.T
    active = int((counts > 0).sum())
    flops = 2 * T * H * E + n_loc * (2 * H * 2 * I + 2 * I * H)
    wbytes = active * 3 * H * I * (1 + 1 / 32)          # fp8 codes + one scale byte per 32
    bytes_alg = wbytes + H * E * 2 + T * H * 2 + T * H * 4
    gu_flops = n_loc * 2 * H * 2 * I
    gu_bytes = active * 2 * H * I * (1 + 1 / 32) + n_loc * H * (1 + 1 / 32) + n_loc * I * (1 + 1 / 32)
    t_gu = stage_ms["gemm_gate_up"] * 1e-3
    # the launcher's rule: few rows per expert stream the weights (HBM-bound form), else the tiled MFMA form
    # (at the prefill shard the gate/up problem sits at the fp8 ridge, so intensity alone cannot name it)
    if T * wl.K > 64 * E:
        ach = gu_flops / t_gu / 1e12
        roof = dict(kernel="grouped_gemm_mx_kernel (gate/up, scaled fp8 MFMA)", bound="mfma", achieved=round(ach, 2),
                    peak=PEAK_FP8_TFLOPS, unit="TFLOP/s", frac=round(ach / PEAK_FP8_TFLOPS, 4),
                    traffic=measured_traffic(wl.name, "mxfp8"),
                    per_launch=dict(flops=gu_flops, us=round(t_gu * 1e6, 2)))
    else:
        ach = gu_bytes / t_gu / 1e9
        roof = dict(kernel="grouped_gemm_mx_skinny_kernel (gate/up, scaled fp8 MFMA)", bound="hbm",
                    achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s", frac=round(ach / PEAK_HBM_GBS, 4),
                    traffic=measured_traffic(wl.name, "mxfp8"),
                    per_launch=dict(bytes=int(gu_bytes), us=round(t_gu * 1e6, 2)))
    sec = ms * 1e-3
    res = {"workload": wl.name, "steps": steps, "ms_per_step": round(ms, 4),
           "ms_median": round(float(np.median(per)), 4), "ms_min": round(float(per.min()), 4),
           "tokens_s": round(T / sec, 1), "tflops": round(flops / sec / 1e12, 2),
           "mfma_frac_fp8_peak": round(flops / sec / 1e12 / PEAK_FP8_TFLOPS, 4),
           "gbs": round(bytes_alg / sec / 1e9, 1), "hbm_frac": round(bytes_alg / sec / 1e9 / PEAK_HBM_GBS, 4),
           "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()}, "roofline": roof,
           "fused_entry_bitwise_equal": bool(torch.equal(out, b["out"]))}
    del packed, ws, out, b, x, wr
    torch.cuda.empty_cache()
    return res


def gemm_single_token_sweep(e_locs=(32, 16, 8, 4, 2), reps=50, warmup=20):
    """The grouped expert GEMMs (gate/up with SwiGLU, then down) with every local expert activated by exactly
    one token, for several local-expert counts: the GEMM micro-benchmark of one expert-parallel decode rank.
    Weights stream from HBM (the packed copy of each count is read once per repetition)."""
    import numpy as np
    import torch

    from moe_layer_03_amd import binding as B
    from moe_layer_03_amd import workloads as W

    dev = torch.device("cuda:0")
    base = W.WORKLOADS["decode_ep16_shard"]
    g, u, d = W.gen_experts(base, range(max(e_locs)))
    x = W.gen_x(base.replace(T=max(e_locs)))
    out = []
    for n in e_locs:
        s = B.Shape(n, base.H, base.E, 1, base.I, 0, n)      # n tokens, one per local expert
        gt, ut, dt_ = (torch.from_numpy(np.ascontiguousarray(a[:n])).view(torch.bfloat16).to(dev) for a in (g, u, d))
        packed = B.moe_pack_weights(s, gt, ut, dt_)
        del gt, ut, dt_
        a = torch.from_numpy(np.ascontiguousarray(x[:n])).view(torch.bfloat16).to(dev)
        offs = torch.arange(n + 1, dtype=torch.int32, device=dev)
        h = torch.empty((n, base.I), dtype=torch.float16, device=dev)
        y = torch.empty((n, base.H), dtype=torch.float16, device=dev)

        def run(ev=None):
            if ev is not None:
                ev[0].record()
            B.moe_grouped_gemm(s, a, offs, packed, B.MOE_GEMM_GATE_UP, B.MOE_EPI_SWIGLU, c=h)
            if ev is not None:
                ev[1].record()
            B.moe_grouped_gemm(s, h, offs, packed, B.MOE_GEMM_DOWN, B.MOE_EPI_NONE, c=y)
            if ev is not None:
                ev[2].record()

        for _ in range(warmup):
            run()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
        torch.cuda.synchronize()
        for k in range(reps):
            run(evs[k])
        torch.cuda.synchronize()
        gu = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e3
        dn = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e3
        tot = gu + dn
        wbytes = n * 3 * base.H * base.I * 2
        med = float(np.median(tot))
        out.append({"local_experts": n, "us_gate_up": round(float(np.median(gu)), 2),
                    "us_down": round(float(np.median(dn)), 2), "us_total": round(med, 2),
                    "us_total_min": round(float(tot.min()), 2), "weight_bytes": wbytes,
                    "gbs": round(wbytes / (med * 1e-6) / 1e9, 1),
                    "hbm_frac": round(wbytes / (med * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)})
        del packed, a, h, y
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              "The expert-parallel share shards by giving each rank its own expert range; run one process per "
              "GPU with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from moe_layer_03_amd import binding as B
    from moe_layer_03_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.load()

    wl = W.WORKLOADS[args.workload]
    if args.mxfp8_only:
        print(json.dumps({"workload": wl.name, "mxfp8": measure_mxfp8(wl, args.steps, args.warmup,
                                                                     args.copy_probe_mib)}), flush=True)
        return
    head, inp = measure(wl, args.steps, args.warmup, args.graph, args.copy_probe_mib)
    print(f"[bench] {wl.name}: {head['ms_per_step']} ms/step", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, inp, args.cpu_tokens)
    del inp

    configs = {wl.name: head}
    if not args.only:
        for name in OTHERS:
            if name == wl.name:
                continue
            r, _ = measure(W.WORKLOADS[name], args.steps, args.warmup, args.graph)
            configs[name] = r
            print(f"[bench] {name}: {r['ms_per_step']} ms/step", file=sys.stderr, flush=True)

    mxfp8 = None
    if not args.only:
        mxfp8 = {}
        for name in ("prefill_ep4_shard", "decode_ep16_shard"):
            mxfp8[name] = measure_mxfp8(W.WORKLOADS[name], args.steps, args.warmup)
            print(f"[bench] mxfp8 {name}: {mxfp8[name]['ms_per_step']} ms/step", file=sys.stderr, flush=True)

    sweep = None
    if not args.only:
        sweep = gemm_single_token_sweep()
        print(f"[bench] single-token GEMM sweep: {[(r['local_experts'], r['us_total']) for r in sweep]}",
              file=sys.stderr, flush=True)

    peaks = None if args.no_peaks else measure_peaks(torch, B, dev)
    if peaks is not None:
        for r in configs.values():
            r["mfma_frac_measured_peak"] = round(r["tflops"] / peaks["mfma_bf16_tflops"], 4)
            r["hbm_frac_measured_copy"] = round(r["gbs"] / peaks["copy_gbs"], 4)

    line = {
        "metric": METRIC,
        "value": head["tokens_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "ms_median": head["ms_median"],
        "ms_min": head["ms_min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16/fp16" if wl.dtype == "bf16" else "f32-in/fp16-mfma",
        "precision": PRECISION if wl.dtype == "bf16" else {"all_gemms": "fp16 x fp16 MFMA, fp32 accumulation"},
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights; no trained weights)",
        "config": dict(workload=wl.name, **head["config"]),
        "tflops": head["tflops"],
        "mfma_frac": head["mfma_frac"],
        "gbs": head["gbs"],
        "hbm_frac": head["hbm_frac"],
        "n_loc": head["n_loc"],
        "expert_rows": head["expert_rows"],
        "stage_ms": head["stage_ms"],
        "ms_per_step_staged": head["ms_per_step_staged"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "fused_entry_bitwise_equal": head["fused_entry_bitwise_equal"],
        "decode": configs.get("decode_ep16_shard"),
        "configs": {k: v for k, v in configs.items() if k != wl.name},
        "gemm_single_token_sweep": sweep,
        "mxfp8": mxfp8,
        "peaks": {"spec_bf16_tflops": PEAK_BF16_TFLOPS, "spec_hbm_gbs": PEAK_HBM_GBS,
                  **(peaks or {})},
        "host_cpu": host_cpu_model(),
        "input_setup_s": head["input_setup_s"],
    }
    if line["decode"] is not None and "decode_ep16_shard" in line["configs"]:
        del line["configs"]["decode_ep16_shard"]
    print(json.dumps(line), flush=True)


# sources of each gate/up GEMM form, hashed into its counter summary
TRAFFIC_SOURCES = {"bf16": ("gemm.hip", "gemm_common.hpp", "common.hpp"),
                   "mxfp8": ("mxfp8.hip", "gemm_common.hpp", "common.hpp")}


def measured_traffic(workload, kind="bf16"):
    """HBM bytes per gate/up GEMM launch from the committed counter summary of this workload, or None.

    The summary's ``traffic:`` line holds FETCH_SIZE/WRITE_SIZE scaled by a plain copy of known size, and a
    SHA-256 of the kernel sources at the time of the counter runs: a kernel changed since then gives None.
    """
    import hashlib
    import re
    name = f"kernels_{workload}.md" if kind == "bf16" else f"kernels_mxfp8_{workload}.md"
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    m = re.search(r"^traffic: kernel=gate_up read_bytes=(\d+) write_bytes=(\d+) sources_sha256=([0-9a-f]+)$",
                  open(path).read(), re.M)
    if not m:
        return None
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[kind]:
        with open(os.path.join(ROOT, "moe_layer_03_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != m.group(3):
        return None
    return int(m.group(1)) + int(m.group(2))


def cpu_baseline(wl, inp, n_tokens):
    """The oracle, as it is, on the first n_tokens tokens of the same workload (host cores)."""
    import oracle
    from moe_layer_03_amd import workloads as W

    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    if n_tokens is None:
        n_tokens = wl.T if wl.T <= 6000 else 4096
    n_tokens = min(n_tokens, wl.T)

    class Lazy:
        def __init__(self, a):
            self.a = a

        def __getitem__(self, i):
            return W.as_f32(self.a[i])

    x = W.as_f32(inp.x[:n_tokens])
    wr = W.as_f32(inp.w_router)
    t0 = time.perf_counter()
    oracle.moe_layer(x, wr, inp.bias, wl.K, wl.e_begin, wl.e_end, Lazy(inp.w_gate), Lazy(inp.w_up),
                     Lazy(inp.w_down))
    dt = time.perf_counter() - t0
    return {"value": round(n_tokens / dt, 1), "unit": "tokens/s", "cores": int(max(oracle.num_threads(), blas)),
            "kind": "oracle", "sample": f"first {n_tokens} of {wl.T} tokens, full route/dispatch/FFN/combine",
            "seconds": round(dt, 2), "host_cpus": os.cpu_count(), "host_cpu": host_cpu_model()}


if __name__ == "__main__":
    main()
