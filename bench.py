#!/usr/bin/env python3
"""Throughput of one expert-parallel rank's share of the MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--graph]

A step is one pass of the whole share -- route, dispatch (count, scan,
scatter, pack), grouped gate/up GEMM with the SwiGLU epilogue, grouped down
GEMM, combine -- over one batch of seeded synthetic inputs that are already
resident in HBM.  The headline value times K steps of the fused entry point
``moe_layer``; ``--graph`` captures that step in a HIP graph and replays it.
A second timed region runs the same K steps through the staged entry points
in the order ``moe_layer`` uses, with HIP events on the launch stream around
every stage, so each kernel's average duration (and the dominant kernel's
roofline) is measured live.  Prints one JSON line.
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

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
METRIC = "MoE-layer tokens/s + % bf16 MFMA peak (prefill) / % HBM GB/s (decode), 1 GPU"


def parse():
    from moe_layer_03_amd.workloads import WORKLOAD_ORDER
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the clocks settle only after a few tens of steps: with 5 warm-up steps the first timed region ran
    # 4-7 % slower than with 30
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="prefill_ep4_shard", choices=WORKLOAD_ORDER)
    ap.add_argument("--graph", action="store_true", help="replay the step as a captured HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=None, help="tokens in the oracle's timed sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before the timed region, run a plain device copy (torch.neg) of this many MiB twice, "
                         "so a counter run can scale FETCH_SIZE/WRITE_SIZE against a kernel of known traffic")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              "The expert-parallel share shards by giving each rank its own expert range; run one process per "
              "GPU with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from moe_layer_03_amd import binding as B
    from moe_layer_03_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = W.WORKLOADS[args.workload]
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

    i32, f32, bf = torch.int32, torch.float32, torch.bfloat16
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
    )
    stages = ["route", "dispatch", "gemm_gate_up", "gemm_down", "combine"]
    gather = wl.dtype == "bf16"

    def step(ev=None):
        b = buf
        if ev is not None:
            ev[0].record()
        B.moe_route(s, x, w_router, bias, topk_idx=b["topk_idx"], topk_w=b["topk_w"])
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

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.randn(n, dtype=f32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # the fused entry point, on buffers of its own (moe_layer carves its scratch from one workspace)
    ws_layer = torch.empty(max(B.moe_layer_workspace_bytes(s), 16), dtype=torch.uint8, device=dev)
    out_fused = torch.empty((s.T, s.H), dtype=f32, device=dev)

    def fused_step():
        B.moe_layer(s, x, w_router, packed, bias, out=out_fused, ws=ws_layer)

    for _ in range(args.warmup):
        fused_step()
        step()
    torch.cuda.synchronize()

    # timed region: K steps of the fused entry point (the headline value)
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        cap_stream = torch.cuda.Stream()
        cap_stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap_stream):
            with torch.cuda.graph(graph, stream=cap_stream):
                fused_step()
        torch.cuda.current_stream().wait_stream(cap_stream)
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fused_step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # second timed region: the same K steps through the staged entry points, with HIP events around every
    # stage on the launch stream (per-stage durations and the dominant kernel's roofline)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    ms_staged = (time.perf_counter() - t0) * 1e3 / args.steps
    stage_ms = {name: float(np.mean([events[k][i].elapsed_time(events[k][i + 1]) for k in range(args.steps)]))
                for i, name in enumerate(stages)}

    counts = buf["counts"].cpu().numpy()
    n_loc = int(buf["offsets"][-1].item())

    # the staged step and the fused entry point launch the same kernels: same bits
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
    roofline = None
    # the library's choice: the weight-streaming kernel when an evenly routed expert gets <= 64 rows
    skinny = T * wl.K <= 64 * E
    kname = ("grouped_gemm_skinny_kernel<SwiGLU,bf16,fp16,4> (gate/up)" if skinny
             else "grouped_gemm_kernel<4,SwiGLU,bf16,fp16,4> (gate/up)")
    if stage_ms is not None:
        t_gu = stage_ms["gemm_gate_up"] * 1e-3
        if gu_flops / max(gu_bytes, 1) >= RIDGE:
            ach = gu_flops / t_gu / 1e12
            roofline = dict(kernel=kname, bound="mfma",
                            achieved=round(ach, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                            frac=round(ach / PEAK_BF16_TFLOPS, 4), traffic=measured_traffic(wl.name),
                            per_launch=dict(flops=gu_flops, us=round(t_gu * 1e6, 2)))
        else:
            ach = gu_bytes / t_gu / 1e9
            roofline = dict(kernel=kname, bound="hbm",
                            achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                            frac=round(ach / PEAK_HBM_GBS, 4), traffic=measured_traffic(wl.name),
                            per_launch=dict(bytes=gu_bytes, us=round(t_gu * 1e6, 2)))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, inp, args.cpu_tokens)

    line = {
        "metric": METRIC,
        "value": round(T / sec, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32-in/bf16-mfma",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights; no trained weights)",
        "config": {"workload": wl.name, "T": T, "H": H, "E": E, "K": wl.K, "I": I,
                   "local_experts": [wl.e_begin, wl.e_end], "zipf_s": wl.zipf_s, "seed": wl.seed,
                   "mode": "graph" if args.graph else "eager"},
        "tflops": round(flops / sec / 1e12, 2),
        "mfma_frac": round(flops / sec / 1e12 / PEAK_BF16_TFLOPS, 4),
        "gbs": round(bytes_alg / sec / 1e9, 1),
        "hbm_frac": round(bytes_alg / sec / 1e9 / PEAK_HBM_GBS, 4),
        "n_loc": n_loc,
        "expert_rows": {"min": int(counts.min()), "mean": round(float(counts.mean()), 2), "max": int(counts.max())},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "ms_per_step_staged": round(ms_staged, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "fused_entry_bitwise_equal": fused_equal,
        "input_setup_s": round(t_gen, 1),
    }
    print(json.dumps(line), flush=True)


def measured_traffic(workload):
    """HBM bytes per gate/up GEMM launch from the committed counter summary of this workload, or None.

    The summary's ``traffic:`` line holds FETCH_SIZE/WRITE_SIZE scaled by a plain copy of known size, and a
    SHA-256 of the kernel sources at the time of the counter runs: a kernel changed since then gives None.
    """
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"kernels_{workload}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"^traffic: kernel=gate_up read_bytes=(\d+) write_bytes=(\d+) sources_sha256=([0-9a-f]+)$",
                  open(path).read(), re.M)
    if not m:
        return None
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.hpp"):
        with open(os.path.join(ROOT, "moe_layer_03_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != m.group(3):
        return None
    return int(m.group(1)) + int(m.group(2))


def cpu_baseline(wl, inp, n_tokens):
    """The oracle, as it is, on the first n_tokens tokens of the same workload (host cores)."""
    import numpy as np

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
            "seconds": round(dt, 2), "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
