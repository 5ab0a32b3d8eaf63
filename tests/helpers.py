"""Shared test plumbing: moving seeded inputs to the GPU, calling the C-ABI
through the binding, and feeding the same inputs to the oracle."""
from __future__ import annotations

import numpy as np
import torch

from moe_layer_03_amd import workloads as W


def to_torch(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy storage array -> torch tensor on the device (uint16 storage becomes bfloat16)."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device)


class LazyF32:
    """Per-expert float32 view of stacked storage arrays, widened on access."""

    def __init__(self, stacked: np.ndarray):
        self.a = stacked

    def __len__(self):
        return self.a.shape[0]

    def __getitem__(self, i):
        return W.as_f32(self.a[i])


def oracle_args(inp: W.Inputs):
    """(x, w_router, bias, w_gate, w_up, w_down) as the oracle takes them."""
    return (W.as_f32(inp.x), W.as_f32(inp.w_router), inp.bias,
            LazyF32(inp.w_gate), LazyF32(inp.w_up), LazyF32(inp.w_down))


class GpuLayer:
    """Device copies of a workload's inputs and packed weights."""

    def __init__(self, inp: W.Inputs, device="cuda"):
        from moe_layer_03_amd import binding as B
        self.B = B
        wl = inp.wl
        self.wl = wl
        self.s = B.Shape.of(wl)
        self.x = to_torch(inp.x, device)
        self.w_router = to_torch(inp.w_router, device)
        self.bias = to_torch(inp.bias, device) if inp.bias is not None else None
        g, u, d = to_torch(inp.w_gate, device), to_torch(inp.w_up, device), to_torch(inp.w_down, device)
        self.packed = B.moe_pack_weights(self.s, g, u, d)
        torch.cuda.synchronize()
        del g, u, d
        self.ws = torch.empty(max(B.moe_layer_workspace_bytes(self.s), 16), dtype=torch.uint8, device=device)

    def run(self, out=None):
        """moe_layer with every optional output requested; returns numpy dict."""
        s, B = self.s, self.B
        dev = self.x.device
        o = dict(
            topk_idx=torch.empty((s.T, s.K), dtype=torch.int32, device=dev),
            topk_w=torch.empty((s.T, s.K), dtype=torch.float32, device=dev),
            counts=torch.empty(s.E_loc, dtype=torch.int32, device=dev),
            offsets=torch.empty(s.E_loc + 1, dtype=torch.int32, device=dev),
            row_token=torch.empty(s.cap, dtype=torch.int32, device=dev),
            row_slot=torch.empty(s.cap, dtype=torch.int32, device=dev),
            slot_row=torch.empty((s.T, s.K), dtype=torch.int32, device=dev),
        )
        out = B.moe_layer(s, self.x, self.w_router, self.packed, self.bias, out=out, ws=self.ws, **o)
        torch.cuda.synchronize()
        res = {k: v.cpu().numpy() for k, v in o.items()}
        n = int(res["offsets"][-1])
        res["row_token"] = res["row_token"][:n]
        res["row_slot"] = res["row_slot"][:n]
        res["out"] = out.cpu().numpy()
        return res


def assert_close_rms(got: np.ndarray, ref: np.ndarray, rel: float = 2e-2, what="out"):
    """max |got - ref| <= rel * RMS(ref) over all elements compared."""
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(np.asarray(got, dtype=np.float64) - ref).max() if ref.size else 0.0
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    assert err <= rel * rms, f"{what}: max|err| {err:.3e} > {rel} * RMS {rms:.3e}"
    return err, rms
