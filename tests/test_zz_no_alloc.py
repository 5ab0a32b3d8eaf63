"""moe_layer_noalloc (the entry point for callers that cannot allocate)
against moe_layer on the same inputs: same kernels, so the same bits."""
import numpy as np
import pytest
import torch

from helpers import GpuLayer, to_torch
from moe_layer_03_amd import workloads as W

pytestmark = pytest.mark.gpu

KEYS = ("topk_idx", "topk_w", "counts", "offsets", "row_token", "row_slot", "slot_row")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _outputs(s, dev):
    return dict(topk_idx=torch.empty((s.T, s.K), dtype=torch.int32, device=dev),
                topk_w=torch.empty((s.T, s.K), dtype=torch.float32, device=dev),
                counts=torch.empty(s.E_loc, dtype=torch.int32, device=dev),
                offsets=torch.empty(s.E_loc + 1, dtype=torch.int32, device=dev),
                row_token=torch.empty(s.cap, dtype=torch.int32, device=dev),
                row_slot=torch.empty(s.cap, dtype=torch.int32, device=dev),
                slot_row=torch.empty((s.T, s.K), dtype=torch.int32, device=dev))


def _host(o, out):
    r = {k: v.cpu().numpy() for k, v in o.items()}
    n = int(r["offsets"][-1])
    r["row_token"], r["row_slot"] = r["row_token"][:n], r["row_slot"][:n]
    r["out"] = out.cpu().numpy()
    return r


def test_noalloc_equals_moe_layer_two_calls():
    """Two no-alloc calls in a row, the second on a smaller input (the static
    workspace still holds the first call's data), each against moe_layer with
    a workspace of its own."""
    big = W.WORKLOADS["decode_ep16_shard"]
    cases = [big, big.replace(name="decode_small", T=37, seed=5),
             W.WORKLOADS["tiny"]]
    layers = [GpuLayer(W.make_inputs(wl)) for wl in cases]
    B = layers[0].B
    refs = [layer.run() for layer in layers]
    got = []
    for layer in layers:       # back to back, largest first
        s, dev = layer.s, layer.x.device
        assert B.moe_layer_workspace_bytes(s) <= B.MOE_LAYER_NOALLOC_MAX_WS_BYTES
        o = _outputs(s, dev)
        out = torch.full((s.T, s.H), float("nan"), dtype=torch.float32, device=dev)
        B.moe_layer_noalloc(s, layer.x, layer.w_router, layer.packed, layer.bias, out=out, **o)
        got.append((o, out))
    torch.cuda.synchronize()
    for wl, ref, (o, out) in zip(cases, refs, got):
        g = _host(o, out)
        for k in KEYS + ("out",):
            assert np.array_equal(g[k], ref[k]), f"{wl.name}: {k} differs from moe_layer"


def test_noalloc_rejects_oversize_workspace():
    wl = W.WORKLOADS["prefill_ep4_shard"].replace(T=2048)
    from moe_layer_03_amd import binding as B
    s = B.Shape.of(wl)
    assert B.moe_layer_workspace_bytes(s) > B.MOE_LAYER_NOALLOC_MAX_WS_BYTES
    x = torch.zeros((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros((s.H, s.E), dtype=torch.bfloat16, device="cuda")
    packed = torch.zeros(256, dtype=torch.uint8, device="cuda")
    out = torch.zeros((s.T, s.H), dtype=torch.float32, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.moe_layer_noalloc(s, x, wr, packed, out=out)
    assert ei.value.status == B.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0, "a rejected call must enqueue nothing"
