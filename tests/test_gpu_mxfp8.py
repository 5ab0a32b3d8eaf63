"""MXFP8 path (quantiser, weight conversion, scaled-MFMA grouped GEMMs, layer)
against the MXFP8 oracle, through the C-ABI."""
import numpy as np
import pytest
import torch

import oracle
import oracle.mxfp8 as MX
from helpers import LazyF32, to_torch
from moe_layer_03_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_layer_03_amd import binding
    binding.load()
    return binding


def _bf16(a):
    return W.f32_to_bf16_bits(np.asarray(a, np.float32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_bit_exact(B, dtype):
    """Codes and scales equal the oracle's on rows with a spread of magnitudes,
    all-zero blocks, exact ties and values that saturate."""
    rng = np.random.default_rng(40)
    x = rng.standard_normal((333, 512)).astype(np.float32) * np.exp2(rng.integers(-40, 40, size=(333, 1)))
    x[5] = 0.0
    x[7, :32] = 0.0
    x[9, ::3] *= 1e-6                                    # subnormal codes next to large values
    pos = MX.e4m3_values()[:0x7F]
    x[11, :126] = ((pos[:-1] + pos[1:]) / 2)[:126] * 2.0 ** -5   # ties (block maxima set the scale 2^-5...)
    x[11, 31::32] = 448 * 2.0 ** -5
    x[13, :] = 1.99 * np.sign(rng.standard_normal(512))        # saturation: 1.99 * 2^8 > 448
    x = x.astype(np.float32)
    if dtype == "bf16":
        xs = _bf16(x)
        xv = W.as_f32(xs)
    else:
        xs = xv = x
    codes, scales = B.moe_quantize_mxfp8(to_torch(xs))
    torch.cuda.synchronize()
    rc, rs = MX.quantize(xv.astype(np.float64))
    assert np.array_equal(scales.cpu().numpy(), rs), "scales differ from the oracle"
    got = codes.cpu().numpy()
    bad = np.argwhere(got != rc)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"


def _int_weights(rng, E_loc, Kd, N):
    """Integers in [-8, 8] with an 8 or -8 in every 32-block along K of every column: MXFP8 with
    scale 2^-5 represents them exactly."""
    w = rng.integers(-8, 9, size=(E_loc, Kd, N)).astype(np.float32)
    pos = rng.integers(0, 32, size=(E_loc, Kd // 32, N))
    sign = np.where(rng.random((E_loc, Kd // 32, N)) < 0.5, -8.0, 8.0)
    for b in range(Kd // 32):
        np.put_along_axis(w[:, 32 * b:32 * b + 32, :], pos[:, b:b + 1, :], sign[:, b:b + 1, :], axis=1)
    return w


def _int_activations(rng, rows, K):
    """Codes of integers in [-8, 8] with block scales 2^-2 .. 2^2: every product and partial sum of the
    GEMMs below is exact in float32."""
    vals = rng.integers(-8, 9, size=(rows, K)).astype(np.float64)
    codes = MX.e4m3_encode(vals)
    scales = (127 + rng.integers(-2, 3, size=(rows, K // 32))).astype(np.uint8)
    return codes, scales, MX.dequantize(codes, scales)


@pytest.mark.parametrize("counts,H,I", [([300, 200, 150, 100, 0, 37], 512, 256),
                                        ([300, 200, 150, 100, 0, 37], 768, 512),
                                        ([1] * 32, 512, 256), ([5, 0, 70, 3], 512, 256)],
                         ids=["tiled", "tiled_half_scale_group", "one_token_per_expert", "weight_streaming"])
def test_grouped_gemm_exact_integers(B, counts, H, I):
    """Both problems, float32 output, bit-exact: the tiled form (many rows per
    expert) and the weight-streaming form (few).  The tiled form stages scales
    8 k-steps (K = 512) at a time: K = 512 is one whole group, K = 768 a whole
    group and a half one; K = 256 (the down problem at I = 256) takes the
    weight-streaming form whatever the rows."""
    rng = np.random.default_rng(41)
    E_loc, n = len(counts), int(sum(counts))
    s = B.Shape(n, H, E_loc, 1, I, 0, E_loc)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    wg, wu = _int_weights(rng, E_loc, H, I), _int_weights(rng, E_loc, H, I)
    wd = _int_weights(rng, E_loc, I, H)
    packed = B.moe_pack_weights_mxfp8(s, to_torch(_bf16(wg)), to_torch(_bf16(wu)), to_torch(_bf16(wd)))
    ac, asc, av = _int_activations(rng, n, H)
    hc, hsc, hv = _int_activations(rng, n, I)
    off = to_torch(offsets)
    c1 = B.moe_grouped_gemm_mxfp8(s, to_torch(ac), to_torch(asc), off, packed, B.MOE_GEMM_GATE_UP, B.MOE_EPI_NONE,
                                  c_dtype=torch.float32)
    c2 = B.moe_grouped_gemm_mxfp8(s, to_torch(hc), to_torch(hsc), off, packed, B.MOE_GEMM_DOWN, B.MOE_EPI_NONE,
                                  c_dtype=torch.float32)
    torch.cuda.synchronize()
    c1, c2 = c1.cpu().numpy(), c2.cpu().numpy()
    for e in range(E_loc):
        r0, r1 = offsets[e], offsets[e + 1]
        gu = np.concatenate([av[r0:r1] @ wg[e], av[r0:r1] @ wu[e]], axis=1).astype(np.float32)
        assert np.array_equal(c1[r0:r1], gu), f"gate/up expert {e}"
        assert np.array_equal(c2[r0:r1], (hv[r0:r1] @ wd[e]).astype(np.float32)), f"down expert {e}"


@pytest.mark.parametrize("counts", [[200, 130, 0, 61], [3, 9, 0, 1]], ids=["tiled", "weight_streaming"])
def test_swiglu_mxfp8_output(B, counts):
    """SwiGLU written as MXFP8: against the oracle's quantisation of silu(g) * u
    computed in float64 from the exact g and u.  The GPU forms h in float32, so
    a value within rounding of an E4M3 tie may take the neighbouring code: at
    most 0.1 % of codes may differ, each by one step, and scales may differ only
    where a block maximum sits at a power-of-two boundary."""
    rng = np.random.default_rng(42)
    H, I = 512, 256
    E_loc, n = len(counts), int(sum(counts))
    s = B.Shape(n, H, E_loc, 1, I, 0, E_loc)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    wg, wu = _int_weights(rng, E_loc, H, I) / 64, _int_weights(rng, E_loc, H, I) / 64
    wd = _int_weights(rng, E_loc, I, H)
    packed = B.moe_pack_weights_mxfp8(s, to_torch(_bf16(wg)), to_torch(_bf16(wu)), to_torch(_bf16(wd)))
    ac, asc, av = _int_activations(rng, n, H)
    hc, hs = B.moe_grouped_gemm_mxfp8(s, to_torch(ac), to_torch(asc), to_torch(offsets), packed, B.MOE_GEMM_GATE_UP,
                                      B.MOE_EPI_SWIGLU, c_dtype=torch.uint8)
    torch.cuda.synchronize()
    hc, hs = hc.cpu().numpy()[:n], hs.cpu().numpy()[:n]
    ref = np.zeros((n, I))
    for e in range(E_loc):
        r0, r1 = offsets[e], offsets[e + 1]
        ref[r0:r1] = oracle.silu(av[r0:r1] @ wg[e]) * (av[r0:r1] @ wu[e])
    rc, rs = MX.quantize(ref)
    assert np.mean(hs == rs) >= 0.999, "h scales"
    same_scale = np.repeat(hs == rs, 32, axis=1)
    diff = hc != rc
    assert np.mean(diff) <= 1e-3, f"{np.mean(diff):.2e} of h codes differ"
    step = np.abs(MX.e4m3_values()[hc.astype(int)] - MX.e4m3_values()[rc.astype(int)])
    assert np.all(step[diff & same_scale] <= 32.0 + 1e-9), "a differing code is more than one E4M3 step away"


def _layer_case(B, wl, sample_check=None):
    inp = W.make_inputs(wl)
    s = B.Shape.of(wl)
    dev = "cuda"
    x, wr = to_torch(inp.x), to_torch(inp.w_router)
    bias = to_torch(inp.bias) if inp.bias is not None else None
    g, u, d = to_torch(inp.w_gate), to_torch(inp.w_up), to_torch(inp.w_down)
    packed = B.moe_pack_weights_mxfp8(s, g, u, d)
    torch.cuda.synchronize()
    del g, u, d
    o = dict(topk_idx=torch.empty((s.T, s.K), dtype=torch.int32, device=dev),
             counts=torch.empty(s.E_loc, dtype=torch.int32, device=dev),
             offsets=torch.empty(s.E_loc + 1, dtype=torch.int32, device=dev),
             slot_row=torch.empty((s.T, s.K), dtype=torch.int32, device=dev))
    out = B.moe_layer_mxfp8(s, x, wr, packed, bias, **o)
    torch.cuda.synchronize()
    ref = MX.moe_layer(W.as_f32(inp.x), W.as_f32(inp.w_router), inp.bias, wl.K, wl.e_begin, wl.e_end,
                       LazyF32(inp.w_gate), LazyF32(inp.w_up), LazyF32(inp.w_down))
    for k in ("topk_idx", "counts", "offsets", "slot_row"):
        assert np.array_equal(o[k].cpu().numpy(), ref[k]), k
    got = out.cpu().numpy()
    stats = mx_layer_close(got, ref["out"])
    none = ~(ref["slot_row"] >= 0).any(1)
    assert np.all(got[none] == 0.0)
    return stats


def mx_layer_close(got, ref):
    """Tolerance of the MXFP8 layer against the MXFP8 oracle.  The scaled fp8
    MFMA does not accumulate exactly in float32 (measured: about 2e-5 relative
    RMS on h, where an exact float32 sum would give about 1e-7), so where h lies
    that close to an E4M3 rounding tie the kernel's code is the neighbouring
    one of the oracle's (about 0.2 % of codes); one such code moves an output
    row by up to one E4M3 step of that h element times its down-weight row.
    Both codes are correct roundings of the same h within float32 accuracy, so
    the bar is statistical: RMS(err) <= 5e-3 RMS(out), at most 1 % of elements
    beyond 2e-2 RMS(out), and max |err| <= 0.25 RMS(out) against gross errors
    (a wrong scale or block moves outputs by 100 % or more)."""
    ref = np.asarray(ref, np.float64)
    e = np.abs(np.asarray(got, np.float64) - ref)
    rms = float(np.sqrt(np.mean(ref * ref)))
    stats = dict(max=float(e.max() / rms), rms=float(np.sqrt(np.mean(e * e)) / rms), frac=float(np.mean(e > 2e-2 * rms)))
    assert stats["rms"] <= 5e-3 and stats["frac"] <= 1e-2 and stats["max"] <= 0.25, stats
    return stats


MID = [
    W.Workload("mx_mid", T=700, H=512, E=32, K=4, I=256, e_begin=8, e_end=24, dtype="bf16"),
    W.Workload("mx_f32", T=301, H=256, E=16, K=3, I=256, e_begin=0, e_end=16, dtype="f32"),
    W.Workload("mx_small_batch", T=96, H=512, E=64, K=8, I=256, e_begin=0, e_end=8, dtype="bf16"),
    # few rows per expert with local experts 24..39: the gate/up launch derives the dispatch itself
    W.Workload("mx_small_offset", T=130, H=512, E=64, K=6, I=256, e_begin=24, e_end=40, dtype="bf16"),
    W.Workload("mx_skewed", T=900, H=256, E=64, K=6, I=256, e_begin=0, e_end=16, dtype="bf16", zipf_s=1.1),
]


@pytest.mark.parametrize("wl", MID, ids=lambda w: w.name)
def test_layer_mxfp8(B, wl):
    st = _layer_case(B, wl)
    print(f"[{wl.name}] error / RMS: max {st['max']:.2e}, rms {st['rms']:.2e}, beyond 2e-2: {st['frac']:.2e}",
          flush=True)


@pytest.mark.parametrize("name", ["prefill_ep4_shard", "decode_ep16_shard"])
def test_layer_mxfp8_full_size(B, name):
    """Full-size shards, every token's output against the MXFP8 oracle."""
    st = _layer_case(B, W.WORKLOADS[name])
    print(f"[{name}] error / RMS: max {st['max']:.2e}, rms {st['rms']:.2e}, beyond 2e-2: {st['frac']:.2e}",
          flush=True)


def test_mxfp8_rejects_unsupported_shapes(B):
    s = B.Shape(64, 256, 8, 2, 128, 0, 8)             # I not a multiple of 256
    assert B.moe_packed_weight_bytes_mxfp8(s) == 0 and B.moe_layer_workspace_bytes_mxfp8(s) == 0
    x = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.moe_layer_mxfp8(s, x, torch.zeros((256, 8), dtype=torch.bfloat16, device="cuda"),
                          torch.zeros(256, dtype=torch.uint8, device="cuda"), ws=torch.zeros(256, dtype=torch.uint8,
                                                                                             device="cuda"))
    assert ei.value.status in (B.MOE_ERR_UNSUPPORTED, B.MOE_ERR_WORKSPACE)


@pytest.mark.parametrize("wl", MID + [W.WORKLOADS["decode_ep16_shard"], W.WORKLOADS["prefill_ep4_shard"]],
                         ids=lambda w: w.name)
def test_layer_mxfp8_equals_staged_calls(B, wl):
    """The fused MXFP8 entry point against the staged entry points in the same
    order, bit for bit.  With few rows per expert the fused layer's
    weight-streaming gate/up derives the dispatch itself, while the staged calls
    dispatch with moe_dispatch and gather rows through row_token; the fused
    layer's router works in its workspace (tiled below 1024 tokens, screened
    above), like the staged call given one."""
    inp = W.make_inputs(wl)
    s = B.Shape.of(wl)
    x, wr = to_torch(inp.x), to_torch(inp.w_router)
    bias = to_torch(inp.bias) if inp.bias is not None else None
    g, u, d = to_torch(inp.w_gate), to_torch(inp.w_up), to_torch(inp.w_down)
    packed = B.moe_pack_weights_mxfp8(s, g, u, d)
    torch.cuda.synchronize()
    del g, u, d
    fused = B.moe_layer_mxfp8(s, x, wr, packed, bias)
    ws = torch.empty(max(B.moe_route_workspace_bytes(s), 16), dtype=torch.uint8, device="cuda")
    idx, tw, _ = B.moe_route(s, x, wr, bias, ws=ws)
    xc, xs = B.moe_quantize_mxfp8(x)
    dd = B.moe_dispatch(s, idx, None)
    hc, hs = B.moe_grouped_gemm_mxfp8(s, xc, xs, dd["offsets"], packed, B.MOE_GEMM_GATE_UP, B.MOE_EPI_SWIGLU,
                                      c_dtype=torch.uint8, a_rows=dd["row_token"])
    y = B.moe_grouped_gemm_mxfp8(s, hc, hs, dd["offsets"], packed, B.MOE_GEMM_DOWN, B.MOE_EPI_NONE)
    out = B.moe_combine(s, y, dd["slot_row"], tw)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), fused.cpu().numpy()), "fused and staged MXFP8 outputs differ"
