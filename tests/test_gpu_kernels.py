"""Per-entry-point parity of the HIP path against the oracle (through the C-ABI)."""
import numpy as np
import pytest
import torch

import oracle
from helpers import to_torch
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


def _route_case(B, T, H, E, K, dtype="bf16", bias=None, seed=0, w=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H), dtype=np.float32)
    if w is None:
        w = rng.standard_normal((H, E), dtype=np.float32) * np.float32(0.02)
    if dtype == "bf16":
        x, w = _bf16(x), _bf16(w)
    s = B.Shape(T, H, E, K, 64, 0, E)
    bt = to_torch(bias) if bias is not None else None
    idx, tw, lg = B.moe_route(s, to_torch(x), to_torch(w), bt, want_logits=True)
    torch.cuda.synchronize()
    ri, rw, rl = oracle.route(W.as_f32(x), W.as_f32(w), bias, K)
    return idx.cpu().numpy(), tw.cpu().numpy(), lg.cpu().numpy(), ri, rw, rl


@pytest.mark.parametrize("T,H,E,K", [(333, 512, 128, 8), (2050, 256, 128, 8), (5, 64, 8, 2), (40, 128, 200, 8),
                                     (17, 64, 1000, 64), (64, 192, 64, 64)])
def test_route_bit_exact_bf16(B, T, H, E, K):
    idx, tw, lg, ri, rw, rl = _route_case(B, T, H, E, K)
    assert np.array_equal(lg.view(np.uint32), rl.view(np.uint32)), "logits differ from the fixed fma order"
    assert np.array_equal(idx, ri)
    assert np.abs(tw - rw).max() <= 1e-6


@pytest.mark.parametrize("T,H,E,K,dt", [(1, 4096, 128, 8, "bf16"), (128, 4096, 128, 8, "bf16"),
                                        (1024, 256, 128, 8, "bf16"), (7, 128, 72, 4, "bf16"),
                                        (5, 128, 8, 2, "bf16"), (33, 64, 24, 2, "f32"), (100, 320, 64, 64, "f32"),
                                        (50, 4096, 16, 16, "f32"), (65, 192, 120, 8, "f32"), (17, 256, 20, 4, "f32"),
                                        (9, 512, 24, 4, "bf16")])
def test_route_small_batch_bit_exact(B, T, H, E, K, dt):
    """Batches of at most 1024 tokens, both small-batch forms: with somewhere
    to put the logits (H a multiple of 256) the tiled form (8 tokens x 8
    experts per workgroup, tiles cut by T and E); without (no workspace, no
    logits output) one workgroup per token.  Logits bit-exact, selections equal."""
    idx, tw, lg, ri, rw, rl = _route_case(B, T, H, E, K, dtype=dt, seed=T + E)
    assert np.array_equal(lg.view(np.uint32), rl.view(np.uint32)), "logits differ from the fixed fma order"
    assert np.array_equal(idx, ri)
    assert np.abs(tw - rw).max() <= 1e-6
    rng = np.random.default_rng(T + E)
    x = rng.standard_normal((T, H), dtype=np.float32)
    w = rng.standard_normal((H, E), dtype=np.float32) * np.float32(0.02)
    if dt == "bf16":
        x, w = _bf16(x), _bf16(w)
    idx_c, tw_c, _ = B.moe_route(B.Shape(T, H, E, K, 64, 0, E), to_torch(x), to_torch(w), screened=False)
    torch.cuda.synchronize()
    assert np.array_equal(idx_c.cpu().numpy(), ri), "per-token form"
    assert np.array_equal(tw_c.cpu().numpy(), tw), "per-token form"


def test_route_bit_exact_f32_tiny(B):
    wl = W.WORKLOADS["tiny"]
    x, w = W.gen_x(wl), W.gen_router(wl)
    s = B.Shape.of(wl)
    idx, tw, lg = B.moe_route(s, to_torch(x), to_torch(w), want_logits=True)
    torch.cuda.synchronize()
    ri, rw, rl = oracle.route(x, w, None, wl.K)
    assert np.array_equal(lg.cpu().numpy().view(np.uint32), rl.view(np.uint32))
    assert np.array_equal(idx.cpu().numpy(), ri)
    assert np.abs(tw.cpu().numpy() - rw).max() <= 1e-6


def test_route_bias(B):
    wl = W.WORKLOADS["skewed_prefill"].replace(T=1500, H=512)
    bias = W.gen_bias(wl)
    idx, tw, lg, ri, rw, rl = _route_case(B, wl.T, wl.H, wl.E, wl.K, bias=bias, seed=3)
    assert np.array_equal(lg.view(np.uint32), rl.view(np.uint32))
    assert np.array_equal(idx, ri)
    assert np.abs(tw - rw).max() <= 1e-6


def test_route_exact_ties(B):
    T, H, E, K = 100, 128, 128, 8
    rng = np.random.default_rng(4)
    w = rng.standard_normal((H, E), dtype=np.float32) * np.float32(0.02)
    w[:, 64:] = w[:, :64]       # every expert e >= 64 ties bitwise with e - 64
    idx, tw, lg, ri, rw, rl = _route_case(B, T, H, E, K, w=w, seed=4)
    assert np.array_equal(lg[:, 64:], lg[:, :64])
    assert np.array_equal(idx, ri)
    # zero router: all logits 0 -> experts 0..K-1, weights exactly 1/K
    idx0, tw0, lg0, _, _, _ = _route_case(B, 70, 64, 16, 4, w=np.zeros((64, 16), np.float32))
    assert np.all(lg0 == 0) and np.array_equal(idx0, np.tile(np.arange(4), (70, 1))) and np.all(tw0 == 0.25)


def _screened(B, x, w, K, bias=None):
    """Screened route (MFMA estimates + canonical chains for the candidates) and the full canonical route."""
    T, H = x.shape
    E = w.shape[1]
    s = B.Shape(T, H, E, K, 64, 0, E)
    assert B.moe_route_workspace_bytes(s) > 0
    xt, wt = to_torch(x), to_torch(w)
    bt = to_torch(bias) if bias is not None else None
    idx, tw, _ = B.moe_route(s, xt, wt, bt)
    idx_c, tw_c, _ = B.moe_route(s, xt, wt, bt, screened=False)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), tw.cpu().numpy(), idx_c.cpu().numpy(), tw_c.cpu().numpy()


@pytest.mark.parametrize("T,H,K,seed", [(512, 128, 1, 0), (513, 128, 8, 1), (1029, 128, 8, 2), (777, 512, 8, 3),
                                        (700, 4096, 8, 4), (2050, 256, 8, 5), (600, 1024, 64, 6),
                                        (3000, 4096, 8, 9), (6000, 4096, 8, 7)])
def test_route_screened_bit_exact(B, T, H, K, seed):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((T, H), dtype=np.float32))
    w = _bf16(rng.standard_normal((H, 128), dtype=np.float32) * np.float32(0.02))
    idx, tw, idx_c, tw_c = _screened(B, x, w, K)
    ri, rw, _ = oracle.route(W.as_f32(x), W.as_f32(w), None, K)
    assert np.array_equal(idx, ri)
    assert np.array_equal(idx, idx_c)
    assert np.abs(tw - rw).max() <= 1e-6
    assert np.abs(tw - tw_c).max() <= 1e-6


def test_route_screened_bias_ties_and_degenerate(B):
    # skewed bias
    wl = W.WORKLOADS["skewed_prefill"].replace(T=1500, H=512)
    rng = np.random.default_rng(8)
    x = _bf16(rng.standard_normal((wl.T, wl.H), dtype=np.float32))
    w = _bf16(rng.standard_normal((wl.H, 128), dtype=np.float32) * np.float32(0.02))
    bias = W.gen_bias(wl)
    idx, tw, idx_c, _ = _screened(B, x, w, 8, bias)
    ri, rw, _ = oracle.route(W.as_f32(x), W.as_f32(w), bias, 8)
    assert np.array_equal(idx, ri) and np.array_equal(idx, idx_c) and np.abs(tw - rw).max() <= 1e-6
    # bitwise ties: experts 64.. copy experts 0..63 (equal estimates and equal canonical logits)
    w2 = w[:256].copy()
    w2[:, 64:] = w2[:, :64]
    x2 = x[:600, :256].copy()
    idx, tw, idx_c, _ = _screened(B, x2, w2, 8)
    ri, rw, _ = oracle.route(W.as_f32(x2), W.as_f32(w2), None, 8)
    assert np.array_equal(idx, ri) and np.array_equal(idx, idx_c) and np.abs(tw - rw).max() <= 1e-6
    # zero router: no estimate error, every expert a candidate; experts 0..K-1, weights 1/K
    idx, tw, _, _ = _screened(B, x[:577, :128].copy(), np.zeros((128, 128), np.uint16), 8)
    assert np.array_equal(idx, np.tile(np.arange(8), (577, 1))) and np.all(tw == np.float32(0.125))
    # H not a multiple of 128: no screened path and no tiled one (no workspace); fewer than 512
    # tokens: no screened path, the workspace holds the tiled path's logits
    assert B.moe_route_workspace_bytes(B.Shape(600, 192, 128, 8, 64, 0, 128)) == 0
    assert B.moe_route_workspace_bytes(B.Shape(511, 256, 128, 8, 64, 0, 128)) == 511 * 128 * 4
    idx, tw, lg = B.moe_route(B.Shape(600, 192, 128, 8, 64, 0, 128), to_torch(x[:600, :192].copy()),
                              to_torch(w[:192].copy()))
    torch.cuda.synchronize()
    ri, rw, _ = oracle.route(W.as_f32(x[:600, :192]), W.as_f32(w[:192]), None, 8)
    assert np.array_equal(idx.cpu().numpy(), ri)
    # large activations (products still exact), K = 1
    x3 = _bf16(W.as_f32(x[:640]) * np.float32(64.0))
    idx, tw, idx_c, _ = _screened(B, x3, w, 1)
    ri, rw, _ = oracle.route(W.as_f32(x3), W.as_f32(w), None, 1)
    assert np.array_equal(idx, ri) and np.all(tw == 1.0)


def _screen_bound(B, x, w, bias=None, K=8):
    """Run the screened route with a workspace of our own, read back the MFMA
    estimates and norms it leaves there, rebuild the interval [A - D, A + D]
    the router uses (float32, in the documented order) and check that it holds
    the canonical logit L of every (token, expert).  Returns max |A - L| / D."""
    T, H = x.shape
    E = w.shape[1]
    s = B.Shape(T, H, E, K, 64, 0, E)
    info = B.moe_route_screen_layout(s)
    assert info["bytes"] == B.moe_route_workspace_bytes(s) > 0
    ws = torch.empty(info["bytes"], dtype=torch.uint8, device="cuda")
    bt = to_torch(bias) if bias is not None else None
    idx, tw, _ = B.moe_route(s, to_torch(x), to_torch(w), bt, ws=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    S = info["slices"]

    def view(off, *shape):
        n = int(np.prod(shape))
        return raw[off:off + 4 * n].view(np.float32).reshape(shape)

    part = view(info["part_offset"], S, T, E)
    nx = view(info["nx_offset"], S, T)
    nw = view(info["nw_offset"], S, E)
    A = part[0].copy()
    for sl in range(1, S):
        A = A + part[sl]
    if bias is not None:
        A = A + np.asarray(bias, np.float32)[None, :]
    nX, nW = nx[0].copy(), nw[0].copy()
    for sl in range(1, S):
        nX, nW = nX + nx[sl], nW + nw[sl]
    f = np.float32
    Hu = f(H) * f(2.0 ** -24)
    sx = np.sqrt(nX) * (f(1.0) + f(3.0) * Hu)
    dcoef = (f(1.0625) * f(H) + f(192.0)) * f(2.0 ** -24)
    D = dcoef * (sx[:, None] * np.sqrt(nW)[None, :]) + f(2.0 ** -21) * np.abs(A) + f(1e-30)
    assert A.dtype == np.float32 and D.dtype == np.float32
    L = oracle.router_logits(W.as_f32(x), W.as_f32(w), bias)
    gap = np.abs(A.astype(np.float64) - L.astype(np.float64))
    worst = np.unravel_index(np.argmax(gap / D), gap.shape)
    assert np.all(gap <= D.astype(np.float64)), f"estimate error beyond the bound at (t, e) = {worst}"
    assert np.all((A - D) <= L) and np.all(L <= (A + D)), "the router's float32 interval misses a canonical logit"
    ri, rw, _ = oracle.route(W.as_f32(x), W.as_f32(w), bias, K)
    assert np.array_equal(idx.cpu().numpy(), ri)
    assert np.abs(tw.cpu().numpy() - rw).max() <= 1e-6
    return float((gap / D).max())


def _bound_inputs(kind, T=1024, H=4096, seed=11):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((H, 128), dtype=np.float32) * np.float32(0.02)
    x = rng.standard_normal((T, H), dtype=np.float32)
    if kind == "scaled64":
        x *= np.float32(64.0)
    elif kind == "cancelling":
        # products cancel in pairs: x[2i+1] = -x[2i] and, for 90 % of the pairs, w[2i+1] = w[2i];
        # the logits are small against sum |x w|, the quantity the bound scales with
        x[:, 1::2] = -x[:, 0::2]
        wb = W.as_f32(_bf16(w))
        keep = rng.random(H // 2) < 0.9
        wb[1::2][keep] = wb[0::2][keep]
        w = wb
    elif kind == "exponent_spread":
        # elements spread over 2^-24 .. 2^24; a few rows at 2^40 (every product and square stays normal)
        x *= np.exp2(rng.integers(-24, 25, size=(T, H))).astype(np.float32)
        x[::97] *= np.float32(2.0 ** 40)
    else:
        raise ValueError(kind)
    return _bf16(x), _bf16(w)


@pytest.mark.parametrize("kind", ["scaled64", "cancelling", "exponent_spread"])
def test_route_screened_error_bound(B, kind):
    """The screened router's MFMA estimates stay within the bound D of the
    canonical logits on every (token, expert), for inputs built to stress it."""
    x, w = _bound_inputs(kind)
    ratio = _screen_bound(B, x, w)
    print(f"[{kind}] max |A - L| / D = {ratio:.3e}", flush=True)


@pytest.mark.parametrize("kind", ["scaled64", "cancelling"])
@pytest.mark.parametrize("H", [128, 16384])
def test_route_screened_error_bound_sizes(B, kind, H):
    """The bound at the smallest reduction length the screened path takes (its constant term
    dominates) and at four times the model's (its H term dominates; 16 H-slices)."""
    x, w = _bound_inputs(kind, T=512, H=H, seed=13)
    ratio = _screen_bound(B, x, w)
    print(f"[{kind}, H={H}] max |A - L| / D = {ratio:.3e}", flush=True)


@pytest.mark.parametrize("name", ["prefill_ep4_shard", "skewed_prefill"])
def test_route_screened_error_bound_workloads(B, name):
    """The same bound on the full prefill-shard inputs and on the skewed inputs (Zipf router bias)."""
    wl = W.WORKLOADS[name]
    ratio = _screen_bound(B, W.gen_x(wl), W.gen_router(wl), W.gen_bias(wl), wl.K)
    print(f"[{name}] max |A - L| / D = {ratio:.3e}", flush=True)


@pytest.mark.parametrize("E,K", [(128, 8), (8, 2), (300, 16), (1024, 64)])
def test_route_from_logits_ties(B, E, K):
    T = 257
    rng = np.random.default_rng(5)
    logits = (np.round(rng.standard_normal((T, E)) * 3) / 4).astype(np.float32)
    logits[::7, :4] = np.array([-0.0, 0.0, -0.0, 0.0], np.float32) + logits[::7, :4].max()  # equal maxima
    logits[3, :] = -0.0
    logits[4, :] = 0.0
    logits[5, :] = -1.0
    logits[5, 3] = -0.0          # -0 and +0 tie for the top: lower index first
    logits[5, 2] = 0.0
    s = B.Shape(T, 64, E, K, 64, 0, E)
    idx, tw = B.moe_route_from_logits(s, to_torch(logits))
    torch.cuda.synchronize()
    ri = oracle.select_topk(logits, K)
    rw = oracle.topk_weights(logits, ri)
    assert np.array_equal(idx.cpu().numpy(), ri)
    assert np.abs(tw.cpu().numpy() - rw).max() <= 1e-6


@pytest.mark.parametrize("T,E,K,e0,e1,xdt", [(1000, 128, 8, 0, 32, "bf16"), (1000, 128, 8, 100, 128, "f32"),
                                             (130, 128, 8, 5, 6, "bf16"), (64, 8, 2, 0, 8, "f32"),
                                             (3001, 1024, 16, 0, 1024, "bf16"), (77, 16, 16, 0, 16, "bf16"),
                                             # one-workgroup dispatch (at most 16 chunks of 64 tokens and
                                             # 4096 chunk-expert cells) at its limits, and just past them
                                             (1024, 256, 8, 0, 256, "bf16"), (200, 512, 8, 0, 512, "bf16"),
                                             (1025, 128, 8, 0, 128, "bf16"), (320, 1024, 8, 0, 1024, "bf16")])
def test_dispatch_bit_exact(B, T, E, K, e0, e1, xdt):
    H = 128
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx = oracle.select_topk(logits, K)
    x = rng.standard_normal((T, H), dtype=np.float32)
    xs = _bf16(x) if xdt == "bf16" else x
    s = B.Shape(T, H, E, K, 64, e0, e1)
    d = B.moe_dispatch(s, to_torch(idx), to_torch(xs))
    torch.cuda.synchronize()
    ref = oracle.dispatch(idx, e0, e1)
    n = int(ref["offsets"][-1])
    assert np.array_equal(d["counts"].cpu().numpy(), ref["counts"])
    assert np.array_equal(d["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(d["row_token"].cpu().numpy()[:n], ref["row_token"])
    assert np.array_equal(d["row_slot"].cpu().numpy()[:n], ref["row_slot"])
    assert np.array_equal(d["slot_row"].cpu().numpy(), ref["slot_row"])
    xp = d["x_packed"].view(torch.uint16).cpu().numpy()[:n] if n else np.zeros((0, H), np.uint16)
    # bf16 x is copied; float32 x is rounded to fp16 (nearest even), the operand type of float32 layers
    expect = xs if xdt == "bf16" else xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(xp, expect[ref["row_token"]]), "pack must copy (bf16) or round to fp16 (f32)"


def _gemm_case(B, counts, H, I, seed=7):
    """Integer-valued bf16 operands: every partial sum is exact in fp32."""
    rng = np.random.default_rng(seed)
    E_loc = len(counts)
    n = int(sum(counts))
    K = 1
    T = max(n, 1)
    s = B.Shape(T, H, E_loc, K, I, 0, E_loc)     # cap = T >= n
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = (rng.integers(-4, 5, size=(s.cap, H)) / 16).astype(np.float32)
    wg = (rng.integers(-4, 5, size=(E_loc, H, I)) / 16).astype(np.float32)
    wu = (rng.integers(-4, 5, size=(E_loc, H, I)) / 16).astype(np.float32)
    wd = (rng.integers(-4, 5, size=(E_loc, I, H)) / 16).astype(np.float32)
    return s, offsets, a, wg, wu, wd


@pytest.mark.parametrize("wdt", ["bf16", "f32"])
@pytest.mark.parametrize("counts,H,I", [([37, 0, 300, 129], 256, 128), ([1], 64, 64), ([128, 128], 128, 192),
                                        ([0, 0, 5], 192, 64),
                                        # the tiled kernel's k-loop is chosen per tile by the count of active
                                        # 32-row groups in each 128-row half: 96 and 70 rows give 3, the
                                        # 200-row tile 4 and 3, 33 rows 2, and idle halves 0
                                        ([96, 200, 70, 33], 256, 128),
                                        # full 256-row tiles (both halves with 4 groups) and 511 rows in two
                                        # 256-row tiles; each half copies only its own active row blocks
                                        ([256, 250, 511], 256, 128),
                                        # few rows per expert on average: the weight-streaming kernel, with
                                        # experts of 0, 1, 31, 33, 64, 65 and 150 rows (row groups of 64)
                                        ([150, 0, 1, 31, 33, 0, 0, 64, 65, 0, 0, 0, 0, 0, 0, 0] + [0] * 16,
                                         256, 128),
                                        # every expert activated by one token (the decode GEMM micro-benchmark)
                                        ([1] * 32, 256, 128), ([1, 1], 512, 192)])
def test_grouped_gemm_exact_integers(B, counts, H, I, wdt):
    """Both problems on integer-grid operands, float32 output: bit-exact in any order.
    bf16 weights multiply in bf16, float32 weights in fp16; down always in fp16."""
    s, offsets, a, wg, wu, wd = _gemm_case(B, counts, H, I)
    if wdt == "bf16":
        packed = B.moe_pack_weights(s, to_torch(_bf16(wg)), to_torch(_bf16(wu)), to_torch(_bf16(wd)))
        at = to_torch(_bf16(a))
    else:
        packed = B.moe_pack_weights(s, to_torch(wg), to_torch(wu), to_torch(wd))
        at = to_torch(a.astype(np.float16))
    off = to_torch(offsets)
    c1 = B.moe_grouped_gemm(s, at, off, packed, B.MOE_GEMM_GATE_UP, B.MOE_EPI_NONE, c_dtype=torch.float32)
    h = (np.random.default_rng(8).integers(-4, 5, size=(s.cap, I)) / 16).astype(np.float32)
    c2 = B.moe_grouped_gemm(s, to_torch(h.astype(np.float16)), off, packed, B.MOE_GEMM_DOWN, B.MOE_EPI_NONE,
                            c_dtype=torch.float32)
    torch.cuda.synchronize()
    c1, c2 = c1.cpu().numpy(), c2.cpu().numpy()
    for e in range(len(counts)):
        r0, r1 = offsets[e], offsets[e + 1]
        gu = np.concatenate([a[r0:r1] @ wg[e], a[r0:r1] @ wu[e]], axis=1)
        assert np.array_equal(c1[r0:r1], gu), f"gate/up expert {e}"
        assert np.array_equal(c2[r0:r1], h[r0:r1] @ wd[e]), f"down expert {e}"


def test_grouped_gemm_exact_integers_many_tiles(B):
    """64 experts x 300 rows, 3072 gate/up columns: 1536 tiles, so every
    persistent workgroup of the tiled kernel runs several tiles (ring and LDS
    reused across tiles, the per-XCD tile ranges); bit-exact on integer-grid
    operands for both problems."""
    counts = [300] * 64
    s, offsets, a, wg, wu, wd = _gemm_case(B, counts, 512, 1536, seed=12)
    packed = B.moe_pack_weights(s, to_torch(_bf16(wg)), to_torch(_bf16(wu)), to_torch(_bf16(wd)))
    off = to_torch(offsets)
    c1 = B.moe_grouped_gemm(s, to_torch(_bf16(a)), off, packed, B.MOE_GEMM_GATE_UP, B.MOE_EPI_NONE,
                            c_dtype=torch.float32)
    h = (np.random.default_rng(13).integers(-4, 5, size=(s.cap, 1536)) / 16).astype(np.float32)
    c2 = B.moe_grouped_gemm(s, to_torch(h.astype(np.float16)), off, packed, B.MOE_GEMM_DOWN, B.MOE_EPI_NONE,
                            c_dtype=torch.float32)
    torch.cuda.synchronize()
    c1, c2 = c1.cpu().numpy(), c2.cpu().numpy()
    for e in range(len(counts)):
        r0, r1 = offsets[e], offsets[e + 1]
        gu = np.concatenate([a[r0:r1] @ wg[e], a[r0:r1] @ wu[e]], axis=1)
        assert np.array_equal(c1[r0:r1], gu), f"gate/up expert {e}"
        assert np.array_equal(c2[r0:r1], h[r0:r1] @ wd[e]), f"down expert {e}"


def test_grouped_gemm_exact_integers_max_experts(B):
    """The largest local expert count the GEMMs take (1024): the tiled kernel's
    per-expert tile table at its full size, with experts of 0 to 150 rows
    (about 75 on average, so the tiled kernel runs); bit-exact on integer-grid
    operands for both problems."""
    counts = list(np.random.default_rng(21).integers(0, 151, size=1024))
    s, offsets, a, wg, wu, wd = _gemm_case(B, counts, 256, 128, seed=22)
    packed = B.moe_pack_weights(s, to_torch(_bf16(wg)), to_torch(_bf16(wu)), to_torch(_bf16(wd)))
    off = to_torch(offsets)
    c1 = B.moe_grouped_gemm(s, to_torch(_bf16(a)), off, packed, B.MOE_GEMM_GATE_UP, B.MOE_EPI_NONE,
                            c_dtype=torch.float32)
    h = (np.random.default_rng(23).integers(-4, 5, size=(s.cap, 128)) / 16).astype(np.float32)
    c2 = B.moe_grouped_gemm(s, to_torch(h.astype(np.float16)), off, packed, B.MOE_GEMM_DOWN, B.MOE_EPI_NONE,
                            c_dtype=torch.float32)
    torch.cuda.synchronize()
    c1, c2 = c1.cpu().numpy(), c2.cpu().numpy()
    for e in range(len(counts)):
        r0, r1 = offsets[e], offsets[e + 1]
        gu = np.concatenate([a[r0:r1] @ wg[e], a[r0:r1] @ wu[e]], axis=1)
        assert np.array_equal(c1[r0:r1], gu), f"gate/up expert {e}"
        assert np.array_equal(c2[r0:r1], h[r0:r1] @ wd[e]), f"down expert {e}"


def test_grouped_gemm_swiglu(B):
    """SwiGLU epilogue against float64: float32 output within accumulation-order
    noise; 16-bit outputs within half an ulp of their format (bf16: 2^-8
    relative, fp16: 2^-11 relative) of that."""
    counts = [200, 3, 0, 129]
    H, I = 512, 256
    rng = np.random.default_rng(9)
    E_loc, n = len(counts), sum(counts)
    s = B.Shape(n, H, E_loc, 1, I, 0, E_loc)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = _bf16(rng.standard_normal((n, H), dtype=np.float32))
    wg = _bf16(rng.standard_normal((E_loc, H, I), dtype=np.float32) * np.float32(0.05))
    wu = _bf16(rng.standard_normal((E_loc, H, I), dtype=np.float32) * np.float32(0.05))
    wd = _bf16(rng.standard_normal((E_loc, I, H), dtype=np.float32) * np.float32(0.05))
    packed = B.moe_pack_weights(s, to_torch(wg), to_torch(wu), to_torch(wd))
    at, off = to_torch(a), to_torch(offsets)
    outs = {}
    for name, dt in (("f32", torch.float32), ("bf16", torch.bfloat16), ("f16", torch.float16)):
        outs[name] = B.moe_grouped_gemm(s, at, off, packed, B.MOE_GEMM_GATE_UP, B.MOE_EPI_SWIGLU, c_dtype=dt)
    torch.cuda.synchronize()
    hf = outs["f32"].cpu().numpy()
    hb = W.as_f32(outs["bf16"].view(torch.uint16).cpu().numpy())
    hh = outs["f16"].cpu().numpy().astype(np.float64)
    for e in range(E_loc):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        X = W.as_f32(a[r0:r1]).astype(np.float64)
        ref = oracle.silu(X @ W.as_f32(wg[e])) * (X @ W.as_f32(wu[e]))
        rms = np.sqrt(np.mean(ref ** 2))
        assert np.abs(hf[r0:r1] - ref).max() <= 1e-4 * rms, f"expert {e} (float32 out)"
        assert np.all(np.abs(hb[r0:r1] - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4 * rms), f"expert {e} (bf16 out)"
        assert np.all(np.abs(hh[r0:r1] - ref) <= 2.0 ** -11 * np.abs(ref) + 1e-4 * rms), f"expert {e} (fp16 out)"


def test_combine_exact(B):
    T, K, H = 300, 8, 256
    rng = np.random.default_rng(10)
    n = 900
    slot_row = np.full(T * K, -1, np.int32)
    slot_row[rng.choice(T * K, n, replace=False)] = rng.permutation(n)
    slot_row = slot_row.reshape(T, K)
    y = (rng.integers(-64, 64, size=(n, H))).astype(np.float32)
    s = B.Shape(T, H, 64, K, 64, 0, 8)           # cap = T*8 >= n
    yb = np.zeros((s.cap, H), np.float32)
    yb[:n] = y
    ref = oracle.combine(y.astype(np.float64), slot_row, np.ones((T, K)), T, H)
    for yt in (to_torch(_bf16(yb)), to_torch(yb.astype(np.float16)), to_torch(yb)):
        out = B.moe_combine(s, yt, to_torch(slot_row), to_torch(np.ones((T, K), np.float32)))
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref.astype(np.float32)), f"y dtype {yt.dtype}"


def test_zero_tokens(B):
    s = B.Shape(0, 128, 16, 4, 64, 2, 10)
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    d = B.moe_dispatch(s, e)
    torch.cuda.synchronize()
    assert d["counts"].cpu().numpy().tolist() == [0] * 8
    assert d["offsets"].cpu().numpy().tolist() == [0] * 9


def test_invalid_arguments_raise(B):
    s = B.Shape(4, 100, 16, 4, 64, 0, 16)      # H not a multiple of 64
    x = torch.zeros((4, 100), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((100, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(s, x, w)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED
