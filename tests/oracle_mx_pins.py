"""Pins of the MXFP8 oracle (``oracle.mxfp8``) against what the formats and
mathematics fix: the FP8 E4M3 and E8M0 definitions of the OCP Microscaling
format, torch's own float32 -> float8_e4m3fn conversion (a library routine),
closed forms, a block-by-block brute force, and reductions of the layer to
the unquantised one.  ``M`` is the module under test.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def pin_e4m3_table(M):
    """Code values fixed by the E4M3 definition (bias 7, 3 mantissa bits, no
    infinities, NaN only at S.1111.111)."""
    v = M.e4m3_values()
    fixed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0, 0x39: 1.125,
             0x3C: 1.5, 0x40: 2.0, 0x78: 256.0, 0x7D: 416.0, 0x7E: 448.0, 0xB8: -1.0, 0x80: -0.0, 0xFE: -448.0}
    for c, val in fixed.items():
        assert v[c] == val, f"code {c:#x}: {v[c]} != {val}"
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isfinite(v[:0x7F]).all() and np.isfinite(v[0x80:0xFF]).all()
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 0 .. 0x7E must be increasing"
    assert np.array_equal(v[0x80:0xFF], -pos)


def pin_e4m3_encode_matches_torch(M):
    """Nearest-even conversion equals torch's float32 -> float8_e4m3fn cast for
    every value in [-448, 448] tried: random values, every exact code value
    and every midpoint between neighbours (the ties)."""
    rng = np.random.default_rng(30)
    pos = M.e4m3_values()[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    vals = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 2.0 ** -6,
                           rng.standard_normal(5000) * 2.0 ** -9, pos, -pos, mids, -mids,
                           np.nextafter(mids, 0), np.nextafter(mids, 1000)]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = M.e4m3_encode(vals.astype(np.float64))
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} codes differ from torch, e.g. {vals[bad[:3]]} -> {got[bad[:3]]} vs {ref[bad[:3]]}"


def pin_e4m3_ties_and_saturation(M):
    """Worked cases: a tie between 1.0 and 1.125 goes to the even code (1.0);
    between 1.125 and 1.25 to 1.25; above 448 saturates; -0 keeps its sign."""
    enc = M.e4m3_encode(np.array([1.0625, 1.1875, 449.0, 1e6, -1e6, -0.0, -2.0 ** -11]))
    assert enc.tolist() == [0x38, 0x3A, 0x7E, 0x7E, 0xFE, 0x80, 0x80]


def pin_mx_scale_rule(M):
    """The shared exponent is floor(log2(max |v|)) - 8: worked blocks."""
    blocks = np.zeros((5, 32))
    blocks[0, 3] = 1.0                      # amax 1 -> 2^-8; 1.0 / 2^-8 = 256 -> 0x78
    blocks[1, :] = 448.0                    # amax 448 -> 2^0; exact
    blocks[2, 0] = 1.99                     # amax 1.99 -> 2^-8; 1.99 * 256 = 509.44 saturates to 448
    blocks[3, 5] = -3.0                     # amax 3 -> 2^(1-8); -3 / 2^-7 = -384 -> 0xFC
    codes, scales = M.quantize(blocks)      # block 4: all zero -> exponent -127 (e8m0 0), codes 0
    assert scales.tolist() == [[119], [127], [119], [120], [0]], scales.tolist()
    assert codes[0, 3] == 0x78 and codes[0, 0] == 0 and np.all(codes[1] == 0x7E)
    assert codes[2, 0] == 0x7E and codes[3, 5] == 0xFC and np.all(codes[4] == 0)
    assert M.dequantize(codes, scales)[3, 5] == -3.0


def pin_mx_round_trip_bound(M):
    """dequantize(quantize(v)) is within half an E4M3 step of v: 2^-4 |v| in the
    normal range, 2^-10 X among the subnormals (X the block scale), except values
    above 448 X, which saturate; values that are E4M3 values times a block scale
    come back exactly."""
    rng = np.random.default_rng(31)
    v = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-30, 30, size=(64, 1)))
    v[:, ::37] *= 1e-4                       # small elements next to large ones: subnormals
    codes, scales = M.quantize(v)
    dq = M.dequantize(codes, scales)
    X = np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=1)
    sat = np.abs(v) > 448 * X
    err = np.abs(dq - v)
    assert np.all(err[~sat] <= np.maximum(2.0 ** -4 * np.abs(v[~sat]), 2.0 ** -10 * X[~sat])), "round-trip error"
    assert np.all(np.abs(dq[sat]) == 448 * X[sat])
    # exact representables: codes times a power of two, each block holding its largest value (448)
    c = rng.integers(0, 0x7F, size=(8, 64)).astype(np.uint8)
    c[:, ::32] = 0x7E
    sc = rng.integers(100, 150, size=(8, 2)).astype(np.uint8)
    exact = M.dequantize(c, sc)
    c2, sc2 = M.quantize(exact)
    assert np.array_equal(M.dequantize(c2, sc2), exact) and np.array_equal(sc2, sc)


def pin_mx_dot_is_block_factored(M):
    """An MXFP8 dot product computed block by block, with the two scales applied
    once per block as integer powers of two, equals the product of the
    dequantised operands (a second algorithm for the scale placement)."""
    rng = np.random.default_rng(32)
    a = rng.standard_normal((5, 128)) * 3
    b = rng.standard_normal((7, 128)) * 0.02
    ca, sa = M.quantize(a)
    cb, sb = M.quantize(b)
    val = M.e4m3_values()
    brute = np.zeros((5, 7))
    for i in range(5):
        for j in range(7):
            tot = 0.0
            for blk in range(4):
                k = slice(32 * blk, 32 * blk + 32)
                part = float(np.sum(val[ca[i, k]] * val[cb[j, k]]))
                tot += part * 2.0 ** (int(sa[i, blk]) + int(sb[j, blk]) - 254)
            brute[i, j] = tot
    ref = M.dequantize(ca, sa) @ M.dequantize(cb, sb).T
    assert np.allclose(brute, ref, rtol=1e-12, atol=1e-300)
    assert np.allclose(ref, a @ b.T, rtol=0.2, atol=0.2 * np.abs(a @ b.T).max()), "quantisation lost the signal"


def _small_layer(rng, T, H, E, I):
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((H, E)) * 0.1).astype(np.float32)
    wg = (rng.standard_normal((E, H, I)) * 0.1).astype(np.float32)
    wu = (rng.standard_normal((E, H, I)) * 0.1).astype(np.float32)
    wd = (rng.standard_normal((E, I, H)) * 0.1).astype(np.float32)
    return x, wr, wg, wu, wd


def pin_mx_layer_identical_experts_is_quantised_mlp(M):
    """All experts copies of expert 0, all local: the MXFP8 layer equals one
    SwiGLU MLP (torch CPU) on operands quantised per row of x, per column of
    each weight, and per row of h -- the axes the format ties to K."""
    rng = np.random.default_rng(33)
    T, H, E, K, I = 20, 64, 4, 2, 64
    x, wr, wg, wu, wd = _small_layer(rng, T, H, E, I)
    wg[:] = wg[0]
    wu[:] = wu[0]
    wd[:] = wd[0]
    r = M.moe_layer(x, wr, None, K, 0, E, wg, wu, wd)

    def q(t, axis):
        c, s = M.quantize(np.moveaxis(np.asarray(t, np.float64), axis, -1))
        return torch.from_numpy(np.moveaxis(M.dequantize(c, s), -1, axis))
    X, G, U, D = q(x, 1), q(wg[0], 0), q(wu[0], 0), q(wd[0], 0)
    h = F.silu(X @ G) * (X @ U)
    ref = (q(h.numpy(), 1) @ D).numpy()
    assert np.allclose(r["out"], ref, rtol=1e-10, atol=1e-12)


def pin_mx_layer_close_to_unquantised(M):
    """MXFP8 changes the layer by the quantisation error only.  E4M3 rounds each
    operand by about 3 % RMS; through x, the weights, h and the SwiGLU product
    the layer moves by about 8 % RMS, so the RMS difference must stay below 15 %
    of the unquantised output's RMS and the two outputs must correlate above
    0.98 (a missing or misplaced scale moves it by 100 % or more); routing is
    identical."""
    import oracle.moe as moe
    rng = np.random.default_rng(34)
    T, H, E, K, I = 40, 128, 8, 2, 64
    x, wr, wg, wu, wd = _small_layer(rng, T, H, E, I)
    r = M.moe_layer(x, wr, None, K, 2, 6, wg[2:6], wu[2:6], wd[2:6])
    u = moe.moe_layer(x, wr, None, K, 2, 6, wg[2:6], wu[2:6], wd[2:6])
    assert np.array_equal(r["topk_idx"], u["topk_idx"]) and np.array_equal(r["slot_row"], u["slot_row"])
    rms = np.sqrt(np.mean(u["out"] ** 2))
    err = np.sqrt(np.mean((r["out"] - u["out"]) ** 2))
    corr = np.corrcoef(r["out"].ravel(), u["out"].ravel())[0, 1]
    assert 0 < err < 0.15 * rms and corr > 0.98, (err, rms, corr)


ALL_MX_PINS = [
    pin_e4m3_table,
    pin_e4m3_encode_matches_torch,
    pin_e4m3_ties_and_saturation,
    pin_mx_scale_rule,
    pin_mx_round_trip_bound,
    pin_mx_dot_is_block_factored,
    pin_mx_layer_identical_experts_is_quantised_mlp,
    pin_mx_layer_close_to_unquantised,
]
