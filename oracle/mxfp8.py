"""ORACLE -- test infrastructure, not part of the library.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the HIP path
and imports nothing from it.

MXFP8 expert GEMMs.  "Hosting Qwen on Blackwell" (Perplexity), section
"Quantification": the deployment quantises the model with the MXFP8
microscaling scheme, converting the weights statically once; microscaling is
what the hardware needs for its best prefill and decode throughput.  The
pages give no more detail, so the format is the Open Compute Project
Microscaling (MX) v1.0 definition of MXFP8 with E4M3 elements:

* a block is 32 consecutive elements along the reduction dimension K;
* each block shares one E8M0 scale X = 2^(e - 127), e in 0 .. 254;
* each element is an FP8 E4M3 value (1 sign, 4 exponent bits with bias 7, 3
  mantissa bits; no infinities; S.1111.111 is NaN; largest finite 448);
* conversion of a block (the spec's reference rule): shared exponent
  floor(log2(max |v|)) - 8 (8 is the exponent of E4M3's largest normal),
  clamped to [-127, 127], or -127 for an all-zero block; each element
  v / X rounded to the nearest E4M3 value, ties to the even code, magnitudes
  above 448 saturating to 448.

Readings taken where the pages are silent (both GEMM operands must be
microscaled for the scaled matrix instructions):

* expert weights are quantised per output column along K (H for gate/up, I
  for down), statically;
* the activations entering each GEMM are quantised per row along K: the token
  rows x per token, the SwiGLU activations h per packed row;
* the router keeps its unquantised inputs (it is not an expert GEMM);
* everything after dequantisation is float64, as in ``moe.py``.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Sequence

import numpy as np

from . import moe as _moe

BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8          # 448 = 1.75 * 2^8
E8M0_BIAS = 127


def e4m3_values() -> np.ndarray:
    """float64 value of each of the 256 E4M3 codes (NaN for 0x7F and 0xFF)."""
    c = np.arange(256, dtype=np.int64)
    sign = (c >> 7) & 1
    exp = (c >> 3) & 15
    man = c & 7
    mag = np.where(exp == 0, (man / 8.0) * 2.0 ** -6, (1.0 + man / 8.0) * 2.0 ** (exp - 7.0))
    v = np.where(sign == 1, -mag, mag)
    v[0x7F] = np.nan
    v[0xFF] = np.nan
    return v


def e4m3_encode(a: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each value, ties to the even code, magnitudes above
    448 saturating to 448; the sign bit follows the sign of the input (so a small
    negative value that rounds to zero gives -0, code 0x80).  uint8.

    Written from the format: a magnitude 2^E * (1 + k/8) with E >= -6 has code
    (E + 7) * 8 + k, so k is (m / 2^E - 1) * 8 rounded half to even (np.rint),
    carrying into the exponent when it reaches 8; below 2^-6 the values are
    k * 2^-9, k = m * 2^9 rounded half to even.  An even code is an even k."""
    a = np.asarray(a, dtype=np.float64)
    mag = np.minimum(np.abs(a), E4M3_MAX)
    _, e = np.frexp(mag)
    E = e.astype(np.int64) - 1                              # floor(log2 mag) for mag > 0
    normal = mag >= 2.0 ** -6
    Es = np.where(normal, E, 0)
    k = np.rint((mag / np.exp2(Es.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
    Es = np.where(k == 8, Es + 1, Es)
    k = np.where(k == 8, 0, k)
    code_normal = ((Es + 7) << 3) | k
    code_sub = np.rint(mag * 512.0).astype(np.int64)
    code = np.where(normal, code_normal, code_sub)
    sign = np.signbit(a).astype(np.int64)
    return ((sign << 7) | code).astype(np.uint8)


def shared_exponent(block_amax: np.ndarray) -> np.ndarray:
    """floor(log2(amax)) - 8, clamped to [-127, 127]; -127 where amax == 0 (int64)."""
    amax = np.asarray(block_amax, dtype=np.float64)
    _, e = np.frexp(amax)                      # amax = m * 2^e, 0.5 <= m < 1
    se = np.where(amax > 0, (e - 1) - E4M3_EMAX, -E8M0_BIAS)
    return np.clip(se, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def quantize(v: np.ndarray):
    """MXFP8 along the last axis (a multiple of 32): (codes uint8 same shape,
    scales uint8 [..., K/32] holding the biased E8M0 exponents)."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    if K % BLOCK:
        raise ValueError("the quantised axis must be a multiple of 32")
    blocks = v.reshape(v.shape[:-1] + (K // BLOCK, BLOCK))
    se = shared_exponent(np.abs(blocks).max(axis=-1))
    codes = e4m3_encode(blocks / np.exp2(se.astype(np.float64))[..., None])
    return codes.reshape(v.shape), (se + E8M0_BIAS).astype(np.uint8)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 values of MXFP8 data (codes [..., K], scales [..., K/32])."""
    codes = np.asarray(codes, dtype=np.uint8)
    K = codes.shape[-1]
    vals = e4m3_values()[codes].reshape(codes.shape[:-1] + (K // BLOCK, BLOCK))
    x = np.exp2(np.asarray(scales, dtype=np.float64) - E8M0_BIAS)
    return (vals * x[..., None]).reshape(codes.shape)


def fake_quant(v: np.ndarray, axis: int = -1) -> np.ndarray:
    """dequantize(quantize(v)) with the blocks running along `axis`."""
    v = np.moveaxis(np.asarray(v, dtype=np.float64), axis, -1)
    return np.moveaxis(dequantize(*quantize(v)), -1, axis)


def expert_ffn(xq: np.ndarray, w_gate, w_up, w_down) -> np.ndarray:
    """SwiGLU expert on MXFP8 operands.  xq: the expert's token rows, already
    quantised (dequantised values, float64).  Weights are quantised per output
    column along K; h is quantised per row before the down projection."""
    wg = fake_quant(w_gate, axis=0)
    wu = fake_quant(w_up, axis=0)
    wd = fake_quant(w_down, axis=0)
    h = _moe.silu(xq @ wg) * (xq @ wu)
    return fake_quant(h, axis=1) @ wd


def moe_layer(x, w_router, bias, K: int, e_begin: int, e_end: int,
              w_gate: Sequence, w_up: Sequence, w_down: Sequence) -> Dict[str, np.ndarray]:
    """The layer share of ``moe.moe_layer`` with MXFP8 expert GEMMs: routing and
    dispatch unchanged (from the unquantised x); each token row quantised once
    along H; combine unchanged."""
    x = np.asarray(x)
    T, H = x.shape
    idx, w, logits = _moe.route(x, w_router, bias, K)
    d = _moe.dispatch(idx, e_begin, e_end)
    xq = fake_quant(np.asarray(x, dtype=np.float64), axis=1)
    n = int(d["offsets"][-1])
    y = np.zeros((n, H), dtype=np.float64)

    def one(i):                      # experts are independent: run them on a thread pool
        a, b = int(d["offsets"][i]), int(d["offsets"][i + 1])
        if b > a:
            y[a:b] = expert_ffn(xq[d["row_token"][a:b]], w_gate[i], w_up[i], w_down[i])

    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        list(ex.map(one, range(e_end - e_begin)))
    out = _moe.combine(y, d["slot_row"], w, T, H)
    return dict(topk_idx=idx, topk_w=w, logits=logits, y_packed=y, out=out, **d)
