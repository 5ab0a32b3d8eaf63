"""ORACLE -- test infrastructure, not part of the library.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the HIP path
(``moe_layer_03_amd``) and imports nothing from it; it takes plain numpy
arrays (float32 or float64) and returns numpy arrays.

What it computes: one expert-parallel rank's share of a Mixture-of-Experts
layer, as "Hosting Qwen on Blackwell" (Perplexity) states the problem:

* route -- every token goes to K of E experts ("Pre-remplisseurs": 128
  experts, 8 per token, so 6000*8/128 = 375 tokens per expert on average);
* dispatch -- the inputs are replicated on every rank, so the rank selects
  the tokens routed to its own experts, gathers the routing information and
  packs those tokens into per-expert buffers that feed the expert GEMMs
  ("Expert Parallel"; "MoE Dispatch - Combine");
* expert GEMMs -- one matrix-multiply problem per local expert over its
  packed tokens ("MoE GEMM");
* combine -- a weighted accumulation of the local experts' outputs back to
  token order; the rank's result is the partial sum that the cross-rank
  all-reduce would add up ("Expert Parallel").

Readings where the pages are silent:

* router: softmax over all E experts, keep the K largest, renormalise them to
  sum to one;
* selection is taken on the float32 logits (softmax is strictly increasing,
  so it picks the same set); ties go to the lower expert index; slot order is
  descending logit; logits come from ``router_logits`` in its fixed order;
* expert FFN: SwiGLU, ``y = (silu(x Wg) * (x Wu)) Wd`` with
  ``silu(z) = z / (1 + exp(-z))``; no shared expert, no FFN biases, no token
  dropping (no capacity limit);
* packed rows of one expert are in ascending token order; experts in
  ascending index; the rank's output row is exactly zero for a token with no
  local expert;
* precision: everything after the logits is float64.

Parity pins for each function live in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Iterable, Optional, Sequence

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.ensure_built()
        lib = ctypes.CDLL(path)
        lib.oracle_router_logits.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_router_logits.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the oracle's C part runs on (OpenMP)."""
    return int(_load().oracle_num_threads())


# ---------------------------------------------------------------------------
# Route ("Pre-remplisseurs": 8 of 128 experts per token)
# ---------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """l[t,e] = sum_h x[t,h] W[h,e] (+ b[e]), float32, one fmaf per term, h ascending.

    x [T,H] and W [H,E] are taken as float32 (bf16 inputs widen exactly)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w_router, dtype=np.float32)
    T, H = x.shape
    H2, E = w.shape
    if H2 != H:
        raise ValueError("x and router weight disagree on H")
    out = np.empty((T, E), dtype=np.float32)
    b_ptr = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.shape != (E,):
            raise ValueError("bias must be [E]")
        b_ptr = bias.ctypes.data
    if T > 0:
        _load().oracle_router_logits(x.ctypes.data, w.ctypes.data, b_ptr, T, H, E, out.ctypes.data)
    return out


def select_topk(logits: np.ndarray, K: int) -> np.ndarray:
    """K rounds of argmax over the experts not chosen yet.

    The largest logit wins; among equal logits (float ==, so -0 equals +0) the
    lower expert index wins (np.argmax returns the first maximum).  Slot 0
    holds the largest logit.  Returns int32 [T, K]."""
    T, E = logits.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    work = np.array(logits, dtype=np.float64)   # exact widening, same order and ties
    idx = np.empty((T, K), dtype=np.int32)
    rows = np.arange(T)
    for r in range(K):
        j = np.argmax(work, axis=1)
        idx[:, r] = j
        work[rows, j] = -np.inf
    return idx


def softmax(logits: np.ndarray) -> np.ndarray:
    """Softmax over the experts of each token, float64."""
    l = np.asarray(logits, dtype=np.float64)
    m = l.max(axis=1, keepdims=True)
    ex = np.exp(l - m)
    return ex / ex.sum(axis=1, keepdims=True)


def topk_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax over all experts, then the chosen K probabilities renormalised to sum to 1."""
    p = softmax(logits)
    pk = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    return pk / pk.sum(axis=1, keepdims=True)


def route(x, w_router, bias, K):
    """(topk_idx int32 [T,K], topk_w float64 [T,K], logits float32 [T,E])."""
    l = router_logits(x, w_router, bias)
    idx = select_topk(l, K)
    return idx, topk_weights(l, idx), l


# ---------------------------------------------------------------------------
# Dispatch ("Expert Parallel": select the local tokens, pack them per expert)
# ---------------------------------------------------------------------------

def dispatch(topk_idx: np.ndarray, e_begin: int, e_end: int) -> Dict[str, np.ndarray]:
    """Group the (token, slot) pairs routed to experts [e_begin, e_end).

    counts[i]   pairs routed to expert e_begin+i
    offsets     exclusive prefix sum of counts, offsets[E_loc] = N_loc
    row_token   token of packed row r; rows of one expert in ascending token order
    row_slot    slot j of packed row r
    slot_row    [T,K] packed row of (t, j), -1 when expert topk_idx[t,j] is not local
    """
    T, K = topk_idx.shape
    E_loc = e_end - e_begin
    counts = np.zeros(E_loc, dtype=np.int32)
    offsets = np.zeros(E_loc + 1, dtype=np.int32)
    slot_row = np.full((T, K), -1, dtype=np.int32)
    tok_parts, slot_parts = [], []
    for i in range(E_loc):
        # np.nonzero walks the array in row-major order: ascending token.
        ts, js = np.nonzero(topk_idx == e_begin + i)
        counts[i] = ts.size
        offsets[i + 1] = offsets[i] + ts.size
        slot_row[ts, js] = offsets[i] + np.arange(ts.size, dtype=np.int32)
        tok_parts.append(ts.astype(np.int32))
        slot_parts.append(js.astype(np.int32))
    row_token = np.concatenate(tok_parts) if tok_parts else np.zeros(0, np.int32)
    row_slot = np.concatenate(slot_parts) if slot_parts else np.zeros(0, np.int32)
    return dict(counts=counts, offsets=offsets, row_token=row_token.astype(np.int32),
                row_slot=row_slot.astype(np.int32), slot_row=slot_row)


def pack(x: np.ndarray, row_token: np.ndarray) -> np.ndarray:
    """x_packed[r] = x[row_token[r]] (float64)."""
    return np.asarray(x, dtype=np.float64)[row_token]


# ---------------------------------------------------------------------------
# Expert FFN ("MoE GEMM")
# ---------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_ffn(xrows: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """SwiGLU expert: (silu(X Wg) * (X Wu)) Wd, float64.  X [n,H], Wg/Wu [H,I], Wd [I,H]."""
    X = np.asarray(xrows, dtype=np.float64)
    g = X @ np.asarray(w_gate, dtype=np.float64)
    u = X @ np.asarray(w_up, dtype=np.float64)
    h = silu(g) * u
    return h @ np.asarray(w_down, dtype=np.float64)


# ---------------------------------------------------------------------------
# Combine ("MoE Dispatch - Combine", "Expert Parallel": local weighted accumulation)
# ---------------------------------------------------------------------------

def combine(y_packed: np.ndarray, slot_row: np.ndarray, topk_w: np.ndarray, T: int, H: int) -> np.ndarray:
    """out[t] = sum over local slots j (ascending) of topk_w[t,j] * y_packed[slot_row[t,j]]; float64 [T,H].

    Tokens with no local slot get an all-zero row."""
    out = np.zeros((T, H), dtype=np.float64)
    K = slot_row.shape[1]
    for j in range(K):
        sel = np.nonzero(slot_row[:, j] >= 0)[0]
        if sel.size:
            out[sel] += np.asarray(topk_w, dtype=np.float64)[sel, j, None] * y_packed[slot_row[sel, j]]
    return out


# ---------------------------------------------------------------------------
# The layer share
# ---------------------------------------------------------------------------

def moe_layer(x, w_router, bias, K: int, e_begin: int, e_end: int,
              w_gate: Sequence, w_up: Sequence, w_down: Sequence) -> Dict[str, np.ndarray]:
    """Route, dispatch, expert FFN per local expert, combine.

    w_gate[i], w_up[i], w_down[i] are the matrices of expert e_begin+i (any
    indexable of 2-D arrays).  Returns routing, dispatch and ``out`` [T,H] float64."""
    x = np.asarray(x)
    T, H = x.shape
    idx, w, logits = route(x, w_router, bias, K)
    d = dispatch(idx, e_begin, e_end)
    n = int(d["offsets"][-1])
    y = np.zeros((n, H), dtype=np.float64)
    for i in range(e_end - e_begin):
        a, b = int(d["offsets"][i]), int(d["offsets"][i + 1])
        if b > a:
            y[a:b] = expert_ffn(pack(x, d["row_token"][a:b]), w_gate[i], w_up[i], w_down[i])
    out = combine(y, d["slot_row"], w, T, H)
    return dict(topk_idx=idx, topk_w=w, logits=logits, y_packed=y, out=out, **d)


def moe_layer_rows(x, topk_w: np.ndarray, slot_row: np.ndarray, topk_idx: np.ndarray,
                   e_begin: int, tokens: Iterable[int],
                   w_gate: Sequence, w_up: Sequence, w_down: Sequence) -> np.ndarray:
    """``out`` rows for the listed tokens only, from routing computed beforehand.

    Same definition as ``moe_layer`` restricted to a sample of tokens, for
    workloads whose full expert FFN is too slow on the CPU.  float64 [n,H]."""
    x = np.asarray(x)
    tokens = np.asarray(list(tokens), dtype=np.int64)
    H = x.shape[1]
    K = slot_row.shape[1]
    out = np.zeros((tokens.size, H), dtype=np.float64)
    # group (sample position, slot) pairs by local expert
    by_expert: Dict[int, list] = {}
    for p, t in enumerate(tokens):
        for j in range(K):
            if slot_row[t, j] >= 0:
                by_expert.setdefault(int(topk_idx[t, j]) - e_begin, []).append((p, j))
    ys = {}
    for i, pairs in by_expert.items():
        rows = np.array([tokens[p] for p, _ in pairs], dtype=np.int64)
        y = expert_ffn(np.asarray(x[rows], dtype=np.float64), w_gate[i], w_up[i], w_down[i])
        for (p, j), yrow in zip(pairs, y):
            ys[(p, j)] = yrow
    for p, t in enumerate(tokens):
        for j in range(K):          # ascending slot order, as in combine()
            if slot_row[t, j] >= 0:
                out[p] += float(topk_w[t, j]) * ys[(p, j)]
    return out
