"""Planted mistakes in the oracle (on the CPU): each must make some pin fail.

This shows the pins are sensitive to the plausible slips named in each case;
the oracle itself is never changed on disk."""
import numpy as np
import pytest

import oracle.moe as O
import oracle_pins as P


def _fails(pin):
    try:
        pin(O)
    except AssertionError:
        return True
    return False


def test_wrong_silu_sign(monkeypatch):
    monkeypatch.setattr(O, "silu", lambda z: z / (1.0 + np.exp(z)))
    assert _fails(P.pin_identical_experts_is_dense_mlp) and _fails(P.pin_silu)


def test_gate_used_for_up(monkeypatch):
    def bad(xrows, wg, wu, wd):
        X = np.asarray(xrows, np.float64)
        g = X @ np.asarray(wg, np.float64)
        return (O.silu(g) * g) @ np.asarray(wd, np.float64)
    monkeypatch.setattr(O, "expert_ffn", bad)
    assert _fails(P.pin_dense_then_mask)


def test_ties_to_higher_index(monkeypatch):
    def bad(logits, K):
        l = np.asarray(logits, np.float64)[:, ::-1]
        E = l.shape[1]
        work = l.copy()
        idx = np.empty((l.shape[0], K), np.int32)
        for r in range(K):
            j = np.argmax(work, 1)
            idx[:, r] = E - 1 - j
            work[np.arange(l.shape[0]), j] = -np.inf
        return idx
    monkeypatch.setattr(O, "select_topk", bad)
    assert _fails(P.pin_topk_special_ties) and _fails(P.pin_topk_verifier_with_ties)


def test_weights_not_renormalised(monkeypatch):
    def bad(logits, idx):
        return np.take_along_axis(O.softmax(logits), idx.astype(np.int64), 1)
    monkeypatch.setattr(O, "topk_weights", bad)
    assert _fails(P.pin_weights) and _fails(P.pin_route_worked_example)


def test_logits_transposed_or_descending(monkeypatch):
    real = O.router_logits

    def descending(x, w, bias=None):
        return real(np.ascontiguousarray(np.asarray(x)[:, ::-1]), np.ascontiguousarray(np.asarray(w)[::-1]), bias)
    monkeypatch.setattr(O, "router_logits", descending)
    assert _fails(P.pin_logits_order_is_ascending_h)


def test_logits_without_fma(monkeypatch):
    def unfused(x, w, bias=None):
        x = np.asarray(x, np.float32)
        w = np.asarray(w, np.float32)
        acc = np.zeros((x.shape[0], w.shape[1]), np.float32)
        for h in range(x.shape[1]):
            acc = (acc + (x[:, h:h + 1] * w[h:h + 1, :]).astype(np.float32)).astype(np.float32)
        return acc if bias is None else (acc + np.asarray(bias, np.float32)).astype(np.float32)
    monkeypatch.setattr(O, "router_logits", unfused)
    assert _fails(P.pin_logits_fused_multiply_add)


def test_dropped_term_in_logits(monkeypatch):
    real = O.router_logits

    def dropped(x, w, bias=None):
        x = np.array(x, np.float32)
        x[:, -1] = 0
        return real(x, w, bias)
    monkeypatch.setattr(O, "router_logits", dropped)
    assert _fails(P.pin_logits_exact_on_integer_grid) and _fails(P.pin_logits_within_rigorous_bound)


def test_unstable_row_order(monkeypatch):
    real = O.dispatch

    def reversed_rows(idx, a, b):
        d = real(idx, a, b)
        rt, rs, sr = d["row_token"].copy(), d["row_slot"].copy(), d["slot_row"].copy()
        for i in range(b - a):
            s, e = int(d["offsets"][i]), int(d["offsets"][i + 1])
            rt[s:e], rs[s:e] = rt[s:e][::-1].copy(), rs[s:e][::-1].copy()
        sr[rt, rs] = np.arange(rt.size)
        return dict(d, row_token=rt, row_slot=rs, slot_row=sr)
    monkeypatch.setattr(O, "dispatch", reversed_rows)
    assert _fails(P.pin_dispatch_invariants_and_brute_force)


def test_combine_ignores_weights(monkeypatch):
    real = O.combine
    monkeypatch.setattr(O, "combine", lambda y, sr, w, T, H: real(y, sr, np.ones_like(w), T, H))
    assert _fails(P.pin_dense_then_mask) and _fails(P.pin_identical_experts_is_dense_mlp)


def test_local_range_off_by_one(monkeypatch):
    """The last local expert's pairs are left out of the packed buffers."""
    real = O.dispatch

    def short(idx, a, b):
        d = real(idx, a, b - 1)
        E_loc = b - a
        counts = np.concatenate([d["counts"], np.zeros(1, np.int32)])
        offsets = np.concatenate([d["offsets"], d["offsets"][-1:]])
        return dict(d, counts=counts[:E_loc], offsets=offsets[:E_loc + 1])
    monkeypatch.setattr(O, "dispatch", short)
    assert _fails(P.pin_shard_sum) and _fails(P.pin_dense_then_mask)
