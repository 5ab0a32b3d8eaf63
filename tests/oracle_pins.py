"""Pins of the oracle against facts fixed by the pages and by mathematics.

Each ``pin_*`` function raises AssertionError when the oracle module ``O``
(normally ``oracle.moe``) disagrees with something that does not come from
the oracle itself: a number printed in "Hosting Qwen on Blackwell", a closed
form, an exact integer computation, a library routine a special case reduces
to (torch CPU), a brute force, or an invariant.  ``test_oracle.py`` runs them
on the oracle; ``test_oracle_mutations.py`` plants mistakes in the oracle and
checks that some pin fails.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    return [dict(kv.split("=") for kv in ln.split()) for ln in lines]


def _grid(rng, shape, lo=-4, hi=4, scale=16):
    """Values k/scale, k integer in [lo, hi]: exact in bf16 and fp32; also returns the integers."""
    k = rng.integers(lo, hi + 1, size=shape)
    return (k / scale).astype(np.float32), k.astype(np.int64)


# ---------------------------------------------------------------------------
# router logits
# ---------------------------------------------------------------------------

def pin_logits_exact_on_integer_grid(O):
    """Products and every partial sum are exact in fp32 on a 1/256 grid: the
    result must equal the integer matrix product (non-square, H != E)."""
    rng = np.random.default_rng(11)
    x, xi = _grid(rng, (7, 64))
    w, wi = _grid(rng, (64, 5))
    exact = (xi @ wi).astype(np.float64) / 256.0
    got = O.router_logits(x, w)
    assert got.dtype == np.float32 and got.shape == (7, 5)
    assert np.array_equal(got.astype(np.float64), exact), "logits differ from the exact integer product"
    b, bi = _grid(rng, (5,), -64, 64, 256)
    got_b = O.router_logits(x, w, b)
    assert np.array_equal(got_b.astype(np.float64), exact + bi / 256.0), "bias not added once per expert"


def pin_logits_order_is_ascending_h(O):
    """Sequential fp32 order, h ascending: 1 + 2^-24 + 2^-24 stays 1 (each add is
    a tie to even), while 2^-24 + 2^-24 + 1 gives 1 + 2^-23."""
    tiny = np.float32(2.0 ** -24)
    w = np.ones((3, 1), dtype=np.float32)
    a = O.router_logits(np.array([[1.0, tiny, tiny]], dtype=np.float32), w)[0, 0]
    b = O.router_logits(np.array([[tiny, tiny, 1.0]], dtype=np.float32), w)[0, 0]
    assert a == np.float32(1.0), f"ascending-h order must give exactly 1.0, got {a!r}"
    assert b == np.float32(1.0 + 2.0 ** -23), f"got {b!r}"


def pin_logits_fused_multiply_add(O):
    """One rounding per term: with a = b = 1 + 2^-12, a*b - 1 = 2^-11 + 2^-24
    exactly under a fused multiply-add (a separate multiply would round the
    2^-24 away)."""
    a = np.float32(1.0 + 2.0 ** -12)
    x = np.array([[1.0, a]], dtype=np.float32)
    w = np.array([[-1.0], [a]], dtype=np.float32)
    got = O.router_logits(x, w)[0, 0]
    assert got == np.float32(2.0 ** -11 + 2.0 ** -24), f"got {got!r}"


def pin_logits_within_rigorous_bound(O):
    """General fp32 inputs: |l - S| <= gamma_H * sum|x w| + |b| u, with S the
    exact sum (fp64 matmul, error far below the bound) -- a sum of the right
    products in some order (a missing or misplaced term breaks the bound)."""
    rng = np.random.default_rng(12)
    T, H, E = 16, 512, 48
    x = rng.standard_normal((T, H)).astype(np.float32)
    w = (rng.standard_normal((H, E)) * 0.02).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    u = 2.0 ** -24
    gamma = H * u / (1 - H * u)
    S = x.astype(np.float64) @ w.astype(np.float64)
    A = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64))
    l = O.router_logits(x, w).astype(np.float64)
    assert np.all(np.abs(l - S) <= gamma * A + 1e-12), "logits outside the summation error bound"
    lb = O.router_logits(x, w, b).astype(np.float64)
    assert np.all(np.abs(lb - (S + b)) <= gamma * A + 2 * u * (np.abs(S) + np.abs(b) + gamma * A) + 1e-12)
    # bound is tight enough to see a single dropped term
    assert np.median(np.abs(x[:, :1] * w[:1, :]) / (gamma * A[:, :])) > 1.0


# ---------------------------------------------------------------------------
# selection and weights
# ---------------------------------------------------------------------------

def _key_beats(l, a, b):
    """(logit descending, index ascending) order: does expert a come before b."""
    return l[a] > l[b] or (l[a] == l[b] and a < b)


def verify_topk(logits, idx, K):
    """Brute-force verifier (not a second implementation): every chosen expert
    beats every unchosen one and slots are sorted by the same key."""
    T, E = logits.shape
    for t in range(T):
        l = logits[t]
        s = [int(v) for v in idx[t]]
        assert len(set(s)) == K and all(0 <= v < E for v in s)
        rest = set(range(E)) - set(s)
        for j in range(K - 1):
            assert _key_beats(l, s[j], s[j + 1]), f"token {t}: slots not ordered"
        last = s[-1]
        for v in rest:
            assert _key_beats(l, last, v), f"token {t}: unchosen {v} beats chosen {last}"


def pin_topk_verifier_with_ties(O):
    rng = np.random.default_rng(13)
    T, E, K = 120, 128, 8
    # coarse grid -> many exact ties among the top logits
    logits = (np.round(rng.standard_normal((T, E)) * 4) / 4).astype(np.float32)
    idx = O.select_topk(logits, K)
    verify_topk(logits, idx, K)
    logits2 = rng.standard_normal((T, E)).astype(np.float32)
    verify_topk(logits2, O.select_topk(logits2, K), K)


def pin_topk_special_ties(O):
    z = np.zeros((3, 10), dtype=np.float32)
    assert np.array_equal(O.select_topk(z, 4), np.tile(np.arange(4), (3, 1))), "all-equal: lowest indices"
    nz = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], dtype=np.float32)
    assert O.select_topk(nz, 1)[:, 0].tolist() == [0, 0], "-0 and +0 compare equal; lower index wins"
    dup = np.array([[0.5, 2.0, 1.0, 2.0, 1.0]], dtype=np.float32)
    assert O.select_topk(dup, 4)[0].tolist() == [1, 3, 2, 4]


def pin_route_worked_example(O):
    """x=[1], W=[[1,2,3,4]], K=2: experts 3 then 2; weights are the two-way
    softmax of (4, 3): 1/(1+e^-1) and 1/(1+e)."""
    idx, w, l = O.route(np.array([[1.0]], np.float32), np.array([[1.0, 2.0, 3.0, 4.0]], np.float32), None, 2)
    assert idx.tolist() == [[3, 2]]
    assert abs(w[0, 0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(w[0, 1] - 1.0 / (1.0 + math.e)) < 1e-15


def pin_weights(O):
    rng = np.random.default_rng(14)
    T, E = 50, 16
    l = (rng.standard_normal((T, E)) * 1.3).astype(np.float32)
    for K in (1, 3, 8):
        idx = O.select_topk(l, K)
        w = O.topk_weights(l, idx)
        assert np.all(np.abs(w.sum(axis=1) - 1.0) < 1e-12), "weights must sum to 1"
        assert np.all(np.diff(w, axis=1) <= 0), "weights descend with the slot"
        if K == 1:
            assert np.all(w == 1.0)
    # K = E: renormalisation over everything is the plain softmax (library routine)
    idx = O.select_topk(l, E)
    w = O.topk_weights(l, idx)
    ref = torch.softmax(torch.from_numpy(l.astype(np.float64)), dim=1).numpy()
    assert np.allclose(w, np.take_along_axis(ref, idx.astype(np.int64), 1), rtol=0, atol=1e-14)
    # zero router weight: every logit is 0, experts 0..K-1, weights exactly 1/K
    K = 4
    i0, w0, _ = O.route(rng.standard_normal((5, 32)).astype(np.float32), np.zeros((32, 16), np.float32), None, K)
    assert np.array_equal(i0, np.tile(np.arange(K), (5, 1))) and np.all(w0 == 1.0 / K)
    # a constant added to every logit changes neither selection nor weights
    x, _ = _grid(rng, (9, 64))
    wr, _ = _grid(rng, (64, 16))
    i1, w1, _ = O.route(x, wr, None, 4)
    i2, w2, _ = O.route(x, wr, np.full(16, 0.5, np.float32), 4)
    assert np.array_equal(i1, i2) and np.allclose(w1, w2, rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------

def pin_pages_tokens_per_expert(O):
    """The pages' worked number: 6000 tokens, 8 of 128 experts each -> on
    average 375 tokens per expert; the counts over all experts sum to T*K."""
    g = read_golden("pages_tokens_per_expert.txt")[0]
    T, K, E, mean = int(g["T"]), int(g["K"]), int(g["E"]), int(g["mean_tokens_per_expert"])
    rng = np.random.default_rng(15)
    x = rng.standard_normal((T, 64)).astype(np.float32)
    w = (rng.standard_normal((64, E)) * 0.1).astype(np.float32)
    idx, _, _ = O.route(x, w, None, K)
    d = O.dispatch(idx, 0, E)
    assert int(d["counts"].sum()) == T * K == int(d["offsets"][-1])
    assert d["counts"].sum() / E == mean


def verify_dispatch(idx, d, e_begin, e_end):
    T, K = idx.shape
    E_loc = e_end - e_begin
    counts, offsets = d["counts"], d["offsets"]
    rt, rs, sr = d["row_token"], d["row_slot"], d["slot_row"]
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    n = int(offsets[-1])
    assert rt.shape == (n,) and rs.shape == (n,)
    local = (idx >= e_begin) & (idx < e_end)
    assert n == int(local.sum())
    for i in range(E_loc):
        a, b = int(offsets[i]), int(offsets[i + 1])
        assert np.all(idx[rt[a:b], rs[a:b]] == e_begin + i), "row in the wrong segment"
        assert np.all(np.diff(rt[a:b]) > 0), "segment not in ascending token order"
    # slot_row is the inverse of (row_token, row_slot), -1 exactly on non-local slots
    assert np.all((sr >= 0) == local)
    assert np.array_equal(sr[rt, rs], np.arange(n))
    seen = np.zeros(n, dtype=np.int64)
    np.add.at(seen, sr[local], 1)
    assert np.all(seen == 1), "not a bijection"


def pin_dispatch_invariants_and_brute_force(O):
    rng = np.random.default_rng(16)
    T, E, K = 300, 32, 4
    l = rng.standard_normal((T, E)).astype(np.float32)
    idx = O.select_topk(l, K)
    for (a, b) in ((0, E), (8, 16), (5, 6), (31, 32)):
        d = O.dispatch(idx, a, b)
        verify_dispatch(idx, d, a, b)
        # brute force: row = start of the expert's segment + earlier tokens routed to it
        for t in range(0, T, 7):
            for j in range(K):
                e = int(idx[t, j])
                if a <= e < b:
                    before = sum(1 for tt in range(t) if e in idx[tt])
                    start = sum(1 for tt in range(T) for ee in idx[tt] if a <= ee < e)
                    assert d["slot_row"][t, j] == start + before
    # four disjoint shards partition the whole layer's pairs
    shards = [O.dispatch(idx, 8 * s, 8 * s + 8) for s in range(4)]
    whole = O.dispatch(idx, 0, E)
    assert np.array_equal(np.concatenate([s["counts"] for s in shards]), whole["counts"])
    owners = sum((s["slot_row"] >= 0).astype(int) for s in shards)
    assert np.all(owners == 1)


# ---------------------------------------------------------------------------
# expert FFN and the whole share
# ---------------------------------------------------------------------------

def _torch_mlp(x, wg, wu, wd):
    X = torch.from_numpy(np.asarray(x, np.float64))
    g = X @ torch.from_numpy(np.asarray(wg, np.float64))
    u = X @ torch.from_numpy(np.asarray(wu, np.float64))
    return (F.silu(g) * u) @ torch.from_numpy(np.asarray(wd, np.float64))


def pin_silu(O):
    z = np.array([-50.0, -1.0, 0.0, 0.5, 3.0, 40.0])
    ref = F.silu(torch.from_numpy(z)).numpy()
    assert np.allclose(O.silu(z), ref, rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0


def _small_layer(rng, T=40, H=64, E=8, K=3, I=32, std=0.3):
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((H, E)) * std).astype(np.float32)
    wg = (rng.standard_normal((E, H, I)) * std).astype(np.float32)
    wu = (rng.standard_normal((E, H, I)) * std).astype(np.float32)
    wd = (rng.standard_normal((E, I, H)) * std).astype(np.float32)
    return x, wr, wg, wu, wd


def pin_identical_experts_is_dense_mlp(O):
    """All experts equal: the whole layer is one dense SwiGLU MLP (weights sum
    to one); a shard returns that MLP scaled by its local weight mass."""
    rng = np.random.default_rng(17)
    x, wr, wg, wu, wd = _small_layer(rng)
    E, K = wr.shape[1], 3
    g = np.repeat(wg[:1], E, 0)
    u = np.repeat(wu[:1], E, 0)
    d = np.repeat(wd[:1], E, 0)
    ref = _torch_mlp(x, wg[0], wu[0], wd[0]).numpy()
    r = O.moe_layer(x, wr, None, K, 0, E, g, u, d)
    assert np.allclose(r["out"], ref, rtol=1e-10, atol=1e-12), "identical experts != dense MLP"
    a, b = 2, 5
    rs = O.moe_layer(x, wr, None, K, a, b, g[a:b], u[a:b], d[a:b])
    mass = np.where((rs["topk_idx"] >= a) & (rs["topk_idx"] < b), rs["topk_w"], 0.0).sum(1)
    assert np.allclose(rs["out"], mass[:, None] * ref, rtol=1e-10, atol=1e-12)


def pin_dense_then_mask(O):
    """Brute force by another algorithm: run every expert on every token, then
    mix with the dense gate matrix G (softmax -> top-K -> renormalise, built
    with torch), via einsum; keep only local experts."""
    rng = np.random.default_rng(18)
    x, wr, wg, wu, wd = _small_layer(rng, T=64, H=256 // 4, E=8, K=2, I=32)
    E, K = 8, 2
    l = O.router_logits(x, wr)     # logits are pinned separately above
    p = torch.softmax(torch.from_numpy(l.astype(np.float64)), dim=1)
    vals, ids = torch.topk(p, K, dim=1)   # random logits: no ties
    G = torch.zeros_like(p).scatter_(1, ids, vals / vals.sum(1, keepdim=True))
    Y = torch.stack([_torch_mlp(x, wg[e], wu[e], wd[e]) for e in range(E)])    # [E,T,H]
    for (a, b) in ((0, E), (2, 5), (7, 8)):
        mask = torch.zeros(E, dtype=torch.float64)
        mask[a:b] = 1
        ref = torch.einsum("te,eth->th", G * mask, Y).numpy()
        r = O.moe_layer(x, wr, None, K, a, b, wg[a:b], wu[a:b], wd[a:b])
        assert np.allclose(r["out"], ref, rtol=1e-10, atol=1e-12), f"shard [{a},{b})"
        assert np.all(r["out"][(r["slot_row"] < 0).all(1)] == 0.0), "tokens with no local expert must be 0"


def pin_shard_sum(O):
    """Expert-parallel partition: the four shards' partial outputs add up to
    the whole layer's output (the sum the cross-rank all-reduce would form)."""
    rng = np.random.default_rng(19)
    x, wr, wg, wu, wd = _small_layer(rng, T=50, H=32, E=16, K=4, I=16)
    whole = O.moe_layer(x, wr, None, 4, 0, 16, wg, wu, wd)["out"]
    acc = np.zeros_like(whole)
    for s in range(4):
        a, b = 4 * s, 4 * s + 4
        acc += O.moe_layer(x, wr, None, 4, a, b, wg[a:b], wu[a:b], wd[a:b])["out"]
    assert np.allclose(acc, whole, rtol=1e-12, atol=1e-14)


def pin_combine_exact(O):
    """Integer rows and unit weights: combine is an exact integer sum."""
    rng = np.random.default_rng(20)
    T, K, H = 10, 3, 6
    slot_row = np.full((T, K), -1, np.int32)
    flat = slot_row.reshape(-1)
    flat[rng.choice(T * K, 17, replace=False)] = np.arange(17)
    y = rng.integers(-50, 50, size=(17, H)).astype(np.float64)
    out = O.combine(y, slot_row, np.ones((T, K)), T, H)
    for t in range(T):
        ref = sum((y[r] for r in slot_row[t] if r >= 0), np.zeros(H))
        assert np.array_equal(out[t], ref)


def pin_sampled_rows_match_full(O):
    """``moe_layer_rows`` is the same definition restricted to some tokens."""
    rng = np.random.default_rng(21)
    x, wr, wg, wu, wd = _small_layer(rng, T=30, H=32, E=8, K=3, I=16)
    r = O.moe_layer(x, wr, None, 3, 2, 6, wg[2:6], wu[2:6], wd[2:6])
    toks = [0, 5, 7, 29]
    rows = O.moe_layer_rows(x, r["topk_w"], r["slot_row"], r["topk_idx"], 2, toks, wg[2:6], wu[2:6], wd[2:6])
    assert np.allclose(rows, r["out"][toks], rtol=1e-13, atol=1e-15)


ALL_PINS = [
    pin_logits_exact_on_integer_grid,
    pin_logits_order_is_ascending_h,
    pin_logits_fused_multiply_add,
    pin_logits_within_rigorous_bound,
    pin_topk_verifier_with_ties,
    pin_topk_special_ties,
    pin_route_worked_example,
    pin_weights,
    pin_pages_tokens_per_expert,
    pin_dispatch_invariants_and_brute_force,
    pin_silu,
    pin_identical_experts_is_dense_mlp,
    pin_dense_then_mask,
    pin_shard_sum,
    pin_combine_exact,
    pin_sampled_rows_match_full,
]
