"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: the pages'
worked examples (``tests/golden``), brute force on tiny inputs, closed forms,
identities, and special cases that reduce to a library routine. CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- top-K ids
def _topk_bruteforce(row, K):
    """Rank by counting beaters: e' beats e iff l[e'] > l[e] or (equal and e' < e)."""
    N = len(row)
    out = [None] * K
    for e in range(N):
        beaters = sum(1 for e2 in range(N)
                      if row[e2] > row[e] or (row[e2] == row[e] and e2 < e))
        if beaters < K:
            out[beaters] = e
    return out


@pytest.mark.parametrize("seed", range(6))
def test_topk_ids_bruteforce_with_ties(seed):
    rng = np.random.default_rng(seed)
    T, N = 40, 7
    # a small value set forces ties; include signed zeros
    vals = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 2.0, 3.0], dtype=np.float32)
    L = rng.choice(vals, size=(T, N)).astype(np.float32)
    for K in range(1, N + 1):
        idx, _ = orc.topk_softmax(L, K)
        for t in range(T):
            assert list(idx[t]) == _topk_bruteforce(L[t], K)


def test_topk_k1_is_argmax_first_max():
    rng = np.random.default_rng(0)
    L = rng.integers(-3, 3, size=(200, 9)).astype(np.float32)
    idx, w = orc.topk_softmax(L, 1)
    assert np.array_equal(idx[:, 0], np.argmax(L, axis=1))
    assert np.all(w == 1.0)


def test_topk_constant_logits_gives_lowest_ids():
    L = np.full((5, 6), 0.3, dtype=np.float32)
    idx, w = orc.topk_softmax(L, 4)
    assert np.array_equal(idx, np.tile(np.arange(4), (5, 1)))
    assert np.allclose(w, 0.25, rtol=0, atol=1e-7)


def test_topk_signed_zero_tie_falls_back_to_id():
    L = np.array([[0.0, -0.0, -1.0], [-0.0, 0.0, -1.0]], dtype=np.float32)
    idx, _ = orc.topk_softmax(L, 2)
    assert idx.tolist() == [[0, 1], [0, 1]]


def _beats_nan_last(a, ia, b, ib):
    """a (expert ia) ranks ahead of b (expert ib): numbers by value (IEEE
    comparison, so -0.0 == +0.0 and -inf is the smallest), NaN after every
    number, ties (NaN with NaN included) by the lower id."""
    na, nb = math.isnan(a), math.isnan(b)
    if na or nb:
        return (nb and not na) or (na and nb and ia < ib)
    return a > b or (a == b and ia < ib)


@pytest.mark.parametrize("seed", range(4))
def test_topk_nonfinite_logits_rank_nan_last(seed):
    rng = np.random.default_rng(100 + seed)
    T, N = 60, 9
    vals = np.array([np.nan, -np.inf, np.inf, -0.0, 0.0, -1.0, 1.0, 2.5], dtype=np.float32)
    L = rng.choice(vals, size=(T, N)).astype(np.float32)
    L[0] = np.nan
    L[1] = -np.inf
    for K in (1, 3, N):
        with np.errstate(invalid="ignore"):   # inf - inf in the weights of such rows
            idx, _ = orc.topk_softmax(L, K)
        for t in range(T):
            row = [float(v) for v in L[t]]
            ranks = [sum(1 for e2 in range(N) if _beats_nan_last(row[e2], e2, row[e], e))
                     for e in range(N)]
            expect = sorted(range(N), key=lambda e: ranks[e])[:K]
            assert list(idx[t]) == expect


def test_topk_full_k_is_a_sorted_permutation():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((30, 11)).astype(np.float32)
    idx, _ = orc.topk_softmax(L, 11)
    for t in range(30):
        assert sorted(idx[t]) == list(range(11))
        assert np.all(np.diff(L[t, idx[t]]) <= 0)


# ---------------------------------------------------------------- weights
def test_weights_reproduce_fig15():
    g = _load("fig15_router.json")
    ids = np.array(g["ids"])
    wts = np.array(g["weights"])
    T, K = ids.shape
    L = np.full((T, g["N"]), -30.0)
    for t in range(T):
        for k in range(K):
            L[t, ids[t, k]] = math.log(wts[t, k])
    idx, w = orc.topk_softmax(L.astype(np.float32), K)
    assert np.array_equal(idx, ids)
    # exact up to the fp32 rounding of ln(w) and of the result
    assert np.allclose(w, wts, rtol=0, atol=3e-7)


def test_weights_equal_full_softmax_renormalised():
    from scipy.special import softmax
    rng = np.random.default_rng(7)
    L = (rng.standard_normal((100, 16)) * 3).astype(np.float32)
    for K in (1, 2, 5, 16):
        idx, w = orc.topk_softmax(L, K)
        full = softmax(L.astype(np.float64), axis=1)
        sel = np.take_along_axis(full, idx.astype(np.int64), axis=1)
        ref = sel / sel.sum(axis=1, keepdims=True)
        assert np.allclose(w, ref, rtol=2e-7, atol=0)


def test_weights_sum_to_one_and_shift_invariant():
    rng = np.random.default_rng(8)
    L = (rng.standard_normal((64, 32)) * 2).astype(np.float32)
    _, w = orc.topk_softmax(L, 8)
    assert np.allclose(w.astype(np.float64).sum(axis=1), 1.0, atol=1e-6)
    # a shift by a power of two is exact in fp32 for these magnitudes
    _, w2 = orc.topk_softmax(L + np.float32(4.0), 8)
    assert np.allclose(w, w2, rtol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)


# ---------------------------------------------------------------- route map
def test_route_map_reproduces_fig16():
    g = _load("fig16_route_map.json")
    ids = np.array(g["ids"], dtype=np.int32)
    for C in (g["capacity_min"], 8, 100):
        rm = orc.route_map(ids, g["N"], g["ep_size"], C, ep_rank=0)
        assert rm["dest_rank"].tolist() == g["dest_rank"]
        assert rm["dest_row"].tolist() == g["dest_row"]
        assert rm["offsets"][0, -1] == g["rank0_rows_used"]
        assert rm["drop_mask"].sum() == 0       # E->1 is invalid, not dropped
    rm = orc.route_map(ids, g["N"], g["ep_size"], 7, ep_rank=1)
    # rank 1's inverse map: rows 0..6 hold A,E,F,J (expert 2) then C,H,I (expert 3)
    assert rm["row_src"][:7].tolist() == [0 * 2 + 1, 4 * 2 + 1, 5 * 2 + 0, 9 * 2 + 1,
                                          2 * 2 + 0, 7 * 2 + 0, 8 * 2 + 1]
    assert np.all(rm["row_src"][7:] == -1)


def _positions_bruteforce(ids):
    """p(t, k) = number of earlier tokens t' < t that route to the same expert."""
    T, K = ids.shape
    p = np.full((T, K), -1)
    for t in range(T):
        for k in range(K):
            e = ids[t, k]
            if e >= 0:
                p[t, k] = int(np.sum(np.any(ids[:t] == e, axis=1)))
    return p


def _check_route_invariants(ids, N, ep_size, C, rm):
    T, K = ids.shape
    E_L = N // ep_size
    p = _positions_bruteforce(ids)
    valid = ids >= 0
    kept = valid & (p < C)
    dropped = valid & (p >= C)
    assert np.array_equal(rm["drop_mask"].astype(bool), dropped)
    assert np.array_equal(rm["dest_rank"] >= 0, kept)
    assert np.array_equal(rm["dest_row"] >= 0, kept)
    counts = np.bincount(ids[valid], minlength=N)
    assert np.array_equal(rm["counts"], counts)
    keptc = np.minimum(counts, C)
    assert keptc.sum() == T * K - dropped.sum() - (~valid).sum()
    for r in range(ep_size):
        off = rm["offsets"][r]
        assert off[0] == 0
        assert np.array_equal(np.diff(off), keptc[r * E_L:(r + 1) * E_L])
    # destination rows: unique per rank, inside the expert interval, increasing in t
    for r in range(ep_size):
        rows = rm["dest_row"][rm["dest_rank"] == r]
        assert len(set(rows.tolist())) == len(rows)
    for t in range(T):
        for k in range(K):
            if kept[t, k]:
                e = ids[t, k]
                r, j = divmod(int(e), E_L)
                assert rm["dest_rank"][t, k] == r
                assert rm["dest_row"][t, k] == rm["offsets"][r, j] + p[t, k]


def test_route_map_exhaustive_tiny():
    """Every id pattern with T=3, N=3, K in {1,2}, including invalid (-1) entries."""
    for K in (1, 2):
        rows = [r for r in itertools.product(range(-1, 3), repeat=K)
                if len({x for x in r if x >= 0}) == sum(1 for x in r if x >= 0)]
        for pattern in itertools.product(rows, repeat=3):
            ids = np.array(pattern, dtype=np.int32).reshape(3, K)
            for C in (1, 2, 3):
                for ep_size in (1, 3):
                    rm = orc.route_map(ids, 3, ep_size, C, ep_rank=0)
                    _check_route_invariants(ids, 3, ep_size, C, rm)


@pytest.mark.parametrize("seed", range(4))
def test_route_map_random_with_drops(seed):
    rng = np.random.default_rng(seed)
    T, N, K = 50, 8, 3
    ids = np.stack([rng.permutation(N)[:K] for _ in range(T)]).astype(np.int32)
    ids[rng.random((T, K)) < 0.1] = -1
    for C in (1, 5, 19, 200):
        for ep_size in (1, 2, 4):
            rm = orc.route_map(ids, N, ep_size, C, ep_rank=ep_size - 1)
            _check_route_invariants(ids, N, ep_size, C, rm)
            # row_src is the inverse of the local part of the route map
            E_L = N // ep_size
            loc = rm["dest_rank"] == ep_size - 1
            n_loc = rm["offsets"][ep_size - 1, -1]
            assert np.all(rm["row_src"][n_loc:] == -1)
            for t, k in zip(*np.nonzero(loc)):
                assert rm["row_src"][rm["dest_row"][t, k]] == t * K + k
            assert np.sum(rm["row_src"] >= 0) == loc.sum()
            assert rm["row_src"].shape == (E_L * C,)


def test_constant_logits_keep_first_c_tokens():
    T, N, K, C = 20, 6, 2, 7
    idx, _ = orc.topk_softmax(np.zeros((T, N), np.float32), K)
    rm = orc.route_map(idx, N, 1, C)
    assert rm["counts"].tolist() == [T, T, 0, 0, 0, 0]
    assert np.all(rm["drop_mask"][:C] == 0) and np.all(rm["drop_mask"][C:] == 1)
    assert rm["dest_row"][:C, 0].tolist() == list(range(C))
    assert rm["dest_row"][:C, 1].tolist() == list(range(C, 2 * C))


def test_large_capacity_never_drops():
    rng = np.random.default_rng(1)
    idx, _ = orc.topk_softmax(rng.standard_normal((60, 10)).astype(np.float32), 3)
    rm = orc.route_map(idx, 10, 2, 60)
    assert rm["drop_mask"].sum() == 0 and np.all(rm["dest_row"] >= 0)


# ---------------------------------------------------------------- dispatch
def test_dispatch_is_exact_copy_and_leaves_tail():
    rng = np.random.default_rng(2)
    T, N, K, d, C = 30, 6, 2, 5, 8
    idx, _ = orc.topk_softmax(rng.standard_normal((T, N)).astype(np.float32), K)
    rm = orc.route_map(idx, N, 2, C, ep_rank=1)
    x = rng.standard_normal((T, d))
    buf = orc.dispatch_rows(x, rm["dest_rank"], rm["dest_row"], 1, 3 * C)
    n = rm["offsets"][1, -1]
    for row in range(n):
        t = rm["row_src"][row] // K
        assert np.array_equal(buf[row], x[t])
    assert np.all(np.isnan(buf[n:]))


# ---------------------------------------------------------------- bf16 rounding
def test_round_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.standard_normal(20000) * s for s in (1e-30, 1e-3, 1, 1e3, 1e30)])
    v32 = v.astype(np.float32)   # fp32-representable: a single rounding either way
    ref = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.round_bf16(v32.astype(np.float64)), ref)


def test_round_bf16_ties_to_even():
    one = 1.0
    ulp = 2.0 ** -7
    assert orc.round_bf16(one + ulp / 2) == one              # tie -> even (1.0)
    assert orc.round_bf16(one + 1.5 * ulp) == one + 2 * ulp  # tie -> even
    assert orc.round_bf16(one + ulp / 2 + 1e-12) == one + ulp
    assert orc.round_bf16(-(one + ulp / 2)) == -one


# ---------------------------------------------------------------- FFN
def test_silu_identities():
    z = np.linspace(-30, 30, 601)
    s = orc.silu(z)
    assert orc.silu(0.0) == 0.0
    assert np.allclose(s - orc.silu(-z), z, rtol=0, atol=1e-12)     # silu(z)-silu(-z)=z
    assert np.allclose(orc.silu(2.0), 2.0 / (1.0 + math.exp(-2.0)), rtol=1e-15)


def test_ffn_closed_form_one_by_one():
    # d = 1, F = 1: gate 2, up 3, down 5 on x = 1 -> Y = 5 * 3 * silu(2)
    w_gu = np.array([[2.0], [3.0]])
    w_d = np.array([[5.0]])
    H, Y = orc.expert_ffn_rows(np.array([[1.0]]), w_gu, w_d, "f32")
    expect_h = 3.0 * 2.0 / (1.0 + math.exp(-2.0))
    assert abs(H[0, 0] - expect_h) < 1e-6
    assert abs(Y[0, 0] - 5 * expect_h) < 1e-5
    # the up half gates nothing: a zero up half gives zero output
    H0, Y0 = orc.expert_ffn_rows(np.array([[1.0]]), np.array([[2.0], [0.0]]), w_d, "f32")
    assert H0[0, 0] == 0 and Y0[0, 0] == 0


def test_ffn_single_expert_equals_dense_swiglu_mlp():
    """One expert over all rows is the textbook dense SwiGLU MLP (torch float64)."""
    rng = np.random.default_rng(5)
    R, d, F = 37, 12, 10
    X = rng.standard_normal((R, d))
    w_gu = rng.standard_normal((1, 2 * F, d)) * 0.3
    w_d = rng.standard_normal((1, d, F)) * 0.3
    H, Y = orc.expert_ffn(X, np.array([0, R]), w_gu, w_d, "f32")
    tx = torch.from_numpy(X)
    g = torch.nn.functional.linear(tx, torch.from_numpy(w_gu[0, :F]))
    u = torch.nn.functional.linear(tx, torch.from_numpy(w_gu[0, F:]))
    ref = torch.nn.functional.linear(torch.nn.functional.silu(g) * u, torch.from_numpy(w_d[0]))
    assert np.allclose(Y, ref.numpy(), rtol=1e-5, atol=1e-6)


def test_ffn_uses_each_experts_own_weights_and_skips_tail():
    rng = np.random.default_rng(6)
    d, F = 8, 6
    w_gu = rng.standard_normal((3, 2 * F, d))
    w_d = rng.standard_normal((3, d, F))
    buf = rng.standard_normal((12, d))
    off = np.array([0, 4, 4, 9])          # expert 1 is empty, rows 9..11 are tail
    H, Y = orc.expert_ffn(buf, off, w_gu, w_d, "f32")
    _, Y0 = orc.expert_ffn_rows(buf[0:4], w_gu[0], w_d[0], "f32")
    _, Y2 = orc.expert_ffn_rows(buf[4:9], w_gu[2], w_d[2], "f32")
    assert np.array_equal(Y[0:4], Y0) and np.array_equal(Y[4:9], Y2)
    assert np.all(np.isnan(Y[9:]))
    # rows are independent: permuting an expert's rows permutes its outputs
    perm = rng.permutation(5)
    _, Yp = orc.expert_ffn_rows(buf[4:9][perm], w_gu[2], w_d[2], "f32")
    assert np.array_equal(Yp, Y2[perm])


# ---------------------------------------------------------------- combine
def test_combine_identity_experts_reproduce_weighted_input():
    rng = np.random.default_rng(9)
    T, N, K, d = 40, 8, 3, 6
    idx, w = orc.topk_softmax(rng.standard_normal((T, N)).astype(np.float32), K)
    for C in (100, 9):           # no drops, then drops
        rm = orc.route_map(idx, N, 1, C)
        x = rng.standard_normal((T, d))
        buf = orc.dispatch_rows(x, rm["dest_rank"], rm["dest_row"], 0, N * C)
        out = orc.combine(buf, rm["dest_rank"], rm["dest_row"], w, 0, "f32")
        wk = np.where(rm["dest_rank"] >= 0, w.astype(np.float64), 0).sum(axis=1)
        assert np.allclose(out, wk[:, None] * x, rtol=1e-6, atol=1e-6)
        if C == 100:
            assert np.allclose(out, x, rtol=1e-6, atol=1e-6)


def test_combine_k1_unit_weight_is_exact_unpermute():
    rng = np.random.default_rng(10)
    T, N, d = 25, 5, 4
    idx, w = orc.topk_softmax(rng.standard_normal((T, N)).astype(np.float32), 1)
    rm = orc.route_map(idx, N, 1, T)
    y = rng.standard_normal((N * T, d)).astype(np.float32).astype(np.float64)
    out = orc.combine(y, rm["dest_rank"], rm["dest_row"], w, 0, "f32")
    assert np.array_equal(out, y[rm["dest_row"][:, 0]])


def test_combine_partial_sums_neuron_example():
    g = _load("neuron_partial_sum.json")
    N, ep = g["N"], g["ep_size"]
    ids = np.array([g["ids"]], dtype=np.int32)
    w = np.array([g["weights"]], dtype=np.float32)
    rng = np.random.default_rng(11)
    d = 5
    y_expert = rng.standard_normal((N, d))      # output row of each expert for this token
    total = np.zeros(d)
    contributing = []
    for r in range(ep):
        rm = orc.route_map(ids, N, ep, 1, ep_rank=r)
        E_L = N // ep
        y = np.zeros((E_L, d))
        for k in range(4):
            if rm["dest_rank"][0, k] == r:
                y[rm["dest_row"][0, k]] = y_expert[ids[0, k]]
        part = orc.combine(y, rm["dest_rank"], rm["dest_row"], w, r, "f32")
        if np.any(part != 0):
            contributing.append(r)
        total += part[0]
    assert contributing == g["contributing_ranks"]
    full = sum(float(w[0, k]) * y_expert[ids[0, k]] for k in range(4))
    assert np.allclose(total, full, rtol=1e-6)


def test_layer_shard_sum_equals_unsharded_layer():
    rng = np.random.default_rng(12)
    T, d, N, K, F, C = 48, 8, 8, 2, 6, 10
    logits = rng.standard_normal((T, N)).astype(np.float32)
    x = rng.standard_normal((T, d))
    w_gu = rng.standard_normal((N, 2 * F, d)) * 0.3
    w_d = rng.standard_normal((N, d, F)) * 0.3
    full = orc.moe_layer(logits, x, w_gu, w_d, K, C, 1, 0, "f32")
    ep = 4
    E_L = N // ep
    total = np.zeros((T, d))
    for r in range(ep):
        part = orc.moe_layer(logits, x, w_gu[r * E_L:(r + 1) * E_L], w_d[r * E_L:(r + 1) * E_L],
                             K, C, ep, r, "f32")
        total += part["out"]
        # the global route map is the same from every rank
        assert np.array_equal(part["drop_mask"], full["drop_mask"])
    assert np.allclose(total, full["out"], rtol=1e-5, atol=1e-6)
