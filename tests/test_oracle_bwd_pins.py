"""Pins of the oracle's backward against the oracle's forward.

The backward is the adjoint of the forward, so on an unrounded (float64)
layer its gradients must equal central finite differences of the scalar
loss L = <dOut, out> -- a check that fails on any dropped term, wrong sign,
transposed operand or wrong activation derivative. Top-K selection and
capacity admission are piecewise constant; the logits used here keep every
selection gap far larger than the finite-difference step.
"""
import numpy as np
import pytest

from oracle import moe_oracle as orc


def _problem(seed, T=10, d=6, N=4, K=2, F=5):
    rng = np.random.default_rng(seed)
    # well-separated logits: the top-K set and order cannot change under +-h
    base = np.stack([rng.permutation(N) * 0.7 for _ in range(T)])
    logits = base + rng.uniform(-0.05, 0.05, size=(T, N))
    x = rng.standard_normal((T, d))
    w_gu = rng.standard_normal((N, 2 * F, d)) * 0.5
    w_d = rng.standard_normal((N, d, F)) * 0.5
    dout = rng.standard_normal((T, d))
    return logits, x, w_gu, w_d, dout


def _loss(logits, x, w_gu, w_d, dout, K, C, ep_size=1, ep_rank=0):
    E_L = logits.shape[1] // ep_size
    sl = slice(ep_rank * E_L, (ep_rank + 1) * E_L)
    out = orc.moe_layer(logits, x, w_gu[sl], w_d[sl], K, C, ep_size, ep_rank, "f64")["out"]
    return float(np.sum(dout * out))


def _fd(f, arr, idxs, h=1e-6):
    g = []
    for i in idxs:
        old = arr[i]
        arr[i] = old + h
        lp = f()
        arr[i] = old - h
        lm = f()
        arr[i] = old
        g.append((lp - lm) / (2 * h))
    return np.array(g)


@pytest.mark.parametrize("C", [100, 3])      # no drops, then capacity drops
def test_backward_matches_finite_differences(C):
    logits, x, w_gu, w_d, dout = _problem(3)
    K = 2
    fwd = orc.moe_layer(logits, x, w_gu, w_d, K, C, 1, 0, "f64")
    bwd = orc.moe_layer_bwd(fwd, dout, x, w_gu, w_d, K, C, 1, 0, "f64")
    if C == 3:
        assert fwd["drop_mask"].sum() > 0
    f = lambda: _loss(logits, x, w_gu, w_d, dout, K, C)
    rng = np.random.default_rng(0)
    xi = [tuple(i) for i in np.argwhere(np.ones_like(x))][::3]
    np.testing.assert_allclose(bwd["dx"][tuple(np.array(xi).T)], _fd(f, x, xi), rtol=1e-5, atol=1e-7)
    gi = [tuple(rng.integers(0, s) for s in w_gu.shape) for _ in range(25)]
    dgu_full = bwd["dw_gu"]
    np.testing.assert_allclose([dgu_full[i] for i in gi], _fd(f, w_gu, gi), rtol=1e-5, atol=1e-7)
    di = [tuple(rng.integers(0, s) for s in w_d.shape) for _ in range(25)]
    np.testing.assert_allclose([bwd["dw_d"][i] for i in di], _fd(f, w_d, di), rtol=1e-5, atol=1e-7)


def test_router_gradient_matches_finite_differences():
    """d L / d logits of the oracle forward itself. The oracle selects and
    weighs on fp32 copies of the logits, so the step is 1e-3 (fp32 rounding of
    the logits then perturbs L by ~1e-7 relative) and the tolerance 2e-3."""
    logits, x, w_gu, w_d, dout = _problem(5)
    K, C = 2, 100
    fwd = orc.moe_layer(logits, x, w_gu, w_d, K, C, 1, 0, "f64")
    bwd = orc.moe_layer_bwd(fwd, dout, x, w_gu, w_d, K, C, 1, 0, "f64")
    T, N = logits.shape
    L = logits.astype(np.float64).copy()
    f = lambda: _loss(L, x, w_gu, w_d, dout, K, C)
    idxs = [(t, e) for t in range(T) for e in range(N)]
    fd = _fd(f, L, idxs, h=1e-3)
    np.testing.assert_allclose(bwd["dlogits"].ravel(), fd, rtol=2e-3, atol=1e-5)
    # unselected experts get exactly zero
    for t in range(T):
        other = np.setdiff1d(np.arange(N), fwd["topk_idx"][t])
        assert np.all(bwd["dlogits"][t, other] == 0)


def test_backward_shards_sum_to_the_unsharded_backward():
    """AWS Neuron EP design: each rank contributes only its local experts; the
    adjoint contributions add up the same way (dx and the logit gradient are
    linear in the per-rank routing-weight gradients)."""
    logits, x, w_gu, w_d, dout = _problem(7, T=16, N=8)
    K, C = 2, 5
    full = orc.moe_layer(logits, x, w_gu, w_d, K, C, 1, 0, "f64")
    fb = orc.moe_layer_bwd(full, dout, x, w_gu, w_d, K, C, 1, 0, "f64")
    ep, E_L = 4, 2
    dx = np.zeros_like(x)
    dl = np.zeros_like(logits)
    for r in range(ep):
        sl = slice(r * E_L, (r + 1) * E_L)
        f = orc.moe_layer(logits, x, w_gu[sl], w_d[sl], K, C, ep, r, "f64")
        b = orc.moe_layer_bwd(f, dout, x, w_gu[sl], w_d[sl], K, C, ep, r, "f64")
        dx += b["dx"]
        dl += b["dlogits"]
        np.testing.assert_allclose(b["dw_gu"], fb["dw_gu"][sl], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(b["dw_d"], fb["dw_d"][sl], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dx, fb["dx"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dl, fb["dlogits"], rtol=1e-10, atol=1e-12)


def test_combine_backward_closed_form_k1():
    """K = 1 with unit weights: dY is dOut un-permuted, dw = <dOut, Y>."""
    rng = np.random.default_rng(9)
    T, N, d = 12, 4, 5
    idx, w = orc.topk_softmax(rng.standard_normal((T, N)).astype(np.float32), 1)
    rm = orc.route_map(idx, N, 1, T)
    y = rng.standard_normal((N * T, d))
    dout = rng.standard_normal((T, d))
    dy, dw = orc.combine_bwd(dout, y, rm["dest_rank"], rm["dest_row"], w, 0, N * T, "f64")
    rows = rm["dest_row"][:, 0]
    np.testing.assert_array_equal(dy[rows], dout)
    np.testing.assert_allclose(dw[:, 0], np.sum(dout * y[rows], axis=1), rtol=1e-14)
    # and the dispatch adjoint of a K=1 layer is the un-permute back
    dX = rng.standard_normal((N * T, d))
    dx = orc.dispatch_bwd(dX, rm["dest_rank"], rm["dest_row"], 0, "f64")
    np.testing.assert_array_equal(dx, dX[rows])
