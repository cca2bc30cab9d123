"""Helpers shared by the GPU parity tests: run the HIP layer stage by stage and
compare with the CPU oracle. The oracle only ever receives inputs drawn by the
seeded generators (or taken from the oracle itself); nothing computed by the
HIP path is fed to it."""
from __future__ import annotations

import numpy as np
import torch

import combine_top_softmax_amd as moe
from oracle import moe_oracle as orc

BF16_NAN = -1   # int16 0xFFFF: a NaN in bfloat16
F32_NAN = -1    # int32 0xFFFFFFFF: a NaN in fp32


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.to(torch.float64).numpy()
    return t.numpy()


def poison_(t: torch.Tensor) -> torch.Tensor:
    """Fill with an all-ones bit pattern (NaN for bf16/fp32)."""
    if t.dtype == torch.bfloat16:
        t.view(torch.int16).fill_(BF16_NAN)
    elif t.dtype == torch.float32:
        t.view(torch.int32).fill_(F32_NAN)
    else:
        t.fill_(-1)
    return t


def is_poison(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16) == BF16_NAN
    if t.dtype == torch.float32:
        return t.view(torch.int32) == F32_NAN
    return t == -1


def tol_of(dtype: str) -> float:
    return 2e-2 if dtype == "bf16" else 1e-4


# Every floating-point comparison made through the helpers below, for the
# end-of-session report (conftest.py prints it; PARITY_REPORT=<path> also
# writes it as JSON): test, quantity, rows compared, worst per-row relative L2
# error, worst element error relative to its scale (max(|ref|, row rms), or
# the Cauchy-Schwarz bound of assert_bounded; either is held to the
# tolerance), largest absolute difference.
REPORT: list = []


def _record(what: str, rows: int, worst_row: float, worst_elem: float, max_abs: float,
            tol: float) -> None:
    import os
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    REPORT.append(dict(test=test, what=what, rows=int(rows), tol=tol, worst_row_l2=worst_row,
                       worst_elem_rel=worst_elem, max_abs_err=max_abs))


def assert_rows_close(got: np.ndarray, ref: np.ndarray, tol: float, what: str,
                      elementwise: bool = True) -> float:
    """Element by element and row by row: for every element
    |got - ref| <= tol * max(|ref|, rms(ref row)), and for every row the
    relative L2 error ||got - ref|| / ||ref|| <= tol; rows that are exactly
    zero in the reference must be exactly zero. The element bound is relative
    to the element itself, floored at the row's rms so that elements near
    zero (where a 1-ulp storage rounding is a large relative change) are held
    to the row's scale. Records the worst values (see REPORT) and returns the
    worst per-row error. elementwise=False records the element statistic
    without holding it to tol (for results that inherit discrete differences
    already validated upstream, such as MXFP8 code flips)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.ndim == 1:
        got, ref = got[None], ref[None]
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    zero = np.all(ref == 0, axis=1)
    assert np.all(got[zero] == 0), f"{what}: rows that must be exactly zero are not"
    nz = ~zero
    if not np.any(nz):
        _record(what, len(ref), 0.0, 0.0, 0.0, tol)
        return 0.0
    g, r = got[nz], ref[nz]
    diff = np.abs(g - r)
    norm = np.linalg.norm(r, axis=1)
    err = np.linalg.norm(g - r, axis=1) / norm
    rms = norm / np.sqrt(r.shape[1])
    bound = np.maximum(np.abs(r), rms[:, None])
    elem = diff / bound
    worst, worst_e, max_abs = float(err.max()), float(elem.max()), float(diff.max())
    _record(what, len(ref), worst, worst_e, max_abs, tol)
    assert worst <= tol, f"{what}: worst per-row relative L2 error {worst:.3e} > {tol:.1e}"
    if elementwise and worst_e > tol:
        i, j = np.unravel_index(int(np.argmax(elem)), elem.shape)
        raise AssertionError(
            f"{what}: element ({i}, {j}) of the nonzero rows off by {diff[i, j]:.3e} = "
            f"{worst_e:.3e} x max(|ref|, row rms) > {tol:.1e} (got {g[i, j]!r}, ref {r[i, j]!r})")
    return worst


def assert_bounded(got: np.ndarray, ref: np.ndarray, scale: np.ndarray, tol: float,
                   what: str) -> float:
    """|got - ref| <= tol * scale elementwise, where ``scale`` is the
    Cauchy-Schwarz bound of the quantity (e.g. ||a|| ||b|| for a dot product
    <a, b>): a relative error tol on the operands moves the result by at most
    that much, however much the dot product itself cancels. Entries whose
    scale is zero must match exactly. Returns the worst |got-ref|/scale."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    assert got.shape == ref.shape == scale.shape, (what, got.shape, ref.shape, scale.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    zero = scale == 0
    assert np.all(got[zero] == ref[zero]), f"{what}: entries with a zero bound differ"
    if not np.any(~zero):
        _record(what, got.shape[0], 0.0, 0.0, 0.0, tol)
        return 0.0
    diff = np.abs(got[~zero] - ref[~zero])
    r = diff / scale[~zero]
    worst = float(r.max())
    _record(what, got.shape[0], float("nan"), worst, float(diff.max()), tol)
    assert worst <= tol, f"{what}: worst error / bound {worst:.3e} > {tol:.1e}"
    return worst


def dw_bound(dout: np.ndarray, y: np.ndarray, dest_rank, dest_row, ep_rank: int) -> np.ndarray:
    """||dout[t]|| * ||y[dest_row[t,k]]|| for the kept local routes, else 0."""
    T, K = dest_rank.shape
    b = np.zeros((T, K))
    dn = np.linalg.norm(np.asarray(dout, dtype=np.float64), axis=1)
    for t in range(T):
        for k in range(K):
            if dest_rank[t, k] == ep_rank:
                b[t, k] = dn[t] * np.linalg.norm(np.asarray(y[int(dest_row[t, k])], np.float64))
    return b


def dlogit_bound(idx, w, dwb, N: int) -> np.ndarray:
    """Bound on the logit-gradient error implied by errors dwb on dw:
    |d dl[t, idx_k]| <= w_k (dwb_k + sum_j w_j dwb_j)."""
    T, K = idx.shape
    b = np.zeros((T, N))
    for t in range(T):
        inner = float(np.dot(w[t], dwb[t]))
        for k in range(K):
            b[t, idx[t, k]] = w[t, k] * (dwb[t, k] + inner)
    return b


def route_gpu(shape: moe.MoeShape, logits_dev: torch.Tensor, row_src: bool = True):
    out = moe.RouteOut.empty(shape, "cuda", row_src=row_src)
    for t in (out.topk_idx, out.dest_rank, out.dest_row, out.counts, out.offsets):
        t.fill_(-7)
    if out.row_src is not None:
        out.row_src.fill_(-7)
    out.drop_mask.fill_(7)
    out.topk_w.fill_(float("nan"))
    ws = torch.empty(moe.moe_route_workspace_size(shape), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)   # contents on entry must not matter
    moe.moe_route(shape, logits_dev, out, ws)
    return out


def check_route(out: moe.RouteOut, ref: dict, shape: moe.MoeShape) -> None:
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(out.topk_idx), ref["topk_idx"])
    np.testing.assert_allclose(to_np(out.topk_w), ref["topk_w"], rtol=1e-6, atol=0)
    np.testing.assert_array_equal(to_np(out.counts), ref["counts"])
    np.testing.assert_array_equal(to_np(out.offsets), ref["offsets"])
    np.testing.assert_array_equal(to_np(out.dest_rank), ref["dest_rank"])
    np.testing.assert_array_equal(to_np(out.dest_row), ref["dest_row"])
    np.testing.assert_array_equal(to_np(out.drop_mask), ref["drop_mask"])
    if out.row_src is not None:
        assert_row_src(to_np(out.row_src), ref["row_src"])


def assert_row_src(got: np.ndarray, ref_rs: np.ndarray) -> None:
    """row_src of Rmax = moe_buffer_rows rows against the oracle's, which spans
    the whole E_L*C capacity envelope: equal on the first Rmax rows, and the
    oracle places no route past them (its rows there are -1)."""
    assert len(got) <= len(ref_rs)
    assert bool((ref_rs[len(got):] == -1).all()), "oracle route past the buffer rows"
    np.testing.assert_array_equal(got, ref_rs[:len(got)], err_msg="row_src")


def assert_route_fields(out: moe.RouteOut, ref: dict, keys) -> None:
    for k in keys:
        if k == "row_src":
            assert_row_src(to_np(out.row_src), ref["row_src"])
        else:
            np.testing.assert_array_equal(to_np(getattr(out, k)), ref[k], err_msg=k)


def oracle_route(cfg, logits_cpu: torch.Tensor) -> dict:
    idx, w = orc.topk_softmax(logits_cpu.numpy(), cfg.K)
    rm = orc.route_map(idx, cfg.N, cfg.ep_size, cfg.capacity, cfg.ep_rank)
    rm["topk_idx"] = idx
    rm["topk_w"] = w
    return rm
