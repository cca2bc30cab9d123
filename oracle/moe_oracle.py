"""CPU oracle for the routed-expert MoE layer: forward and backward.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The product
path (the HIP library and its Python binding) never does, and this module never
imports the product package: the two share no code.

What it computes is the plain definition of a capacity-limited top-K MoE layer
with rowwise dispatch, as the pages describe it:

  * Olmo-core MoE report, Sec. 05 "Expert Parallelism": Fig. 15 (router ids and
    weights of the two-rank example), Sec. 5.4 "Rowwise EP Removes Block Packing"
    and Fig. 16 (route map: destination rank and row, negatives for invalid or
    dropped routes, row = offset of the expert on its rank + earlier accepted
    routes for that expert), Sec. 5.6 Table 8 (dispatch PUT / combine GET and
    weighted reduce), Sec. 5.7 (packed prefix, unwritten tail).
  * Olmo-core MoE report, Sec. 08 "Synchronization-Free Training", Sec. 8.5
    (device cumulative offsets for grouped GEMM, tail-aware SwiGLU).
  * AWS Neuron vLLM "Expert Parallelism (EP)" design: contiguous expert-to-rank
    placement, every rank sees all tokens, partial sums over ranks add up to
    the full combine (GPT-OSS-20B case study, "Why a single all-reduce works").
  * Backward: Olmo-core MoE report Sec. 5.6 Table 8 (adjoint row movements
    sharing the saved route map, router-weight gradient from the gathered
    expert outputs) and Sec. 5.7 (weight-gradient GEMMs over the valid prefix).
  * MXFP8 forward: Olmo-core MoE report Sec. 5.5 (rows quantized during
    dispatch; the grouped GEMM consumes the quantized data and scales
    directly), Sec. 5.8 (an MXFP8 route carries a qdata row and a scale row
    that follow the same destination indices and validity mask), Sec. 5.9
    (E4M3 data with E8M0 scales on forward dispatch, MXFP8 expert GEMMs,
    forward combine in BF16). The block format is the OCP microscaling (MX)
    format the report cites; see the MXFP8 section below.

Arithmetic is float64; values are rounded once to the layer's storage type at
the points where the layer stores them (routing weights -> fp32; expert hidden
activations H and expert outputs Y -> layer dtype; combined output -> layer
dtype). Loops are used wherever order matters; library primitives (a stable
sort, a matmul) serve as single steps.

Readings of points the pages leave open (each is listed with its reason in the
design notes of the repository):
  * gating: softmax over the K selected logits (every printed weight set sums
    to one and is in descending order);
  * ties in top-K: lower expert id first; -0.0 equals +0.0;
  * capacity is per expert and an input here (the workloads take
    C = ceil(T*K*cf/N), or C = T for the dropless mode, where no expert can
    receive more than C routes and none is dropped); the first C routes of an expert
    in token order are kept, later ones dropped -- this admission order is
    PARITY UNPINNED by the pages (the drawing's single drop cannot come from
    any per-expert token-order rule); it is pinned only by brute force of the
    stated rule;
  * gate/up split of W_gu: rows [0, F) gate, rows [F, 2F) up -- PARITY UNPINNED
    by the pages (the pages give the fused [H, 2I] shape only); pinned by
    closed forms of the stated convention;
  * weights of dropped routes are not renormalised (a dropped route adds zero).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "round_bf16", "round_to", "topk_softmax", "route_map", "dispatch_rows",
    "silu", "expert_ffn", "expert_ffn_rows", "combine", "combine_tokens",
    "moe_layer", "local_offsets", "combine_bwd", "expert_ffn_bwd_rows", "expert_ffn_bwd",
    "dispatch_bwd", "route_bwd", "moe_layer_bwd",
    "E4M3_MAX", "e4m3_decode", "e4m3_encode", "e8m0_decode", "mx_quantize", "mx_dequantize",
    "dispatch_mx", "expert_up_mx_rows", "expert_down_mx_rows", "expert_ffn_mx_rows",
    "expert_ffn_mx", "moe_layer_mx",
]


# --------------------------------------------------------------------------
# Rounding to storage types
# --------------------------------------------------------------------------
def round_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and the fp32 exponent range. Written from
    that definition: the quantum of a value with binary exponent e (v = m*2^e,
    0.5 <= |m| < 1) is 2^(e-8), but never below 2^-133 (the subnormal spacing).
    Values beyond the largest finite bfloat16 become +-inf. Returned as float64.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.array(v, copy=True)
    finite = np.isfinite(v) & (v != 0)
    if np.any(finite):
        _, e = np.frexp(v[finite])
        q = np.ldexp(1.0, np.maximum(e - 8, -133))
        r = np.rint(v[finite] / q) * q          # rint = round half to even
        bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
        r = np.where(np.abs(r) > bf16_max, np.sign(r) * np.inf, r)
        out[finite] = r
    return out


def round_to(v, dtype: str) -> np.ndarray:
    """Round float64 values to the storage type ("f32", "bf16", or "f64" = no
    rounding, used by the finite-difference checks); float64 result."""
    if dtype == "f64":
        return np.asarray(v, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_bf16(v)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# a1: top-K gating
# --------------------------------------------------------------------------
def topk_softmax(logits: np.ndarray, K: int):
    """Top-K expert ids per token and their softmax weights.

    Olmo-core MoE report, Sec. 05, Fig. 15: the router gives each token K expert
    indices and K weights; every printed weight set is in descending order and
    sums to one. Selection: experts ordered by (logit descending, id ascending),
    the first K kept (a stable sort of -logit; IEEE comparison makes -0.0 and
    +0.0 equal, so such ties fall back to the id). Weights: with m the largest
    selected logit, w_k = exp(l_k - m) / sum_j exp(l_j - m) over the K selected
    logits, evaluated in float64 and rounded once to fp32.

    Returns (idx [T,K] int32, w [T,K] float32).
    """
    L = np.asarray(logits, dtype=np.float32)
    T, N = L.shape
    if not (1 <= K <= N):
        raise ValueError("need 1 <= K <= N")
    order = np.argsort(-L, axis=1, kind="stable")
    idx = order[:, :K].astype(np.int32)
    sel = np.take_along_axis(L, idx.astype(np.int64), axis=1).astype(np.float64)
    m = sel[:, :1]
    e = np.exp(sel - m)
    w = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx, w


# --------------------------------------------------------------------------
# a2: route metadata (counts, admission, offsets, route map)
# --------------------------------------------------------------------------
def route_map(idx: np.ndarray, N: int, ep_size: int, C: int, ep_rank: int = 0):
    """Route-map builder for a capacity-limited, expert-sharded layer.

    Olmo-core MoE report, Sec. 5.4 and Fig. 16: two [T, K] tensors give, for
    every route, the destination rank and the destination row in that rank's
    expert-capacity buffer; negative entries mark invalid or dropped routes.
    The row is the offset of the expert on its rank plus the number of earlier
    accepted routes for that expert, and the capacity decision is applied before
    any movement. AWS Neuron EP design: rank r owns experts [r*E_L, (r+1)*E_L).

    ``idx`` may hold -1 for an invalid route. Steps, in order:
      1. walk the routes in token order (t ascending, then k) and give each
         valid route its position p among the earlier routes of its expert;
         counts[e] is the number of routes to e;
      2. a route is kept iff p < C;
      3. kept[e] = min(counts[e], C); for rank r, off[r][j] is the sum of kept
         over local experts j' < j (j = 0..E_L);
      4. kept route: dest_rank = e // E_L, dest_row = off[rank][e % E_L] + p;
         dropped route: both -1, drop_mask = 1; invalid route: both -1,
         drop_mask = 0;
      5. row_src (for ``ep_rank``): row_src[dest_row] = t*K + k for kept local
         routes, -1 on the rows after the packed prefix.

    Returns a dict of numpy arrays.
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, K = idx.shape
    if N % ep_size != 0:
        raise ValueError("N must be a multiple of ep_size")
    E_L = N // ep_size
    counts = np.zeros(N, dtype=np.int64)
    pos = np.full((T, K), -1, dtype=np.int64)
    for t in range(T):
        for k in range(K):
            e = idx[t, k]
            if e < 0:
                continue
            pos[t, k] = counts[e]
            counts[e] += 1
    kept = np.minimum(counts, C)
    offsets = np.zeros((ep_size, E_L + 1), dtype=np.int64)
    for r in range(ep_size):
        for j in range(E_L):
            offsets[r, j + 1] = offsets[r, j] + kept[r * E_L + j]
    dest_rank = np.full((T, K), -1, dtype=np.int64)
    dest_row = np.full((T, K), -1, dtype=np.int64)
    drop_mask = np.zeros((T, K), dtype=np.uint8)
    row_src = np.full(E_L * C, -1, dtype=np.int64)
    for t in range(T):
        for k in range(K):
            e = idx[t, k]
            if e < 0:
                continue
            if pos[t, k] >= C:
                drop_mask[t, k] = 1
                continue
            r, j = divmod(int(e), E_L)
            row = offsets[r, j] + pos[t, k]
            dest_rank[t, k] = r
            dest_row[t, k] = row
            if r == ep_rank:
                row_src[row] = t * K + k
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "dest_rank": dest_rank.astype(np.int32),
        "dest_row": dest_row.astype(np.int32),
        "drop_mask": drop_mask,
        "row_src": row_src.astype(np.int32),
        "pos": pos.astype(np.int32),
    }


def local_offsets(offsets: np.ndarray, ep_rank: int) -> np.ndarray:
    """The cumulative row offsets [E_L+1] of rank ``ep_rank``'s local experts."""
    return np.asarray(offsets)[ep_rank]


# --------------------------------------------------------------------------
# a3: rowwise dispatch
# --------------------------------------------------------------------------
def dispatch_rows(x: np.ndarray, dest_rank: np.ndarray, dest_row: np.ndarray,
                  ep_rank: int, n_rows: int) -> np.ndarray:
    """buf[dest_row[t,k]] = x[t] for every route whose dest_rank is ``ep_rank``.

    Olmo-core MoE report, Sec. 5.6 Table 8 (dispatch forward: the token-source
    rank pushes x_t to the capacity row assigned to the selected expert) and
    the closing paragraph of Sec. 5.6 (PUT skips negative destinations). Rows
    not written stay NaN here, so a reader of the tail is visible.
    Returns buf [n_rows, d] with x's dtype (an exact copy, no arithmetic).
    """
    x = np.asarray(x)
    buf = np.full((n_rows, x.shape[1]), np.nan, dtype=x.dtype)
    T, K = dest_rank.shape
    for t in range(T):
        for k in range(K):
            if dest_rank[t, k] == ep_rank and dest_row[t, k] >= 0:
                buf[dest_row[t, k]] = x[t]
    return buf


# --------------------------------------------------------------------------
# a4: grouped expert SwiGLU FFN over the packed prefix
# --------------------------------------------------------------------------
def silu(z):
    """silu(z) = z / (1 + exp(-z)) (float64)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn_rows(X: np.ndarray, w_gu_j: np.ndarray, w_d_j: np.ndarray, dtype: str):
    """Bias-free SwiGLU MLP of one expert on rows X.

    Olmo-core MoE report, Sec. 5.2 and Fig. 14 (Linear 1 -> SwiGLU -> Linear 2)
    and Sec. 04 "Distributed Data Parallel" (bias-free SwiGLU expert MLP).
    With W_gu[j] of shape [2F, d] (rows [0,F) gate, [F,2F) up) and W_d[j] of
    shape [d, F]: G = X W_gate^T, U = X W_up^T, H = silu(G) * U rounded to the
    storage type, Y = H W_d^T rounded to the storage type.
    Returns (H, Y) as float64 arrays holding storage-type values.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(w_gu_j, dtype=np.float64)
    F = W.shape[0] // 2
    G = X @ W[:F].T
    U = X @ W[F:].T
    H = round_to(silu(G) * U, dtype)
    Y = round_to(H @ np.asarray(w_d_j, dtype=np.float64).T, dtype)
    return H, Y


def expert_ffn(buf: np.ndarray, offsets_local: np.ndarray, w_gu: np.ndarray,
               w_d: np.ndarray, dtype: str):
    """Grouped expert FFN over each local expert's row interval.

    Olmo-core MoE report, Sec. 5.7 (the local experts' rows are packed back to
    back from row 0, one unwritten tail follows; grouped GEMM skips the tail)
    and Sec. 08 Sec. 8.5 (int32 cumulative offsets; tail-aware SwiGLU). Expert
    j owns rows [off[j], off[j+1]). Rows after off[E_L] are left NaN.
    Returns (H [rows, F], Y [rows, d]) float64.
    """
    E_L = len(offsets_local) - 1
    rows = buf.shape[0]
    F = w_gu.shape[1] // 2
    d = w_d.shape[1]
    H = np.full((rows, F), np.nan)
    Y = np.full((rows, d), np.nan)
    for j in range(E_L):
        a, b = int(offsets_local[j]), int(offsets_local[j + 1])
        if b > a:
            H[a:b], Y[a:b] = expert_ffn_rows(buf[a:b], w_gu[j], w_d[j], dtype)
    return H, Y


# --------------------------------------------------------------------------
# a5: weighted combine back to token order
# --------------------------------------------------------------------------
def combine_tokens(tokens, y_of_row, dest_rank, dest_row, w, ep_rank: int, d: int,
                   dtype: str) -> np.ndarray:
    """Combine for a subset of tokens; ``y_of_row(row)`` returns that expert row.

    Olmo-core MoE report, Sec. 5.6 Table 8 (combine forward: the token source
    pulls the selected expert outputs and performs the router-weighted
    reduction) and its closing paragraph (invalid entries gather zero).
    AWS Neuron EP design: a rank contributes only its local experts' outputs,
    tokens not routed to it get zero. out[t] = sum over k ascending with
    dest_rank[t,k] == ep_rank of w[t,k] * y[dest_row[t,k]], in float64,
    rounded once to the storage type.
    """
    out = np.zeros((len(tokens), d), dtype=np.float64)
    K = dest_rank.shape[1]
    for i, t in enumerate(tokens):
        acc = np.zeros(d, dtype=np.float64)
        for k in range(K):
            if dest_rank[t, k] == ep_rank and dest_row[t, k] >= 0:
                acc += float(w[t, k]) * np.asarray(y_of_row(int(dest_row[t, k])), dtype=np.float64)
        out[i] = acc
    return round_to(out, dtype)


def combine(y: np.ndarray, dest_rank, dest_row, w, ep_rank: int, dtype: str) -> np.ndarray:
    """Combine for all tokens (see ``combine_tokens``). Returns [T, d] float64."""
    T = dest_rank.shape[0]
    y = np.asarray(y)
    return combine_tokens(range(T), lambda r: y[r], dest_rank, dest_row, w, ep_rank,
                          y.shape[1], dtype)


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------
def moe_layer(logits, x, w_gu, w_d, K: int, C: int, ep_size: int, ep_rank: int, dtype: str):
    """Route -> dispatch -> grouped SwiGLU FFN -> combine, for one rank's shard.

    The step order of the rowwise path in Olmo-core MoE report Sec. 05 Fig. 16:
    route-map build, row dispatch, grouped expert computation, row gather and
    weighted reduce. Returns a dict with every intermediate.
    """
    logits = np.asarray(logits, dtype=np.float32)
    N = logits.shape[1]
    idx, w = topk_softmax(logits, K)
    rm = route_map(idx, N, ep_size, C, ep_rank)
    E_L = N // ep_size
    buf = dispatch_rows(np.asarray(x, dtype=np.float64), rm["dest_rank"], rm["dest_row"],
                        ep_rank, E_L * C)
    H, Y = expert_ffn(buf, rm["offsets"][ep_rank], w_gu, w_d, dtype)
    out = combine(Y, rm["dest_rank"], rm["dest_row"], w, ep_rank, dtype)
    res = dict(rm)
    res.update(topk_idx=idx, topk_w=w, buf=buf, h=H, y=Y, out=out)
    return res


# --------------------------------------------------------------------------
# Backward: the adjoint of each forward step
# --------------------------------------------------------------------------
# Olmo-core MoE report, Sec. 5.6 Table 8: backward reverses each forward
# movement with the same saved route map -- combine backward pushes each
# router-weighted output gradient to its expert-output-gradient row, dispatch
# backward pulls the route gradients and sums them into the token's gradient;
# the router-weight gradient comes from the gathered expert outputs and the
# token-output gradient of the same accepted routes. Sec. 5.7: the expert
# weight-gradient GEMMs run over the valid prefix only. Storage points mirror
# the forward: expert-side activations and row gradients are stored in the
# layer dtype, weight gradients and routing-weight gradients are float.

def combine_bwd(dout, y, dest_rank, dest_row, w, ep_rank: int, n_rows: int, dtype: str):
    """dY[row] = w[t,k] * dOut[t] (stored in dtype) and dw[t,k] = <dOut[t], Y[row]>
    for every kept route of rank ``ep_rank``; dw = 0 for every other route.
    Returns (dY [n_rows, d] float64, NaN on rows no route writes; dw [T, K] float64)."""
    dout = np.asarray(dout, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    T, K = dest_rank.shape
    dy = np.full((n_rows, dout.shape[1]), np.nan)
    dw = np.zeros((T, K))
    for t in range(T):
        for k in range(K):
            if dest_rank[t, k] == ep_rank and dest_row[t, k] >= 0:
                r = int(dest_row[t, k])
                dy[r] = round_to(float(w[t, k]) * dout[t], dtype)
                dw[t, k] = float(np.dot(dout[t], y[r]))
    return dy, dw


def expert_ffn_bwd_rows(X, w_gu_j, w_d_j, H, dY, dtype: str):
    """Backward of the SwiGLU MLP of one expert on rows X (see expert_ffn_rows).

    G and U are recomputed from X and stored in dtype, as the forward stores H;
    with s = sigmoid(G): dH = dY W_d, dG = dH * U * s * (1 + G (1 - s)),
    dU = dH * G * s, [dG, dU] stored in dtype, dX = [dG, dU] W_gu stored in
    dtype, dW_d = dY^T H and dW_gu = [dG, dU]^T X (float).
    Returns dict(gu, dgu, dx, dw_gu, dw_d)."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(w_gu_j, dtype=np.float64)
    Wd = np.asarray(w_d_j, dtype=np.float64)
    F = W.shape[0] // 2
    gu = round_to(X @ W.T, dtype)
    G, U = gu[:, :F], gu[:, F:]
    dH = np.asarray(dY, dtype=np.float64) @ Wd
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-G))
    dG = dH * U * s * (1.0 + G * (1.0 - s))
    dU = dH * G * s
    dgu = round_to(np.concatenate([dG, dU], axis=1), dtype)
    dx = round_to(dgu @ W, dtype)
    dw_d = np.asarray(dY, dtype=np.float64).T @ np.asarray(H, dtype=np.float64)
    dw_gu = dgu.T @ X
    return {"gu": gu, "dgu": dgu, "dx": dx, "dw_gu": dw_gu, "dw_d": dw_d}


def expert_ffn_bwd(buf, offsets_local, w_gu, w_d, H, dY, dtype: str):
    """Grouped backward over each local expert's rows [off[j], off[j+1]).
    Row outputs are NaN after the packed prefix; an expert with no row gets
    zero weight gradients."""
    E_L = len(offsets_local) - 1
    rows = buf.shape[0]
    F = w_gu.shape[1] // 2
    d = w_d.shape[1]
    res = {"gu": np.full((rows, 2 * F), np.nan), "dgu": np.full((rows, 2 * F), np.nan),
           "dx": np.full((rows, d), np.nan), "dw_gu": np.zeros((E_L, 2 * F, d)),
           "dw_d": np.zeros((E_L, d, F))}
    for j in range(E_L):
        a, b = int(offsets_local[j]), int(offsets_local[j + 1])
        if b > a:
            r = expert_ffn_bwd_rows(buf[a:b], w_gu[j], w_d[j], H[a:b], dY[a:b], dtype)
            for k in ("gu", "dgu", "dx"):
                res[k][a:b] = r[k]
            res["dw_gu"][j] = r["dw_gu"]
            res["dw_d"][j] = r["dw_d"]
    return res


def dispatch_bwd(dX, dest_rank, dest_row, ep_rank: int, dtype: str):
    """dx[t] = sum over k ascending of dX[dest_row[t,k]] for the kept routes of
    rank ``ep_rank`` (accumulated in float64, stored in dtype; zero when the
    token has none). Returns [T, d] float64."""
    dX = np.asarray(dX, dtype=np.float64)
    T, K = dest_rank.shape
    dx = np.zeros((T, dX.shape[1]))
    for t in range(T):
        for k in range(K):
            if dest_rank[t, k] == ep_rank and dest_row[t, k] >= 0:
                dx[t] += dX[int(dest_row[t, k])]
    return round_to(dx, dtype)


def route_bwd(idx, w, dw, N: int):
    """Gradient of the logits through the softmax over the K selected logits:
    dl[t, idx[t,k]] = w[t,k] * (dw[t,k] - sum_j w[t,j] dw[t,j]); zero on the
    experts a token did not select (the selection itself is piecewise
    constant). Returns [T, N] float64."""
    idx = np.asarray(idx)
    w = np.asarray(w, dtype=np.float64)
    dw = np.asarray(dw, dtype=np.float64)
    T, K = idx.shape
    dl = np.zeros((T, N))
    for t in range(T):
        inner = float(np.dot(w[t], dw[t]))
        for k in range(K):
            dl[t, idx[t, k]] = w[t, k] * (dw[t, k] - inner)
    return dl


def moe_layer_bwd(fwd: dict, dout, x, w_gu, w_d, K: int, C: int, ep_size: int, ep_rank: int,
                  dtype: str):
    """Backward of moe_layer for the output gradient ``dout``, from the dict
    ``fwd`` that moe_layer returned. Returns a dict with every intermediate and
    the gradients dx [T,d], dlogits [T,N], dw_gu, dw_d."""
    T, d = np.asarray(dout).shape
    N = fwd["counts"].shape[0]
    E_L = N // ep_size
    n_rows = E_L * C
    dy, dw = combine_bwd(dout, fwd["y"], fwd["dest_rank"], fwd["dest_row"], fwd["topk_w"],
                         ep_rank, n_rows, dtype)
    ffn = expert_ffn_bwd(fwd["buf"], fwd["offsets"][ep_rank], w_gu, w_d, fwd["h"], dy, dtype)
    dx = dispatch_bwd(ffn["dx"], fwd["dest_rank"], fwd["dest_row"], ep_rank, dtype)
    dl = route_bwd(fwd["topk_idx"], fwd["topk_w"], dw, N)
    res = dict(ffn)
    res.update(dy=dy, dw=dw, dx_rows=ffn["dx"], dx=dx, dlogits=dl)
    return res


# --------------------------------------------------------------------------
# MXFP8 forward
# --------------------------------------------------------------------------
# Olmo-core MoE report, Sec. 5.5 / 5.8 / 5.9: forward dispatch moves E4M3
# data with E8M0 scales, the expert GEMMs consume them directly, combine stays
# BF16. The block format is the OCP microscaling format the report cites
# (Rouhani et al. 2023; Open Compute Project 2023), read here as:
#   * a block is 32 consecutive elements along the contraction dimension of a
#     GEMM operand (the contiguous dimension of x rows, H rows and of the
#     [out, in] expert weights);
#   * the block's shared scale is X = 2^(floor(log2(amax)) - 8), amax the
#     largest magnitude in the block and 8 the exponent of E4M3's largest
#     normal (448 = 1.75 * 2^8); it is stored as an E8M0 code (biased exponent
#     127, clamped to [0, 254]); an all-zero block gets code 0;
#   * each element is V / X rounded to the nearest E4M3 value, ties to the
#     even code, magnitudes past the largest normal saturating to 448; the sign
#     bit follows the sign of V (so -0.0 and negative values that round to
#     zero give code 0x80).
# Where the pages leave the MX path open it mirrors the BF16 path: H is
# computed in float64, rounded to bf16, then quantized along F for the down
# GEMM; Y is rounded to bf16; combine is the BF16 combine.

E4M3_MAX = 448.0


def e4m3_decode(code) -> np.ndarray:
    """Value of OCP E4M3 (FN variant) codes: 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6;
    S.1111.111 is NaN; there are no infinities. Returns float64."""
    c = np.asarray(code).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return s * val


# the 127 finite non-negative E4M3 values, code order == value order
_E4M3_POS = e4m3_decode(np.arange(127))


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code to each finite value (ties to the even code),
    magnitudes past 448 saturating to 448. Returns uint8."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    sign = np.signbit(v)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def e8m0_decode(code) -> np.ndarray:
    """2^(code - 127) (code 255 is NaN). Returns float64."""
    c = np.asarray(code).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def mx_quantize(v: np.ndarray, block: int = 32):
    """MX quantization of each row of ``v`` [rows, n] along the row in blocks of
    ``block`` elements. Returns (qdata [rows, n] uint8 E4M3 codes,
    scales [rows, n/block] uint8 E8M0 codes)."""
    v = np.asarray(v, dtype=np.float64)
    rows, n = v.shape
    assert n % block == 0
    vb = v.reshape(rows, n // block, block)
    amax = np.max(np.abs(vb), axis=2)
    # floor(log2(amax)) exactly: amax = f * 2^ex with f in [0.5, 1)
    _, ex = np.frexp(amax)
    shared = np.where(amax > 0, ex - 1 - 8, -127)
    shared = np.clip(shared, -127, 127)
    scales = (shared + 127).astype(np.uint8)
    q = e4m3_encode(vb / np.exp2(shared.astype(np.float64))[:, :, None])
    return q.reshape(rows, n), scales


def mx_dequantize(q: np.ndarray, scales: np.ndarray, block: int = 32) -> np.ndarray:
    """E4M3 value times the block's E8M0 scale. Returns float64 [rows, n]."""
    q = np.asarray(q)
    rows, n = q.shape
    x = e4m3_decode(q).reshape(rows, n // block, block)
    return (x * e8m0_decode(scales)[:, :, None]).reshape(rows, n)


def dispatch_mx(x, dest_rank, dest_row, ep_rank: int, n_rows: int):
    """Quantize-on-dispatch: every token row of x is MX-quantized along d and
    its qdata and scale rows are copied to each kept local route's capacity
    row (Sec. 5.8: both follow the route's destination indices and validity
    mask). Returns (qdata [n_rows, d] uint8, scales [n_rows, d/32] uint8,
    written [n_rows] bool)."""
    q, sc = mx_quantize(np.asarray(x, dtype=np.float64))
    T, K = dest_rank.shape
    qb = np.zeros((n_rows, q.shape[1]), dtype=np.uint8)
    sb = np.zeros((n_rows, sc.shape[1]), dtype=np.uint8)
    written = np.zeros(n_rows, dtype=bool)
    for t in range(T):
        for k in range(K):
            if dest_rank[t, k] == ep_rank and dest_row[t, k] >= 0:
                r = int(dest_row[t, k])
                qb[r] = q[t]
                sb[r] = sc[t]
                written[r] = True
    return qb, sb, written


def expert_up_mx_rows(Xq, Xs, gu_q, gu_s):
    """Up half of the MXFP8 expert: G, U are the float64 products of the
    dequantized rows and W_gu[j] (gu_q/gu_s: [2F, d] quantized along d);
    H = silu(G) * U rounded to bf16, then MX-quantized along F.
    Returns (Hq [rows, F], Hs [rows, F/32])."""
    X = mx_dequantize(Xq, Xs)
    W = mx_dequantize(gu_q, gu_s)
    F = W.shape[0] // 2
    G = X @ W[:F].T
    U = X @ W[F:].T
    return mx_quantize(round_bf16(silu(G) * U))


def expert_down_mx_rows(Hq, Hs, d_q, d_s):
    """Down half of the MXFP8 expert: Y = dequantized H times dequantized
    W_d[j]^T (d_q/d_s: [d, F] quantized along F), rounded to bf16.
    Returns Y float64 [rows, d] holding bf16 values."""
    return round_bf16(mx_dequantize(Hq, Hs) @ mx_dequantize(d_q, d_s).T)


def expert_ffn_mx_rows(Xq, Xs, gu_q, gu_s, d_q, d_s):
    """SwiGLU MLP of one expert on MXFP8 operands: expert_up_mx_rows, then
    expert_down_mx_rows on the quantized H. Xq/Xs: rows' qdata/scales along d.
    Returns (Hq, Hs, Y) with Y float64 holding bf16 values."""
    Hq, Hs = expert_up_mx_rows(Xq, Xs, gu_q, gu_s)
    return Hq, Hs, expert_down_mx_rows(Hq, Hs, d_q, d_s)


def expert_ffn_mx(qbuf, sbuf, offsets_local, gu_q, gu_s, d_q, d_s):
    """Grouped MXFP8 expert FFN over each local expert's rows [off[j], off[j+1]).
    gu_q [E_L, 2F, d], gu_s [E_L, 2F, d/32], d_q [E_L, d, F], d_s [E_L, d, F/32].
    Returns (Hq [rows, F], Hs [rows, F/32], Y [rows, d] float64, NaN past the prefix)."""
    E_L = len(offsets_local) - 1
    rows = qbuf.shape[0]
    F = gu_q.shape[1] // 2
    d = d_q.shape[1]
    Hq = np.zeros((rows, F), dtype=np.uint8)
    Hs = np.zeros((rows, F // 32), dtype=np.uint8)
    Y = np.full((rows, d), np.nan)
    for j in range(E_L):
        a, b = int(offsets_local[j]), int(offsets_local[j + 1])
        if b > a:
            Hq[a:b], Hs[a:b], Y[a:b] = expert_ffn_mx_rows(qbuf[a:b], sbuf[a:b], gu_q[j], gu_s[j],
                                                          d_q[j], d_s[j])
    return Hq, Hs, Y


def moe_layer_mx(logits, x, w_gu, w_d, K: int, C: int, ep_size: int, ep_rank: int):
    """The MXFP8 forward of a bf16 layer: routing as moe_layer, quantize-on-
    dispatch, expert weights MX-quantized along their contraction dimension,
    the MXFP8 grouped FFN, and the BF16 combine. Returns a dict."""
    idx, w = topk_softmax(logits, K)
    N = logits.shape[1]
    rm = route_map(idx, N, ep_size, C, ep_rank)
    E_L = N // ep_size
    n_rows = E_L * C
    x = np.asarray(x, dtype=np.float64)
    w_gu = np.asarray(w_gu, dtype=np.float64)
    w_d = np.asarray(w_d, dtype=np.float64)
    d = x.shape[1]
    F = w_gu.shape[1] // 2
    qbuf, sbuf, written = dispatch_mx(x, rm["dest_rank"], rm["dest_row"], ep_rank, n_rows)
    gq, gs = mx_quantize(w_gu.reshape(-1, d))
    dq, ds = mx_quantize(w_d.reshape(-1, F))
    gq, gs = gq.reshape(E_L, 2 * F, d), gs.reshape(E_L, 2 * F, d // 32)
    dq, ds = dq.reshape(E_L, d, F), ds.reshape(E_L, d, F // 32)
    Hq, Hs, Y = expert_ffn_mx(qbuf, sbuf, rm["offsets"][ep_rank], gq, gs, dq, ds)
    out = combine(Y, rm["dest_rank"], rm["dest_row"], w, ep_rank, "bf16")
    res = dict(rm)
    res.update(topk_idx=idx, topk_w=w, qbuf=qbuf, sbuf=sbuf, written=written, w_gu_q=gq,
               w_gu_s=gs, w_d_q=dq, w_d_s=ds, h_q=Hq, h_s=Hs, y=Y, out=out)
    return res
