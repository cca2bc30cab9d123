"""GPU parity of the layer backward: the HIP path (through the C ABI) against
the oracle's adjoint (pinned by finite differences in test_oracle_bwd_pins).

Stage by stage, each call gets the same seeded inputs on both sides (route
metadata from the oracle, stand-in rows from the seeded generators); then the
whole forward + backward runs on the GPU against the oracle's forward +
backward. Bars: per-row relative L2 <= 2e-2 (bf16) or 1e-4 (fp32) for row
tensors and weight-gradient rows, rows the oracle gives as exact zeros exactly
zero, buffer tails untouched (poisoned before the call). The router-weight
gradient is a dot product of d terms and may cancel, so it is held to the
Cauchy-Schwarz bound of its operands' error instead: |d dw| <= tol ||dout||
||y|| (and the logit gradient to the bound this implies through the softmax).
"""
import numpy as np
import pytest
import torch

import combine_top_softmax_amd as moe
from combine_top_softmax_amd.workloads import make_inputs, random_rows
from oracle import moe_oracle as orc
from gpu_util import (assert_bounded, assert_rows_close, dlogit_bound, dw_bound, is_poison,
                      oracle_route, poison_, to_np, tol_of)
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

ACC_TOL = 2e-5   # fp32 accumulation of a dot product, relative to its bound


def _f64(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).numpy()


def _dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t if dtype is None else t.to(dtype)).cuda()


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_combine_bwd_matches_oracle(cfg):
    print(f"[case] combine_bwd {cfg.name}", flush=True)
    inp = make_inputs(cfg, "cpu", with_weights=False)
    ref = oracle_route(cfg, inp.logits)
    shape = moe.MoeShape.from_config(cfg)
    dt = cfg.torch_dtype
    y = random_rows(shape.rows, cfg.d, dt, seed=cfg.seed + 200)
    dout = random_rows(cfg.T, cfg.d, dt, seed=cfg.seed + 300)
    dy = poison_(torch.empty(shape.rows, cfg.d, dtype=dt, device="cuda"))
    dw = poison_(torch.empty(cfg.T, cfg.K, dtype=torch.float32, device="cuda"))
    moe.moe_combine_bwd(shape, dout.cuda(), y.cuda(), _dev(ref["dest_rank"]),
                        _dev(ref["dest_row"]), _dev(ref["topk_w"]), dy, dw)
    torch.cuda.synchronize()
    dy_ref, dw_ref = orc.combine_bwd(_f64(dout), _f64(y), ref["dest_rank"], ref["dest_row"],
                                     ref["topk_w"], cfg.ep_rank, shape.rows, cfg.dtype)
    n = int(ref["offsets"][cfg.ep_rank, -1])
    if n > 0:
        assert_rows_close(to_np(dy[:n]), dy_ref[:n], tol_of(cfg.dtype), "dy")
    assert bool(is_poison(dy[n:]).all()), "dy tail written"
    b = dw_bound(_f64(dout), _f64(y), ref["dest_rank"], ref["dest_row"], cfg.ep_rank)
    assert_bounded(to_np(dw), dw_ref, b, ACC_TOL, "dw")


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_expert_ffn_bwd_matches_oracle(cfg):
    print(f"[case] expert_ffn_bwd {cfg.name}", flush=True)
    inp = make_inputs(cfg, "cpu")
    ref = oracle_route(cfg, inp.logits)
    shape = moe.MoeShape.from_config(cfg)
    dt = cfg.torch_dtype
    rows, F, d, E_L = shape.rows, cfg.F, cfg.d, cfg.E_L
    n = int(ref["offsets"][cfg.ep_rank, -1])
    x64 = _f64(inp.x)
    buf = orc.dispatch_rows(x64, ref["dest_rank"], ref["dest_row"], cfg.ep_rank, rows)
    buf = np.nan_to_num(buf)   # the tail is never read; keep it finite for the copy
    h = random_rows(rows, F, dt, seed=cfg.seed + 400)
    dy = random_rows(rows, d, dt, seed=cfg.seed + 500)
    buf_t = torch.from_numpy(buf).to(dt)
    gu = poison_(torch.empty(rows, 2 * F, dtype=dt, device="cuda"))
    dgu = poison_(torch.empty(rows, 2 * F, dtype=dt, device="cuda"))
    dx_rows = poison_(torch.empty(rows, d, dtype=dt, device="cuda"))
    dw_gu = poison_(torch.empty(E_L, 2 * F, d, dtype=torch.float32, device="cuda"))
    dw_d = poison_(torch.empty(E_L, d, F, dtype=torch.float32, device="cuda"))
    moe.moe_expert_ffn_bwd(shape, buf_t.cuda(), _dev(ref["offsets"]), inp.w_gu.cuda(),
                           inp.w_d.cuda(), h.cuda(), dy.cuda(), gu, dgu, dx_rows, dw_gu, dw_d)
    torch.cuda.synchronize()
    r = orc.expert_ffn_bwd(_f64(buf_t), ref["offsets"][cfg.ep_rank], _f64(inp.w_gu),
                           _f64(inp.w_d), _f64(h), _f64(dy), cfg.dtype)
    tol = tol_of(cfg.dtype)
    if n > 0:
        assert_rows_close(to_np(gu[:n]), r["gu"][:n], tol, "gu")
        assert_rows_close(to_np(dgu[:n]), r["dgu"][:n], tol, "dgu")
        assert_rows_close(to_np(dx_rows[:n]), r["dx"][:n], tol, "dx_rows")
    for name, t in (("gu", gu), ("dgu", dgu), ("dx_rows", dx_rows)):
        assert bool(is_poison(t[n:]).all()), f"{name} tail written"
    assert_rows_close(to_np(dw_gu).reshape(-1, d), r["dw_gu"].reshape(-1, d), tol, "dw_gu")
    assert_rows_close(to_np(dw_d).reshape(-1, F), r["dw_d"].reshape(-1, F), tol, "dw_down")


@pytest.mark.parametrize("cfg", SMALL[:3] + SMALL[6:7], ids=lambda c: c.name)
def test_expert_ffn_bwd_variants_agree(cfg):
    """Separate [G U] and [dG dU] buffers, dgu == gu in place, and the data
    and weight halves called one after the other all give the same bits."""
    inp = make_inputs(cfg, "cpu")
    ref = oracle_route(cfg, inp.logits)
    shape = moe.MoeShape.from_config(cfg)
    dt = cfg.torch_dtype
    rows, F, d, E_L = shape.rows, cfg.F, cfg.d, cfg.E_L
    buf = random_rows(rows, d, dt, seed=cfg.seed + 600).cuda()
    h = random_rows(rows, F, dt, seed=cfg.seed + 601).cuda()
    dy = random_rows(rows, d, dt, seed=cfg.seed + 602).cuda()
    off = _dev(ref["offsets"])
    w_gu, w_d = inp.w_gu.cuda(), inp.w_d.cuda()
    outs = []
    for variant in ("separate", "in_place", "halves"):
        gu = torch.zeros(rows, 2 * F, dtype=dt, device="cuda")
        dgu = torch.zeros(rows, 2 * F, dtype=dt, device="cuda") if variant == "separate" else gu
        dx_rows = torch.zeros(rows, d, dtype=dt, device="cuda")
        dw_gu = torch.zeros(E_L, 2 * F, d, dtype=torch.float32, device="cuda")
        dw_d = torch.zeros(E_L, d, F, dtype=torch.float32, device="cuda")
        if variant == "halves":
            moe.moe_expert_ffn_bwd_data(shape, buf, off, w_gu, w_d, dy, gu, dgu, dx_rows)
            moe.moe_expert_ffn_bwd_weight(shape, buf, off, h, dy, dgu, dw_gu, dw_d)
        else:
            moe.moe_expert_ffn_bwd(shape, buf, off, w_gu, w_d, h, dy, gu, dgu, dx_rows, dw_gu,
                                   dw_d)
        outs.append((dgu, dx_rows, dw_gu, dw_d))
    torch.cuda.synchronize()
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert torch.equal(a, b)


# bf16 with d % 64 != 0 takes the register-staged GEMM instead of the big-tile one
SAVED_GU_CASES = SMALL + [SMALL[1].with_(name="small_d200_bf16", d=200, seed=41)]


@pytest.mark.parametrize("cfg", SAVED_GU_CASES, ids=lambda c: c.name)
def test_saved_gu_matches_recompute(cfg):
    """moe_expert_up_save_gu writes the H of moe_expert_up and the [G U] that
    the backward recompute writes, bit for bit, and nothing past the prefix;
    moe_expert_ffn_bwd_data_saved_gu on it gives the recompute path's dgu and
    dx_rows bit for bit (separate and in-place dgu); [G U] against the oracle."""
    print(f"[case] saved gu {cfg.name}", flush=True)
    inp = make_inputs(cfg, "cpu")
    ref = oracle_route(cfg, inp.logits)
    shape = moe.MoeShape.from_config(cfg)
    dt = cfg.torch_dtype
    rows, F, d = shape.rows, cfg.F, cfg.d
    n = int(ref["offsets"][cfg.ep_rank, -1])
    buf = random_rows(rows, d, dt, seed=cfg.seed + 610)
    h_any = random_rows(rows, F, dt, seed=cfg.seed + 611)
    dy = random_rows(rows, d, dt, seed=cfg.seed + 612)
    off = _dev(ref["offsets"])
    w_gu, w_d = inp.w_gu.cuda(), inp.w_d.cuda()
    bufc, dyc = buf.cuda(), dy.cuda()

    h_ref = poison_(torch.empty(rows, F, dtype=dt, device="cuda"))
    moe.moe_expert_up(shape, bufc, off, w_gu, h_ref)
    h = poison_(torch.empty(rows, F, dtype=dt, device="cuda"))
    gu = poison_(torch.empty(rows, 2 * F, dtype=dt, device="cuda"))
    moe.moe_expert_up_save_gu(shape, bufc, off, w_gu, h, gu)

    gu_re = poison_(torch.empty(rows, 2 * F, dtype=dt, device="cuda"))
    dgu_re = poison_(torch.empty(rows, 2 * F, dtype=dt, device="cuda"))
    dx_re = poison_(torch.empty(rows, d, dtype=dt, device="cuda"))
    moe.moe_expert_ffn_bwd_data(shape, bufc, off, w_gu, w_d, dyc, gu_re, dgu_re, dx_re)
    dgu = poison_(torch.empty(rows, 2 * F, dtype=dt, device="cuda"))
    dx = poison_(torch.empty(rows, d, dtype=dt, device="cuda"))
    moe.moe_expert_ffn_bwd_data_saved_gu(shape, off, w_gu, w_d, dyc, gu, dgu, dx)
    gu_in_place = gu.clone()
    dx_ip = poison_(torch.empty(rows, d, dtype=dt, device="cuda"))
    moe.moe_expert_ffn_bwd_data_saved_gu(shape, off, w_gu, w_d, dyc, gu_in_place, gu_in_place,
                                         dx_ip)
    torch.cuda.synchronize()
    assert torch.equal(h[:n], h_ref[:n]), "H differs from moe_expert_up"
    assert torch.equal(gu[:n], gu_re[:n]), "[G U] differs from the backward recompute"
    for name, t in (("h", h), ("gu", gu), ("dgu", dgu), ("dx_rows", dx)):
        assert bool(is_poison(t[n:]).all()), f"{name} tail written"
    assert torch.equal(dgu[:n], dgu_re[:n]) and torch.equal(dx[:n], dx_re[:n])
    assert torch.equal(gu_in_place[:n], dgu_re[:n]) and torch.equal(dx_ip[:n], dx_re[:n])
    if n > 0:
        r = orc.expert_ffn_bwd(_f64(buf), ref["offsets"][cfg.ep_rank], _f64(inp.w_gu),
                               _f64(inp.w_d), _f64(h_any), _f64(dy), cfg.dtype)
        assert_rows_close(to_np(gu[:n]), r["gu"][:n], tol_of(cfg.dtype), "gu")


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_dispatch_bwd_matches_oracle(cfg):
    inp = make_inputs(cfg, "cpu", with_weights=False)
    ref = oracle_route(cfg, inp.logits)
    shape = moe.MoeShape.from_config(cfg)
    dt = cfg.torch_dtype
    dxr = random_rows(shape.rows, cfg.d, dt, seed=cfg.seed + 700)
    dx = poison_(torch.empty(cfg.T, cfg.d, dtype=dt, device="cuda"))
    moe.moe_dispatch_bwd(shape, dxr.cuda(), _dev(ref["dest_rank"]), _dev(ref["dest_row"]), dx)
    torch.cuda.synchronize()
    expect = orc.dispatch_bwd(_f64(dxr), ref["dest_rank"], ref["dest_row"], cfg.ep_rank,
                              cfg.dtype)
    assert_rows_close(to_np(dx), expect, tol_of(cfg.dtype), "dx")


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_route_bwd_matches_oracle(cfg):
    inp = make_inputs(cfg, "cpu", with_weights=False)
    ref = oracle_route(cfg, inp.logits)
    shape = moe.MoeShape.from_config(cfg)
    g = torch.Generator()
    g.manual_seed(cfg.seed + 800)
    dw = torch.randn(cfg.T, cfg.K, generator=g, dtype=torch.float32)
    dl = poison_(torch.empty(cfg.T, cfg.N, dtype=torch.float32, device="cuda"))
    moe.moe_route_bwd(shape, _dev(ref["topk_idx"]), _dev(ref["topk_w"]), dw.cuda(), dl)
    torch.cuda.synchronize()
    expect = orc.route_bwd(ref["topk_idx"], ref["topk_w"], dw.numpy(), cfg.N)
    bound = dlogit_bound(ref["topk_idx"], ref["topk_w"], np.abs(dw.numpy()), cfg.N)
    # fp32: the inner sum of K terms, a subtraction and a product
    assert_bounded(to_np(dl), expect, bound, 4e-6, "dlogits")


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_layer_backward_matches_oracle(cfg):
    """Forward + backward on the GPU (MoELayer, [G U] buffer reused in place
    for [dG dU]) against the oracle's forward + backward."""
    print(f"[case] layer backward {cfg.name}", flush=True)
    inp = make_inputs(cfg, "cpu")
    dt = cfg.torch_dtype
    dout = random_rows(cfg.T, cfg.d, dt, seed=cfg.seed + 900)
    shape = moe.MoeShape.from_config(cfg)
    layer = moe.MoELayer(shape, "cuda")
    layer.alloc_backward("cuda")
    for t in (layer.dy, layer.gu, layer.dx_rows, layer.dx, layer.dw, layer.dw_gu,
              layer.dw_down, layer.dlogits):
        poison_(t)
    w_gu, w_d = inp.w_gu.cuda(), inp.w_d.cuda()
    layer.forward(inp.logits.cuda(), inp.x.cuda(), w_gu, w_d)
    dx, dl, dwgu, dwd = layer.backward(dout.cuda(), w_gu, w_d)
    torch.cuda.synchronize()

    fwd = orc.moe_layer(inp.logits.numpy(), _f64(inp.x), _f64(inp.w_gu), _f64(inp.w_d), cfg.K,
                        cfg.capacity, cfg.ep_size, cfg.ep_rank, cfg.dtype)
    bwd = orc.moe_layer_bwd(fwd, _f64(dout), _f64(inp.x), _f64(inp.w_gu), _f64(inp.w_d),
                            cfg.K, cfg.capacity, cfg.ep_size, cfg.ep_rank, cfg.dtype)
    tol = tol_of(cfg.dtype)
    n = int(fwd["offsets"][cfg.ep_rank, -1])
    if n > 0:
        assert_rows_close(to_np(layer.dy[:n]), bwd["dy"][:n], tol, "dy")
        assert_rows_close(to_np(layer.dx_rows[:n]), bwd["dx_rows"][:n], tol, "dx_rows")
    assert bool(is_poison(layer.dy[n:]).all()) and bool(is_poison(layer.dx_rows[n:]).all())
    assert_rows_close(to_np(dx), bwd["dx"], tol, "dx")
    assert_rows_close(to_np(dwgu).reshape(-1, cfg.d), bwd["dw_gu"].reshape(-1, cfg.d), tol,
                      "dw_gu")
    assert_rows_close(to_np(dwd).reshape(-1, cfg.F), bwd["dw_d"].reshape(-1, cfg.F), tol,
                      "dw_down")
    # router-weight and logit gradients: within the bound that y's row
    # tolerance implies (plus the fp32 accumulation of the dot)
    dwb = dw_bound(_f64(dout), fwd["y"], fwd["dest_rank"], fwd["dest_row"], cfg.ep_rank)
    assert_bounded(to_np(layer.dw), bwd["dw"], dwb, tol + ACC_TOL, "dw")
    dlb = dlogit_bound(fwd["topk_idx"], fwd["topk_w"], dwb, cfg.N)
    assert_bounded(to_np(dl), bwd["dlogits"], dlb, tol + ACC_TOL, "dlogits")


def test_backward_shards_sum_to_unsharded_on_gpu():
    """Expert-parallel shards: the per-rank dx and dlogits add up to the
    unsharded layer's, and each rank's weight gradients are its slice of the
    unsharded ones (AWS Neuron EP design; each rank holds E_L experts)."""
    base = SMALL[1].with_(name="shard_sum_bf16", T=400, N=16, seed=31)
    inp = make_inputs(base, "cpu")
    dout = random_rows(base.T, base.d, base.torch_dtype, seed=77).cuda()
    logits, x = inp.logits.cuda(), inp.x.cuda()
    full = moe.MoELayer(moe.MoeShape.from_config(base), "cuda")
    full.forward(logits, x, inp.w_gu.cuda(), inp.w_d.cuda())
    fdx, fdl, fgu, fd = [t.clone() for t in full.backward(dout, inp.w_gu.cuda(), inp.w_d.cuda())]
    ep = 4
    E_L = base.N // ep
    dx = torch.zeros(base.T, base.d, dtype=torch.float64, device="cuda")
    dl = torch.zeros(base.T, base.N, dtype=torch.float64, device="cuda")
    for r in range(ep):
        cfg = base.with_(ep_size=ep, ep_rank=r)
        sl = slice(r * E_L, (r + 1) * E_L)
        lay = moe.MoELayer(moe.MoeShape.from_config(cfg), "cuda")
        wg, wd = inp.w_gu[sl].contiguous().cuda(), inp.w_d[sl].contiguous().cuda()
        lay.forward(logits, x, wg, wd)
        a, b, c, e = lay.backward(dout, wg, wd)
        dx += a.double()
        dl += b.double()
        # the same rows in the same order on the shard: identical results
        torch.testing.assert_close(c, fgu[sl], rtol=0, atol=0)
        torch.testing.assert_close(e, fd[sl], rtol=0, atol=0)
    torch.cuda.synchronize()
    assert_rows_close(dx.cpu().numpy(), to_np(fdx), 2e-2, "dx shard sum")
    fdl = to_np(fdl)
    np.testing.assert_allclose(dl.cpu().numpy(), fdl, rtol=1e-5, atol=1e-6 * np.abs(fdl).max())


FULL = ["tiny_f32", "olmoe_bf16", "gptoss_shard_bf16", "zipf_skew_bf16", "finegrained_shard_bf16",
        "zipf_dropless_bf16"]


@pytest.mark.parametrize("name", ["olmoe_bf16", "gptoss_shard_bf16"])
def test_full_config_saved_gu_layer(name):
    """Full workload sizes: MoELayer.forward(save_gu=True) + backward gives the
    outputs and every gradient of forward + backward with the recompute, bit
    for bit (the oracle check of that path is test_full_config_backward)."""
    from combine_top_softmax_amd.workloads import CONFIGS
    cfg = CONFIGS[name]
    print(f"[case] full saved gu {name}", flush=True)
    inp = make_inputs(cfg, "cuda")
    dout = random_rows(cfg.T, cfg.d, cfg.torch_dtype, seed=cfg.seed + 900).cuda()
    layer = moe.MoELayer(moe.MoeShape.from_config(cfg), "cuda")
    got = []
    for save in (False, True):
        out = layer.forward(inp.logits, inp.x, inp.w_gu, inp.w_d, save_gu=save).clone()
        h = layer.h.clone()
        grads = [t.clone() for t in layer.backward(dout, inp.w_gu, inp.w_d)]
        got.append([out, h, layer.dw.clone(), layer.dx_rows.clone()] + grads)
        assert not layer.gu_saved
    torch.cuda.synchronize()
    n = int(layer.route.offsets[cfg.ep_rank, -1])
    names = ["out", "h", "dw", "dx_rows", "dx", "dlogits", "dw_gu", "dw_down"]
    for nm, a, b in zip(names, *got):
        if nm in ("h", "dx_rows"):
            a, b = a[:n], b[:n]
        assert torch.equal(a, b), f"{nm} differs with the saved [G U]"


@pytest.mark.parametrize("name", FULL)
def test_full_config_backward(name):
    """Full workload sizes, MoELayer.forward + backward as one stream of calls.
    The oracle recomputes sampled tokens (dx, dw, dlogits, dy rows) and the
    weight gradients of sampled experts one by one in float64 from the same
    seeded inputs and route map."""
    from combine_top_softmax_amd.workloads import CONFIGS
    cfg = CONFIGS[name]
    print(f"[case] full backward {name}", flush=True)
    inp = make_inputs(cfg, "cuda")
    shape = moe.MoeShape.from_config(cfg)
    dt = cfg.torch_dtype
    dout_cpu = random_rows(cfg.T, cfg.d, dt, seed=cfg.seed + 900)
    layer = moe.MoELayer(shape, "cuda")
    layer.forward(inp.logits, inp.x, inp.w_gu, inp.w_d)
    dx, dl, dwgu, dwd = layer.backward(dout_cpu.cuda(), inp.w_gu, inp.w_d)
    torch.cuda.synchronize()

    ref = oracle_route(cfg, inp.logits.cpu())
    K, E_L, d, F = cfg.K, cfg.E_L, cfg.d, cfg.F
    off = ref["offsets"][cfg.ep_rank]
    x = _f64(inp.x.cpu())
    dout = _f64(dout_cpu)
    tol = tol_of(cfg.dtype)
    rng = np.random.default_rng(cfg.seed + 1)
    w_cache = {}

    def weights(j):
        if j not in w_cache:
            w_cache[j] = (_f64(inp.w_gu[j].cpu()), _f64(inp.w_d[j].cpu()))
        return w_cache[j]

    # sampled tokens: every kept local route recomputed row by row
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.integers(0, cfg.T, size=24)]))
    dx_ref = np.zeros((len(toks), d))
    dw_ref = np.zeros((len(toks), K))
    dwb = np.zeros((len(toks), K))
    dy_rows, dy_ref = [], []
    for i, t in enumerate(toks):
        dX = np.zeros((K, d))
        drow = np.full((1, K), -1, dtype=np.int32)
        for k in range(K):
            if ref["dest_rank"][t, k] != cfg.ep_rank:
                continue
            j = int(ref["topk_idx"][t, k]) - cfg.ep_rank * E_L
            wg, wd = weights(j)
            H, Y = orc.expert_ffn_rows(x[t:t + 1], wg, wd, cfg.dtype)
            dY = orc.round_to(float(ref["topk_w"][t, k]) * dout[t:t + 1], cfg.dtype)
            b = orc.expert_ffn_bwd_rows(x[t:t + 1], wg, wd, H, dY, cfg.dtype)
            dX[k] = b["dx"][0]
            drow[0, k] = k
            dw_ref[i, k] = float(np.dot(dout[t], Y[0]))
            dwb[i, k] = np.linalg.norm(dout[t]) * np.linalg.norm(Y[0])
            dy_rows.append(int(ref["dest_row"][t, k]))
            dy_ref.append(dY[0])
        dx_ref[i] = orc.dispatch_bwd(dX, ref["dest_rank"][t:t + 1], drow, cfg.ep_rank,
                                     cfg.dtype)[0]
    sel = torch.from_numpy(toks).cuda()
    assert_rows_close(to_np(dx[sel]), dx_ref, tol, "dx")
    assert_bounded(to_np(layer.dw[sel]), dw_ref, dwb, tol + ACC_TOL, "dw")
    dl_ref = orc.route_bwd(ref["topk_idx"][toks], ref["topk_w"][toks], dw_ref, cfg.N)
    dlb = dlogit_bound(ref["topk_idx"][toks], ref["topk_w"][toks], dwb, cfg.N)
    assert_bounded(to_np(dl[sel]), dl_ref, dlb, tol + ACC_TOL, "dlogits")
    if dy_rows:
        got = to_np(layer.dy[torch.tensor(dy_rows).cuda()])
        assert_rows_close(got, np.array(dy_ref), tol, "dy")

    # sampled experts: whole weight gradients over all of the expert's rows
    nonempty = [j for j in range(E_L) if off[j + 1] > off[j]]
    experts = sorted({nonempty[0], int(rng.choice(nonempty))})
    for j in experts:
        a, b = int(off[j]), int(off[j + 1])
        src = ref["row_src"][a:b]
        t_of, k_of = src // K, src % K
        X = x[t_of]
        wg, wd = weights(j)
        H, _ = orc.expert_ffn_rows(X, wg, wd, cfg.dtype)
        dY = orc.round_to(ref["topk_w"][t_of, k_of][:, None].astype(np.float64) * dout[t_of],
                          cfg.dtype)
        r = orc.expert_ffn_bwd_rows(X, wg, wd, H, dY, cfg.dtype)
        assert_rows_close(to_np(dwgu[j]), r["dw_gu"], tol, f"dw_gu expert {j}")
        assert_rows_close(to_np(dwd[j]), r["dw_d"], tol, f"dw_down expert {j}")
        rr = np.unique(np.concatenate([[0, b - a - 1], rng.integers(0, b - a, size=16)]))
        rows_dev = torch.from_numpy(rr + a).cuda()
        assert_rows_close(to_np(layer.gu[rows_dev]), r["dgu"][rr], tol, f"dgu expert {j}")
        assert_rows_close(to_np(layer.dx_rows[rows_dev]), r["dx"][rr], tol, f"dx_rows expert {j}")
