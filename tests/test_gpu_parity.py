"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: bit-exact for ids, route map, counts, offsets, drop mask, row_src and the
dispatch-buffer prefix; relative 1e-6 for routing weights; per-row relative L2
<= 2e-2 (bf16) or 1e-4 (fp32) for H, Y and the combined output, with rows the
oracle gives as exact zeros required to be exact zeros. Every capacity tail
is poisoned (NaN bit pattern) before the call and must be untouched after it.
"""
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import combine_top_softmax_amd as moe
from combine_top_softmax_amd.workloads import LayerConfig, CONFIGS, make_inputs, random_rows, random_ids
from oracle import moe_oracle as orc
from gpu_util import (assert_route_fields, assert_row_src, assert_rows_close, check_route,
                      is_poison, oracle_route, poison_, route_gpu, to_np, tol_of)

pytestmark = pytest.mark.gpu

SMALL = [
    CONFIGS["tiny_f32"],
    LayerConfig("small_bf16", T=1000, d=256, N=16, K=4, F=192, cf=Fraction(5, 4),
                dtype="bf16", seed=11),
    LayerConfig("small_shard_bf16", T=777, d=384, N=32, K=4, F=256, cf=Fraction(1),
                dtype="bf16", ep_size=4, ep_rank=1, seed=12),
    LayerConfig("small_zipf_drops_bf16", T=1500, d=128, N=24, K=3, F=136, cf=Fraction(1),
                dtype="bf16", logits="zipf", zipf_s=1.1, seed=13),
    LayerConfig("ragged_shard_f32", T=333, d=72, N=6, K=2, F=40, cf=Fraction(1), dtype="f32",
                ep_size=3, ep_rank=2, seed=14),
    LayerConfig("k_equals_n_bf16", T=130, d=64, N=16, K=16, F=64, cf=Fraction(1, 2),
                dtype="bf16", seed=15),
    LayerConfig("d2880_slice_bf16", T=512, d=2880, N=32, K=4, F=320, cf=Fraction(1),
                dtype="bf16", ep_size=8, ep_rank=5, seed=16),
    LayerConfig("many_experts_bf16", T=300, d=64, N=320, K=8, F=64, cf=Fraction(2),
                dtype="bf16", ep_size=2, ep_rank=1, seed=17),
    # dropless (capacity T, upper-bound buffers) on skewed routing
    LayerConfig("small_zipf_dropless_bf16", T=1500, d=128, N=24, K=3, F=136, cf=Fraction(1),
                dtype="bf16", logits="zipf", zipf_s=1.1, seed=13, dropless=True),
    LayerConfig("dropless_shard_zipf_bf16", T=777, d=384, N=32, K=4, F=256, cf=Fraction(1),
                dtype="bf16", ep_size=4, ep_rank=0, logits="zipf", zipf_s=1.1, seed=18,
                dropless=True),
]


def _to_dev(inp):
    return SimpleNamespace(logits=inp.logits.cuda(), x=inp.x.cuda(), w_gu=inp.w_gu.cuda(),
                           w_d=inp.w_d.cuda())


def _run_layer_stages(cfg, inp_dev):
    """Run the four stages on the GPU with poisoned buffers; return a dict."""
    shape = moe.MoeShape.from_config(cfg)
    layer = moe.MoELayer(shape, "cuda")
    for t in (layer.buf, layer.h, layer.y, layer.out):
        poison_(t)
    layer.route_step(inp_dev.logits)
    layer.dispatch_step(inp_dev.x)
    layer.up_step(inp_dev.w_gu)
    layer.down_step(inp_dev.w_d)
    layer.combine_step()
    torch.cuda.synchronize()
    return shape, layer


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_layer_stages_match_oracle(cfg):
    print(f"[case] {cfg.name}", flush=True)
    inp = make_inputs(cfg, "cpu")
    shape, layer = _run_layer_stages(cfg, _to_dev(inp))

    ref = orc.moe_layer(inp.logits.numpy(), inp.x.to(torch.float64).numpy(),
                        inp.w_gu.to(torch.float64).numpy(), inp.w_d.to(torch.float64).numpy(),
                        cfg.K, cfg.capacity, cfg.ep_size, cfg.ep_rank, cfg.dtype)
    check_route(layer.route, ref, shape)
    n = int(ref["offsets"][cfg.ep_rank, -1])
    # dispatch: bit-exact prefix, untouched tail
    np.testing.assert_array_equal(to_np(layer.buf[:n]), ref["buf"][:n])
    assert bool(is_poison(layer.buf[n:]).all())
    # expert FFN: H and Y prefix within tolerance, tails untouched
    tol = tol_of(cfg.dtype)
    if n > 0:
        assert_rows_close(to_np(layer.h[:n]), ref["h"][:n], tol, "h")
        assert_rows_close(to_np(layer.y[:n]), ref["y"][:n], tol, "y")
    assert bool(is_poison(layer.h[n:]).all()) and bool(is_poison(layer.y[n:]).all())
    # combine
    assert_rows_close(to_np(layer.out), ref["out"], tol, "out")


@pytest.mark.parametrize("cfg", [c for c in SMALL if c.dropless], ids=lambda c: c.name)
def test_dropless_keeps_every_route(cfg):
    """Dropless mode (capacity T, upper-bound buffers of moe_buffer_rows rows):
    on skewed routing that drops routes at capacity factor 1, every local
    route is kept and packed, and the buffers are smaller than the E_L*C
    envelope. Sync-free: the whole layer runs with host syncs forbidden."""
    print(f"[case] dropless {cfg.name}", flush=True)
    inp = make_inputs(cfg, "cpu")
    capped = cfg.with_(dropless=False)
    assert int(oracle_route(capped, inp.logits)["drop_mask"].sum()) > 0
    shape = moe.MoeShape.from_config(cfg)
    assert shape.rows == cfg.T * min(cfg.K, cfg.E_L) < cfg.E_L * cfg.capacity
    layer = moe.MoELayer(shape, "cuda")
    dev = _to_dev(inp)
    torch.cuda.synchronize()
    torch.cuda.set_sync_debug_mode("error")
    try:
        layer.forward(dev.logits, dev.x, dev.w_gu, dev.w_d)
    finally:
        torch.cuda.set_sync_debug_mode(0)
    torch.cuda.synchronize()
    idx = to_np(layer.route.topk_idx)
    local = (idx // cfg.E_L) == cfg.ep_rank
    assert int(to_np(layer.route.drop_mask).sum()) == 0
    assert np.array_equal(to_np(layer.route.dest_rank) >= 0, np.ones_like(local))
    n = int(to_np(layer.route.offsets)[cfg.ep_rank, -1])
    assert n == int(local.sum())
    rows = to_np(layer.route.dest_row)[local]
    assert np.array_equal(np.sort(rows), np.arange(n))   # a permutation of the prefix


@pytest.mark.parametrize("cfg", SMALL[:4], ids=lambda c: c.name)
def test_combine_alone_matches_oracle(cfg):
    """Combine on stand-in expert rows (seeded, not computed by the HIP path)."""
    inp = make_inputs(cfg, "cpu", with_weights=False)
    ref = oracle_route(cfg, inp.logits)
    shape = moe.MoeShape.from_config(cfg)
    y = random_rows(shape.rows, cfg.d, cfg.torch_dtype, seed=cfg.seed + 100)
    expect = orc.combine(y.to(torch.float64).numpy(), ref["dest_rank"], ref["dest_row"],
                         ref["topk_w"], cfg.ep_rank, cfg.dtype)
    out = poison_(torch.empty(cfg.T, cfg.d, dtype=cfg.torch_dtype, device="cuda"))
    moe.moe_combine(shape, y.cuda(), torch.from_numpy(ref["dest_rank"]).cuda(),
                    torch.from_numpy(ref["dest_row"]).cuda(),
                    torch.from_numpy(ref["topk_w"]).cuda(), out)
    assert_rows_close(to_np(out), expect, tol_of(cfg.dtype), "combine")


def test_route_map_fig16_on_gpu(golden_dir):
    import json, os
    with open(os.path.join(golden_dir, "fig16_route_map.json")) as f:
        g = json.load(f)
    ids = torch.tensor(g["ids"], dtype=torch.int32)
    for ep_rank in (0, 1):
        shape = moe.MoeShape(T=10, d=8, N=4, K=2, F=8, ep_size=2, ep_rank=ep_rank,
                             capacity=g["capacity_min"], dtype="bf16")
        out = moe.RouteOut.empty(shape, "cuda")
        ws = torch.empty(moe.moe_route_workspace_size(shape), dtype=torch.uint8, device="cuda")
        moe.moe_route_map(shape, ids.cuda(), out, ws)
        torch.cuda.synchronize()
        assert to_np(out.dest_rank).tolist() == g["dest_rank"]
        assert to_np(out.dest_row).tolist() == g["dest_row"]
        assert int(to_np(out.offsets)[0, -1]) == g["rank0_rows_used"]
        ref = orc.route_map(ids.numpy(), 4, 2, g["capacity_min"], ep_rank)
        assert_row_src(to_np(out.row_src), ref["row_src"])
        np.testing.assert_array_equal(to_np(out.drop_mask), ref["drop_mask"])


@pytest.mark.parametrize("T,N,K,C,ep,frac", [
    (1000, 64, 8, 100, 4, 0.1), (65, 5, 5, 13, 5, 0.3), (4097, 256, 6, 40, 8, 0.02),
    (1, 1, 1, 1, 1, 0.0),
    # both sides of each bound of the two-kernel route (N <= 256, <= 256 tiles,
    # N * tiles <= 16384) and each group width of its column sums
    (1000, 256, 8, 40, 4, 0.05), (4000, 257, 4, 30, 1, 0.0), (16384, 64, 2, 600, 2, 0.01),
    (16385, 64, 2, 600, 2, 0.0), (300, 3, 2, 150, 1, 0.1), (5000, 100, 8, 300, 5, 0.02)])
def test_route_map_random_ids_with_invalid(T, N, K, C, ep, frac):
    ids = random_ids(T, N, K, seed=T + N, invalid_frac=frac)
    for ep_rank in sorted({0, ep - 1}):
        shape = moe.MoeShape(T=T, d=8, N=N, K=K, F=8, ep_size=ep, ep_rank=ep_rank, capacity=C,
                             dtype="f32")
        out = moe.RouteOut.empty(shape, "cuda")
        ws = torch.empty(moe.moe_route_workspace_size(shape), dtype=torch.uint8, device="cuda")
        moe.moe_route_map(shape, ids.cuda(), out, ws)
        ref = orc.route_map(ids.numpy(), N, ep, C, ep_rank)
        ref["topk_idx"] = ids.numpy()
        torch.cuda.synchronize()
        assert_route_fields(out, ref, ("counts", "offsets", "dest_rank", "dest_row",
                                       "drop_mask", "row_src"))


@pytest.mark.parametrize("case", ["single_token", "one_expert", "constant_logits", "capacity_one"])
def test_degenerate_routing(case):
    if case == "single_token":
        cfg = LayerConfig(case, T=1, d=64, N=8, K=3, F=64, cf=Fraction(1), dtype="bf16", seed=21)
    elif case == "one_expert":
        cfg = LayerConfig(case, T=200, d=64, N=1, K=1, F=64, cf=Fraction(1, 4), dtype="bf16", seed=22)
    elif case == "constant_logits":
        cfg = LayerConfig(case, T=300, d=64, N=12, K=4, F=64, cf=Fraction(1), dtype="f32", seed=23)
    else:
        cfg = LayerConfig(case, T=150, d=64, N=64, K=2, F=64, cf=Fraction(1, 5), dtype="bf16",
                          ep_size=4, ep_rank=3, seed=24)
    inp = make_inputs(cfg, "cpu")
    if case == "constant_logits":
        inp.logits.zero_()
    shape, layer = _run_layer_stages(cfg, _to_dev(inp))
    ref = orc.moe_layer(inp.logits.numpy(), inp.x.to(torch.float64).numpy(),
                        inp.w_gu.to(torch.float64).numpy(), inp.w_d.to(torch.float64).numpy(),
                        cfg.K, cfg.capacity, cfg.ep_size, cfg.ep_rank, cfg.dtype)
    check_route(layer.route, ref, shape)
    assert_rows_close(to_np(layer.out), ref["out"], tol_of(cfg.dtype), "out")
    if case == "constant_logits":
        assert int(ref["drop_mask"].sum()) > 0


def test_shard_partial_outputs_sum_to_full_layer():
    """AWS Neuron EP design: per-rank partial outputs add up to the full layer."""
    cfg = LayerConfig("shard_sum_f32", T=400, d=64, N=16, K=4, F=96, cf=Fraction(5, 4),
                      dtype="f32", seed=31)
    inp = make_inputs(cfg, "cpu")
    full = orc.moe_layer(inp.logits.numpy(), inp.x.to(torch.float64).numpy(),
                         inp.w_gu.to(torch.float64).numpy(), inp.w_d.to(torch.float64).numpy(),
                         cfg.K, cfg.capacity, 1, 0, "f32")["out"]
    ep = 4
    E_L = cfg.N // ep
    total = torch.zeros(cfg.T, cfg.d, dtype=torch.float64)
    for r in range(ep):
        shape = moe.MoeShape(cfg.T, cfg.d, cfg.N, cfg.K, cfg.F, ep, r, cfg.capacity, "f32")
        layer = moe.MoELayer(shape, "cuda")
        layer.forward(inp.logits.cuda(), inp.x.cuda(),
                      inp.w_gu[r * E_L:(r + 1) * E_L].contiguous().cuda(),
                      inp.w_d[r * E_L:(r + 1) * E_L].contiguous().cuda())
        total += layer.out.cpu().double()
    assert_rows_close(total.numpy(), full, 1e-4, "shard sum")


def test_layer_is_deterministic_and_sync_free():
    cfg = SMALL[1]
    inp = make_inputs(cfg, "cuda")
    shape = moe.MoeShape.from_config(cfg)
    layer = moe.MoELayer(shape, "cuda")
    torch.cuda.synchronize()
    torch.cuda.set_sync_debug_mode("error")
    try:
        out1 = layer.forward(inp.logits, inp.x, inp.w_gu, inp.w_d).clone()
        out2 = layer.forward(inp.logits, inp.x, inp.w_gu, inp.w_d).clone()
    finally:
        torch.cuda.set_sync_debug_mode(0)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
