"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (``MoELayer.forward``: four calls back to back on one stream).

Routing metadata is compared bit-exactly on the whole tensors. The dispatch
buffer is checked bit-exactly on sampled rows; expert outputs on sampled rows
of sampled experts, and the combined output on sampled tokens, each recomputed
one by one by the oracle in float64 from the same seeded inputs.
"""
import numpy as np
import pytest
import torch

import combine_top_softmax_amd as moe
from combine_top_softmax_amd.workloads import CONFIGS, make_inputs
from oracle import moe_oracle as orc
from gpu_util import assert_rows_close, check_route, oracle_route, poison_, to_np, tol_of

pytestmark = pytest.mark.gpu

FULL = ["tiny_f32", "olmoe_bf16", "gptoss_shard_bf16", "zipf_skew_bf16", "finegrained_shard_bf16",
        "zipf_dropless_bf16"]


@pytest.mark.parametrize("name", FULL)
def test_full_config_parity(name):
    cfg = CONFIGS[name]
    print(f"[case] full {name}", flush=True)
    inp = make_inputs(cfg, "cuda")
    shape = moe.MoeShape.from_config(cfg)
    layer = moe.MoELayer(shape, "cuda")
    for t in (layer.buf, layer.h, layer.y, layer.out):
        poison_(t)
    layer.forward(inp.logits, inp.x, inp.w_gu, inp.w_d)
    torch.cuda.synchronize()

    logits = inp.logits.cpu()
    ref = oracle_route(cfg, logits)
    check_route(layer.route, ref, shape)
    rng = np.random.default_rng(cfg.seed)
    n = int(ref["offsets"][cfg.ep_rank, -1])
    K = cfg.K
    x_cpu = inp.x.cpu()
    assert n > 0

    # dispatch: sampled prefix rows are exact copies of their source token
    rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, size=256)]))
    src_tok = ref["row_src"][rows] // K
    got = layer.buf[torch.from_numpy(rows).cuda()].cpu()
    assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                       (x_cpu[torch.from_numpy(src_tok)].view(torch.int16)
                        if got.dtype == torch.bfloat16 else x_cpu[torch.from_numpy(src_tok)]))

    # expert FFN on sampled rows of sampled experts
    off = ref["offsets"][cfg.ep_rank]
    E_L = cfg.E_L
    nonempty = [j for j in range(E_L) if off[j + 1] > off[j]]
    experts = sorted(set([nonempty[0], nonempty[-1]] +
                         list(rng.choice(nonempty, size=min(3, len(nonempty)), replace=False))))
    tol = tol_of(cfg.dtype)
    w_cache = {}

    def weights(j):
        if j not in w_cache:
            w_cache[j] = (inp.w_gu[j].cpu().double().numpy(), inp.w_d[j].cpu().double().numpy())
        return w_cache[j]

    for j in experts:
        a, b = int(off[j]), int(off[j + 1])
        rr = np.unique(np.concatenate([[a, b - 1], rng.integers(a, b, size=12)]))
        X = x_cpu[torch.from_numpy(ref["row_src"][rr] // K)].double().numpy()
        wg, wd = weights(j)
        H, Y = orc.expert_ffn_rows(X, wg, wd, cfg.dtype)
        sel = torch.from_numpy(rr).cuda()
        assert_rows_close(to_np(layer.h[sel]), H, tol, f"h expert {j}")
        assert_rows_close(to_np(layer.y[sel]), Y, tol, f"y expert {j}")

    # combine on sampled tokens, expert rows recomputed by the oracle
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.integers(0, cfg.T, size=24)]))

    def y_of_row(row):
        j = int(np.searchsorted(off, row, side="right") - 1)
        t = int(ref["row_src"][row] // K)
        wg, wd = weights(j)
        return orc.expert_ffn_rows(x_cpu[t:t + 1].double().numpy(), wg, wd, cfg.dtype)[1][0]

    expect = orc.combine_tokens(toks, y_of_row, ref["dest_rank"], ref["dest_row"],
                                ref["topk_w"], cfg.ep_rank, cfg.d, cfg.dtype)
    got = to_np(layer.out[torch.from_numpy(toks).cuda()])
    assert_rows_close(got, expect, tol, "out")
