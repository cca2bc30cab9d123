"""moe_route_noalloc: moe_route on the library's static per-GPU scratch array
(no workspace argument, no allocation). Its outputs must equal moe_route's bit
for bit on consecutive calls, the second with a smaller input (the array keeps
the previous call's contents), and shapes whose workspace does not fit the
array are refused on the host."""
import ctypes
from fractions import Fraction

import pytest
import torch

import combine_top_softmax_amd as moe
from combine_top_softmax_amd import _abi
from combine_top_softmax_amd.workloads import CONFIGS, LayerConfig, make_inputs

FIELDS = ("topk_idx", "topk_w", "dest_rank", "dest_row", "drop_mask", "counts", "offsets",
          "row_src")


def test_noalloc_refuses_shapes_past_its_scratch():
    lib = _abi.load()
    big = moe.MoeShape(T=800_000, d=64, N=256, K=8, F=64, ep_size=1, ep_rank=0, capacity=100,
                       dtype="bf16")
    assert moe.moe_route_workspace_size(big) > _abi.MOE_NOALLOC_SCRATCH_BYTES
    out = _abi.moe_route_out_t(16, 16, 16, 16, 16, 16, 16, None)
    assert lib.moe_route_noalloc(ctypes.byref(big.c()), 16, ctypes.byref(out), None) == \
        _abi.MOE_ESCRATCH
    fits = moe.MoeShape(T=600_000, d=64, N=256, K=8, F=64, ep_size=1, ep_rank=0, capacity=100,
                        dtype="bf16")
    assert moe.moe_route_workspace_size(fits) <= _abi.MOE_NOALLOC_SCRATCH_BYTES
    bad = moe.MoeShape(T=64, d=64, N=8, K=9, F=64, ep_size=1, ep_rank=0, capacity=8,
                       dtype="bf16")
    assert lib.moe_route_noalloc(ctypes.byref(bad.c()), 16, ctypes.byref(out), None) == \
        _abi.MOE_EINVAL
    ok = moe.MoeShape(T=64, d=64, N=8, K=2, F=64, ep_size=1, ep_rank=0, capacity=8, dtype="bf16")
    assert lib.moe_route_noalloc(ctypes.byref(ok.c()), 8, ctypes.byref(out), None) == \
        _abi.MOE_EALIGN
    assert "scratch" in moe.moe_strerror(_abi.MOE_ESCRATCH)


def _poisoned(shape, fill):
    out = moe.RouteOut.empty(shape, "cuda")
    for name in FIELDS:
        t = getattr(out, name)
        if t.dtype == torch.float32:
            t.view(torch.int32).fill_(fill)
        else:
            t.fill_(fill)
    return out


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


@pytest.mark.gpu
def test_noalloc_route_equals_moe_route_on_consecutive_calls():
    """Three calls in a row on one stream: the OLMoE-shaped layer's routing,
    then a smaller expert-sharded Zipf layer that drops routes, then an empty
    batch; each against moe_route with a caller-owned workspace, bit for
    bit."""
    cases = [CONFIGS["olmoe_bf16"],
             LayerConfig("noalloc_small", T=1000, d=64, N=16, K=4, F=64, cf=Fraction(1),
                         dtype="bf16", ep_size=2, ep_rank=1, logits="zipf", seed=51),
             LayerConfig("noalloc_empty", T=0, d=64, N=16, K=4, F=64, cf=Fraction(1),
                         dtype="bf16", seed=52, dropless=True)]
    for cfg in cases:
        print(f"[case] noalloc {cfg.name}", flush=True)
        shape = moe.MoeShape.from_config(cfg)
        inp = make_inputs(cfg, "cuda", with_weights=False)
        ref = _poisoned(shape, -7)
        ws = torch.full((moe.moe_route_workspace_size(shape),), 0xA5, dtype=torch.uint8,
                        device="cuda")
        moe.moe_route(shape, inp.logits, ref, ws)
        got = _poisoned(shape, -3)
        moe.moe_route_noalloc(shape, inp.logits, got)
        torch.cuda.synchronize()
        for name in FIELDS:
            a, b = _bits(getattr(got, name)), _bits(getattr(ref, name))
            assert torch.equal(a, b), f"{cfg.name}: {name} differs from moe_route's"
        if cfg.T > 0:
            assert int(got.drop_mask.sum()) == int(ref.drop_mask.sum())
