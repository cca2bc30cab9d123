"""The C-ABI library loads and exports every symbol include/moe.h declares,
and host-side validation rejects bad shapes before anything is enqueued.
No GPU needed: invalid calls return before any HIP call."""
import ctypes
import os
import re

import pytest

import combine_top_softmax_amd as moe
from combine_top_softmax_amd import _abi
from combine_top_softmax_amd.workloads import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _abi.load()
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"
    assert set(names) == set(_abi.SIGNATURES), "binding and header disagree"


def test_every_named_workload_is_a_valid_shape():
    for cfg in CONFIGS.values():
        s = moe.MoeShape.from_config(cfg)
        assert moe.moe_validate_shape(s) == 0
        assert moe.moe_route_workspace_size(s) > 0


BASE = dict(T=64, d=64, N=8, K=2, F=64, ep_size=2, ep_rank=1, capacity=16, dtype="bf16")


@pytest.mark.parametrize("bad,code", [
    (dict(T=-1), _abi.MOE_EINVAL), (dict(d=0), _abi.MOE_EINVAL), (dict(K=9), _abi.MOE_EINVAL),
    (dict(K=0), _abi.MOE_EINVAL), (dict(N=9), _abi.MOE_EINVAL), (dict(ep_rank=2), _abi.MOE_EINVAL),
    (dict(ep_rank=-1), _abi.MOE_EINVAL), (dict(capacity=0), _abi.MOE_EINVAL),
    (dict(d=60), _abi.MOE_EINVAL), (dict(F=12), _abi.MOE_EINVAL),
    (dict(N=2048, K=2, ep_size=1, ep_rank=0), _abi.MOE_EINVAL),
    (dict(N=32, K=17, ep_size=1, ep_rank=0), _abi.MOE_EINVAL),
    (dict(T=1 << 28, K=8, N=8), _abi.MOE_EINVAL),
    # one expert's weight matrix past 2^31 elements, a row wider than the limit
    (dict(d=1 << 16, F=1 << 14), _abi.MOE_EINVAL),
    (dict(d=_abi.MOE_MAX_WIDTH + 8, F=8), _abi.MOE_EINVAL),
    (dict(F=_abi.MOE_MAX_WIDTH + 8, d=8), _abi.MOE_EINVAL),
    # grouped-GEMM tile count past a 32-bit grid: 2^30 buffer rows of 2F = 2^15
    (dict(T=1 << 27, K=8, N=8, ep_size=1, ep_rank=0, capacity=1 << 27, d=8, F=1 << 14),
     _abi.MOE_EINVAL),
])
def test_validation_rejects_bad_shapes(bad, code):
    s = moe.MoeShape(**{**BASE, **bad})
    assert moe.moe_validate_shape(s) == code


def test_empty_batch_is_a_valid_shape():
    assert moe.moe_validate_shape(moe.MoeShape(**{**BASE, "T": 0})) == 0
    lib = _abi.load()
    s = moe.MoeShape(**{**BASE, "T": 0}).c()
    # with no token, dispatch and combine touch nothing: NULL pointers are fine
    assert lib.moe_dispatch_rows(ctypes.byref(s), None, None, None, None, None) == 0
    assert lib.moe_combine(ctypes.byref(s), None, None, None, None, None, None) == 0


def test_bad_dtype_and_null_pointers_return_codes():
    lib = _abi.load()
    cs = moe.MoeShape(**BASE).c()
    cs.dtype = 7
    assert lib.moe_validate_shape(ctypes.byref(cs)) == _abi.MOE_EDTYPE
    good = moe.MoeShape(**BASE).c()
    # NULL / misaligned pointers are rejected on the host
    assert lib.moe_dispatch_rows(ctypes.byref(good), None, None, None, None, None) == _abi.MOE_EALIGN
    assert lib.moe_combine(ctypes.byref(good), 16, 16, 16, 16, 8, None) == _abi.MOE_EALIGN
    out = _abi.moe_route_out_t(16, 16, 16, 16, 16, 16, 16, None)
    assert lib.moe_route(ctypes.byref(good), 16, ctypes.byref(out), 16, 1, None) == _abi.MOE_EWORKSPACE
    assert lib.moe_route(ctypes.byref(good), 8, ctypes.byref(out), 16, 1 << 20, None) == _abi.MOE_EALIGN
    assert lib.moe_route(None, 16, ctypes.byref(out), 16, 1 << 20, None) == _abi.MOE_EINVAL
    n = ctypes.c_size_t(0)
    assert lib.moe_route_workspace_size(ctypes.byref(good), None) == _abi.MOE_EINVAL
    assert lib.moe_route_workspace_size(ctypes.byref(good), ctypes.byref(n)) == 0 and n.value > 0
    for c in (0, -1, -2, -3, -4, -5, -99):
        assert isinstance(moe.moe_strerror(c), str) and moe.moe_strerror(c)


def test_python_binding_checks_shapes_before_calling():
    import torch
    s = moe.MoeShape(**BASE)
    with pytest.raises(ValueError):
        moe.moe_dispatch_rows(s, torch.zeros(3, 3), None, None, None)


def test_backward_entry_points_validate_on_the_host():
    lib = _abi.load()
    good = moe.MoeShape(**BASE).c()
    assert lib.moe_combine_bwd(ctypes.byref(good), 16, 16, 16, 16, 16, 8, 16, None) == _abi.MOE_EALIGN
    # 11 pointers then the stream: a NULL dw_down
    assert lib.moe_expert_ffn_bwd(ctypes.byref(good), *([16] * 10), None, None) == _abi.MOE_EALIGN
    assert lib.moe_expert_ffn_bwd(ctypes.byref(good), *([16] * 9), 8, 16, None) == _abi.MOE_EALIGN
    assert lib.moe_dispatch_bwd(ctypes.byref(good), None, 16, 16, 16, None) == _abi.MOE_EALIGN
    assert lib.moe_route_bwd(ctypes.byref(good), 16, 16, 16, 2, None) == _abi.MOE_EALIGN
    bad = moe.MoeShape(**{**BASE, "K": 0}).c()
    assert lib.moe_route_bwd(ctypes.byref(bad), 16, 16, 16, 16, None) == _abi.MOE_EINVAL
    assert lib.moe_expert_ffn_bwd(ctypes.byref(bad), *([16] * 11), None) == _abi.MOE_EINVAL
    f32 = moe.MoeShape(**{**BASE, "dtype": "f32"}).c()
    assert lib.moe_combine_bwd(ctypes.byref(f32), 16, 16, 16, 16, 16, 16, None, None) == _abi.MOE_EALIGN
    # an empty batch moves nothing in the row and router steps
    empty = moe.MoeShape(**{**BASE, "T": 0}).c()
    assert lib.moe_combine_bwd(ctypes.byref(empty), *([None] * 7), None) == 0
    assert lib.moe_dispatch_bwd(ctypes.byref(empty), None, None, None, None, None) == 0
    assert lib.moe_route_bwd(ctypes.byref(empty), None, None, None, None, None) == 0


def test_backward_halves_validate_on_the_host():
    lib = _abi.load()
    good = moe.MoeShape(**BASE).c()
    assert lib.moe_expert_ffn_bwd_data(ctypes.byref(good), *([16] * 7), None, None) == _abi.MOE_EALIGN
    assert lib.moe_expert_ffn_bwd_weight(ctypes.byref(good), *([16] * 6), None, None) == _abi.MOE_EALIGN
    bad = moe.MoeShape(**{**BASE, "F": 12}).c()
    assert lib.moe_expert_ffn_bwd_data(ctypes.byref(bad), *([16] * 8), None) == _abi.MOE_EINVAL
    assert lib.moe_expert_ffn_bwd_weight(ctypes.byref(bad), *([16] * 7), None) == _abi.MOE_EINVAL


def test_buffer_rows_bound_the_oracle_prefix():
    """moe_buffer_rows never cuts the packed prefix the oracle's route map
    fills (the kept local routes), and it is reached when every route is
    local and kept (dropless, one rank) or every expert is overfull."""
    import numpy as np
    from combine_top_softmax_amd.workloads import random_ids
    from oracle import moe_oracle as orc
    cases = [(300, 16, 4, 1, 0, 300), (300, 16, 4, 4, 2, 300), (300, 16, 4, 4, 3, 20),
             (257, 5, 5, 1, 0, 7), (64, 64, 8, 8, 7, 64), (1, 4, 2, 2, 1, 1)]
    for T, N, K, ep, r, C in cases:
        ids = random_ids(T, N, K, seed=T + N + C).numpy()
        s = moe.MoeShape(T=T, d=8, N=N, K=K, F=8, ep_size=ep, ep_rank=r, capacity=C, dtype="f32")
        kept = int(orc.route_map(ids, N, ep, C, r)["offsets"][r, -1])
        assert kept <= s.rows, (T, N, K, ep, r, C)
    # dropless on one rank: every route kept, the bound T*K reached exactly
    ids = random_ids(200, 8, 3, seed=5).numpy()
    s = moe.MoeShape(T=200, d=8, N=8, K=3, F=8, ep_size=1, ep_rank=0, capacity=200, dtype="f32")
    rm = orc.route_map(ids, 8, 1, 200, 0)
    assert int(rm["drop_mask"].sum()) == 0 and int(rm["offsets"][0, -1]) == s.rows == 600
    # one-row capacity with every expert over it: the envelope E_L*C reached
    s = moe.MoeShape(T=200, d=8, N=8, K=3, F=8, ep_size=2, ep_rank=1, capacity=1, dtype="f32")
    assert int(orc.route_map(ids, 8, 2, 1, 1)["offsets"][1, -1]) == s.rows == 4


def test_buffer_rows_of_special_shapes():
    lib = _abi.load()
    # an empty batch keeps one-row buffers; a capacity past 2^31 / E_L is valid
    assert moe.MoeShape(**{**BASE, "T": 0}).rows == 2
    big = moe.MoeShape(**{**BASE, "capacity": (1 << 31) - 1})
    assert moe.moe_validate_shape(big) == 0 and big.rows == 64 * 2
    cs = moe.MoeShape(**{**BASE, "K": 0}).c()
    assert lib.moe_buffer_rows(ctypes.byref(cs)) == _abi.MOE_EINVAL
    with pytest.raises(moe.MoeError):
        moe.MoeShape(**{**BASE, "K": 0}).rows


def test_validation_admits_the_bounds_themselves():
    ok = [dict(d=_abi.MOE_MAX_WIDTH, F=8), dict(F=_abi.MOE_MAX_WIDTH, d=8),
          dict(d=1 << 16, F=(1 << 14) - 8)]
    for kw in ok:
        assert moe.moe_validate_shape(moe.MoeShape(**{**BASE, **kw})) == 0, kw


def test_backward_refuses_to_follow_the_mx_forward():
    """MoELayer.backward differentiates the BF16 forward only: after the MXFP8
    forward (or before any forward) it raises before enqueueing anything."""
    import torch
    s = moe.MoeShape(**BASE)
    layer = moe.MoELayer(s, device="cpu")   # host buffers: nothing is launched
    dout = torch.zeros(s.T, s.d, dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="BF16 forward"):
        layer.backward(dout, None, None)
    layer.last_forward = "mx"
    with pytest.raises(RuntimeError, match="inference-only"):
        layer.backward(dout, None, None)
