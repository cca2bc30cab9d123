"""ctypes view of the C ABI in include/moe.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

from .build import lib_path

MOE_OK = 0
MOE_EINVAL = -1
MOE_EDTYPE = -2
MOE_EALIGN = -3
MOE_EWORKSPACE = -4
MOE_EHIP = -5
MOE_ESCRATCH = -6
MOE_NOALLOC_SCRATCH_BYTES = 16 << 20
MOE_MAX_K = 16
MOE_MAX_EXPERTS = 1024
MOE_MAX_WIDTH = 1 << 20
MOE_F32 = 0
MOE_BF16 = 1


class moe_shape_t(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("N", ctypes.c_int32),
                ("K", ctypes.c_int32), ("F", ctypes.c_int32), ("ep_size", ctypes.c_int32),
                ("ep_rank", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("dtype", ctypes.c_int)]


class moe_route_out_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "topk_w", "dest_rank", "dest_row", "drop_mask", "counts",
                 "offsets", "row_src")]


_P = ctypes.c_void_p
_SHAPE = ctypes.POINTER(moe_shape_t)
_ROUTE = ctypes.POINTER(moe_route_out_t)

SIGNATURES = {
    "moe_route_workspace_size": (ctypes.c_int, [_SHAPE, ctypes.POINTER(ctypes.c_size_t)]),
    "moe_route": (ctypes.c_int, [_SHAPE, _P, _ROUTE, _P, ctypes.c_size_t, _P]),
    "moe_route_map": (ctypes.c_int, [_SHAPE, _P, _ROUTE, _P, ctypes.c_size_t, _P]),
    "moe_route_noalloc": (ctypes.c_int, [_SHAPE, _P, _ROUTE, _P]),
    "moe_dispatch_rows": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _P]),
    "moe_expert_ffn": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _P, _P, _P]),
    "moe_buffer_rows": (ctypes.c_int64, [_SHAPE]),
    "moe_expert_up": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _P]),
    "moe_expert_up_save_gu": (ctypes.c_int, [_SHAPE] + [_P] * 6),
    "moe_expert_down": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _P]),
    "moe_combine": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _P, _P]),
    "moe_combine_bwd": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn_bwd": (ctypes.c_int, [_SHAPE] + [_P] * 12),
    "moe_expert_ffn_bwd_data": (ctypes.c_int, [_SHAPE] + [_P] * 9),
    "moe_expert_ffn_bwd_data_saved_gu": (ctypes.c_int, [_SHAPE] + [_P] * 8),
    "moe_expert_ffn_bwd_weight": (ctypes.c_int, [_SHAPE] + [_P] * 8),
    "moe_dispatch_bwd": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _P]),
    "moe_route_bwd": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _P]),
    "moe_mx_quantize_rows": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, _P, _P, _P, _P]),
    "moe_dispatch_rows_mx": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _P, _P]),
    "moe_expert_up_mx": (ctypes.c_int, [_SHAPE] + [_P] * 8),
    "moe_expert_down_mx": (ctypes.c_int, [_SHAPE] + [_P] * 7),
    "moe_expert_ffn_mx": (ctypes.c_int, [_SHAPE] + [_P] * 11),
    "moe_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_validate_shape": (ctypes.c_int, [_SHAPE]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree libmoe_hip.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"HIP extension {path} is missing: build it with "
                "`python -m combine_top_softmax_amd.build` (or __graft_entry__.build()).")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        msg = load().moe_strerror(code).decode()
        super().__init__(f"{fn} failed with code {code}: {msg}")


def check(fn: str, code: int) -> None:
    if code != MOE_OK:
        raise MoeError(fn, code)
