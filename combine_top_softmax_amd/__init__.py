"""MI355X-native routed-expert MoE forward layer: thin Python binding.

Every step of the layer runs in the HIP library ``libmoe_hip.so`` (C ABI in
``include/moe.h``); this module only checks tensor shapes on the host and
passes device pointers and the current HIP stream. There is no CPU fallback:
if the library is missing, every call raises.

    shape = MoeShape.from_config(cfg)
    layer = MoELayer(shape, device="cuda")      # buffers allocated once
    out = layer.forward(logits, x, w_gu, w_d)   # 4 calls, no host sync
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _abi
from ._abi import MoeError  # noqa: F401

__all__ = [
    "MoeShape", "RouteOut", "MoELayer", "MoeError", "moe_route_workspace_size", "moe_route",
    "moe_route_map", "moe_route_noalloc", "moe_dispatch_rows", "moe_expert_ffn", "moe_expert_up",
    "moe_expert_down", "moe_combine", "moe_combine_bwd", "moe_expert_ffn_bwd",
    "moe_expert_ffn_bwd_data", "moe_expert_ffn_bwd_weight", "moe_expert_up_save_gu",
    "moe_expert_ffn_bwd_data_saved_gu",
    "moe_dispatch_bwd", "moe_route_bwd", "moe_mx_quantize_rows", "moe_dispatch_rows_mx",
    "moe_expert_up_mx", "moe_expert_down_mx", "MxWeights", "mx_scale_cols", "moe_strerror",
    "moe_validate_shape",
]


@dataclass(frozen=True)
class MoeShape:
    T: int
    d: int
    N: int
    K: int
    F: int
    ep_size: int
    ep_rank: int
    capacity: int
    dtype: str  # "f32" | "bf16"

    @classmethod
    def from_config(cls, cfg) -> "MoeShape":
        return cls(cfg.T, cfg.d, cfg.N, cfg.K, cfg.F, cfg.ep_size, cfg.ep_rank,
                   cfg.capacity, cfg.dtype)

    @property
    def E_L(self) -> int:
        return self.N // self.ep_size

    @property
    def rows(self) -> int:
        """Rows of the capacity-shaped buffers (moe_buffer_rows)."""
        r = _abi.load().moe_buffer_rows(ctypes.byref(self.c()))
        if r < 0:
            _abi.check("moe_buffer_rows", int(r))
        return int(r)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def c(self) -> _abi.moe_shape_t:
        if self.dtype not in ("f32", "bf16"):
            raise ValueError(f"dtype must be 'f32' or 'bf16', got {self.dtype!r}")
        return _abi.moe_shape_t(self.T, self.d, self.N, self.K, self.F, self.ep_size,
                                self.ep_rank, self.capacity,
                                _abi.MOE_F32 if self.dtype == "f32" else _abi.MOE_BF16)


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, name: str, shape: tuple, dtype: torch.dtype) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclass
class RouteOut:
    topk_idx: torch.Tensor   # [T,K] int32
    topk_w: torch.Tensor     # [T,K] fp32
    dest_rank: torch.Tensor  # [T,K] int32
    dest_row: torch.Tensor   # [T,K] int32
    drop_mask: torch.Tensor  # [T,K] uint8
    counts: torch.Tensor     # [N] int32
    offsets: torch.Tensor    # [ep_size, E_L+1] int32
    row_src: torch.Tensor | None  # [rows] int32

    @classmethod
    def empty(cls, shape: MoeShape, device="cuda", row_src: bool = True) -> "RouteOut":
        T, K = shape.T, shape.K
        i32 = dict(dtype=torch.int32, device=device)
        return cls(torch.empty(T, K, **i32), torch.empty(T, K, dtype=torch.float32, device=device),
                   torch.empty(T, K, **i32), torch.empty(T, K, **i32),
                   torch.empty(T, K, dtype=torch.uint8, device=device),
                   torch.empty(shape.N, **i32), torch.empty(shape.ep_size, shape.E_L + 1, **i32),
                   torch.empty(shape.rows, **i32) if row_src else None)

    def check(self, shape: MoeShape, need_topk: bool = True) -> None:
        T, K = shape.T, shape.K
        if need_topk:
            _need(self.topk_idx, "topk_idx", (T, K), torch.int32)
            _need(self.topk_w, "topk_w", (T, K), torch.float32)
        _need(self.dest_rank, "dest_rank", (T, K), torch.int32)
        _need(self.dest_row, "dest_row", (T, K), torch.int32)
        _need(self.drop_mask, "drop_mask", (T, K), torch.uint8)
        _need(self.counts, "counts", (shape.N,), torch.int32)
        _need(self.offsets, "offsets", (shape.ep_size, shape.E_L + 1), torch.int32)
        if self.row_src is not None:
            _need(self.row_src, "row_src", (shape.rows,), torch.int32)

    def c(self, need_topk: bool = True) -> _abi.moe_route_out_t:
        return _abi.moe_route_out_t(
            self.topk_idx.data_ptr() if need_topk else None,
            self.topk_w.data_ptr() if need_topk else None,
            self.dest_rank.data_ptr(), self.dest_row.data_ptr(), self.drop_mask.data_ptr(),
            self.counts.data_ptr(), self.offsets.data_ptr(),
            None if self.row_src is None else self.row_src.data_ptr())


# ----------------------------------------------------------------- C ABI calls
def moe_strerror(code: int) -> str:
    return _abi.load().moe_strerror(code).decode()


def moe_validate_shape(shape: MoeShape) -> int:
    return _abi.load().moe_validate_shape(ctypes.byref(shape.c()))


def moe_route_workspace_size(shape: MoeShape) -> int:
    n = ctypes.c_size_t(0)
    _abi.check("moe_route_workspace_size",
               _abi.load().moe_route_workspace_size(ctypes.byref(shape.c()), ctypes.byref(n)))
    return n.value


def _ws_check(ws: torch.Tensor, shape: MoeShape) -> None:
    need = moe_route_workspace_size(shape)
    if ws.device.type != "cuda" or ws.numel() * ws.element_size() < need or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous device tensor of >= {need} bytes")


def moe_route(shape: MoeShape, logits: torch.Tensor, out: RouteOut, ws: torch.Tensor,
              stream=None) -> None:
    _need(logits, "logits", (shape.T, shape.N), torch.float32)
    out.check(shape)
    _ws_check(ws, shape)
    rc = _abi.load().moe_route(ctypes.byref(shape.c()), _ptr(logits), ctypes.byref(out.c()),
                               _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _abi.check("moe_route", rc)


def moe_route_noalloc(shape: MoeShape, logits: torch.Tensor, out: RouteOut,
                      stream=None) -> None:
    """moe_route on the library's static per-GPU scratch: no workspace, no
    allocation (see include/moe.h for its size limit and sharing rules)."""
    _need(logits, "logits", (shape.T, shape.N), torch.float32)
    out.check(shape)
    rc = _abi.load().moe_route_noalloc(ctypes.byref(shape.c()), _ptr(logits),
                                       ctypes.byref(out.c()), _stream(stream))
    _abi.check("moe_route_noalloc", rc)


def moe_route_map(shape: MoeShape, topk_idx_in: torch.Tensor, out: RouteOut, ws: torch.Tensor,
                  stream=None) -> None:
    _need(topk_idx_in, "topk_idx_in", (shape.T, shape.K), torch.int32)
    out.check(shape, need_topk=False)
    _ws_check(ws, shape)
    rc = _abi.load().moe_route_map(ctypes.byref(shape.c()), _ptr(topk_idx_in),
                                   ctypes.byref(out.c(need_topk=False)), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream))
    _abi.check("moe_route_map", rc)


def moe_dispatch_rows(shape: MoeShape, x, dest_rank, dest_row, buf, stream=None) -> None:
    dt = shape.torch_dtype
    _need(x, "x", (shape.T, shape.d), dt)
    _need(dest_rank, "dest_rank", (shape.T, shape.K), torch.int32)
    _need(dest_row, "dest_row", (shape.T, shape.K), torch.int32)
    _need(buf, "buf", (shape.rows, shape.d), dt)
    rc = _abi.load().moe_dispatch_rows(ctypes.byref(shape.c()), _ptr(x), _ptr(dest_rank),
                                       _ptr(dest_row), _ptr(buf), _stream(stream))
    _abi.check("moe_dispatch_rows", rc)


def _ffn_checks(shape, offsets):
    _need(offsets, "offsets", (shape.ep_size, shape.E_L + 1), torch.int32)


def moe_expert_up(shape: MoeShape, buf, offsets, w_gu, h, stream=None) -> None:
    dt = shape.torch_dtype
    _need(buf, "buf", (shape.rows, shape.d), dt)
    _ffn_checks(shape, offsets)
    _need(w_gu, "w_gu", (shape.E_L, 2 * shape.F, shape.d), dt)
    _need(h, "h", (shape.rows, shape.F), dt)
    rc = _abi.load().moe_expert_up(ctypes.byref(shape.c()), _ptr(buf), _ptr(offsets),
                                   _ptr(w_gu), _ptr(h), _stream(stream))
    _abi.check("moe_expert_up", rc)


def moe_expert_up_save_gu(shape: MoeShape, buf, offsets, w_gu, h, gu, stream=None) -> None:
    dt = shape.torch_dtype
    _need(buf, "buf", (shape.rows, shape.d), dt)
    _ffn_checks(shape, offsets)
    _need(w_gu, "w_gu", (shape.E_L, 2 * shape.F, shape.d), dt)
    _need(h, "h", (shape.rows, shape.F), dt)
    _need(gu, "gu", (shape.rows, 2 * shape.F), dt)
    rc = _abi.load().moe_expert_up_save_gu(ctypes.byref(shape.c()), _ptr(buf), _ptr(offsets),
                                           _ptr(w_gu), _ptr(h), _ptr(gu), _stream(stream))
    _abi.check("moe_expert_up_save_gu", rc)


def moe_expert_down(shape: MoeShape, h, offsets, w_down, y, stream=None) -> None:
    dt = shape.torch_dtype
    _need(h, "h", (shape.rows, shape.F), dt)
    _ffn_checks(shape, offsets)
    _need(w_down, "w_down", (shape.E_L, shape.d, shape.F), dt)
    _need(y, "y", (shape.rows, shape.d), dt)
    rc = _abi.load().moe_expert_down(ctypes.byref(shape.c()), _ptr(h), _ptr(offsets),
                                     _ptr(w_down), _ptr(y), _stream(stream))
    _abi.check("moe_expert_down", rc)


def moe_expert_ffn(shape: MoeShape, buf, offsets, w_gu, w_down, h, y, stream=None) -> None:
    dt = shape.torch_dtype
    _need(buf, "buf", (shape.rows, shape.d), dt)
    _ffn_checks(shape, offsets)
    _need(w_gu, "w_gu", (shape.E_L, 2 * shape.F, shape.d), dt)
    _need(w_down, "w_down", (shape.E_L, shape.d, shape.F), dt)
    _need(h, "h", (shape.rows, shape.F), dt)
    _need(y, "y", (shape.rows, shape.d), dt)
    rc = _abi.load().moe_expert_ffn(ctypes.byref(shape.c()), _ptr(buf), _ptr(offsets),
                                    _ptr(w_gu), _ptr(w_down), _ptr(h), _ptr(y), _stream(stream))
    _abi.check("moe_expert_ffn", rc)


def moe_combine(shape: MoeShape, y, dest_rank, dest_row, topk_w, out, stream=None) -> None:
    dt = shape.torch_dtype
    _need(y, "y", (shape.rows, shape.d), dt)
    _need(dest_rank, "dest_rank", (shape.T, shape.K), torch.int32)
    _need(dest_row, "dest_row", (shape.T, shape.K), torch.int32)
    _need(topk_w, "topk_w", (shape.T, shape.K), torch.float32)
    _need(out, "out", (shape.T, shape.d), dt)
    rc = _abi.load().moe_combine(ctypes.byref(shape.c()), _ptr(y), _ptr(dest_rank),
                                 _ptr(dest_row), _ptr(topk_w), _ptr(out), _stream(stream))
    _abi.check("moe_combine", rc)


# ----------------------------------------------------------------- backward
def moe_combine_bwd(shape: MoeShape, dout, y, dest_rank, dest_row, topk_w, dy, dw,
                    stream=None) -> None:
    dt = shape.torch_dtype
    _need(dout, "dout", (shape.T, shape.d), dt)
    _need(y, "y", (shape.rows, shape.d), dt)
    _need(dest_rank, "dest_rank", (shape.T, shape.K), torch.int32)
    _need(dest_row, "dest_row", (shape.T, shape.K), torch.int32)
    _need(topk_w, "topk_w", (shape.T, shape.K), torch.float32)
    _need(dy, "dy", (shape.rows, shape.d), dt)
    _need(dw, "dw", (shape.T, shape.K), torch.float32)
    rc = _abi.load().moe_combine_bwd(ctypes.byref(shape.c()), _ptr(dout), _ptr(y),
                                     _ptr(dest_rank), _ptr(dest_row), _ptr(topk_w), _ptr(dy),
                                     _ptr(dw), _stream(stream))
    _abi.check("moe_combine_bwd", rc)


def moe_expert_ffn_bwd(shape: MoeShape, buf, offsets, w_gu, w_down, h, dy, gu, dgu, dx_rows,
                       dw_gu, dw_down, stream=None) -> None:
    dt = shape.torch_dtype
    _need(buf, "buf", (shape.rows, shape.d), dt)
    _ffn_checks(shape, offsets)
    _need(w_gu, "w_gu", (shape.E_L, 2 * shape.F, shape.d), dt)
    _need(w_down, "w_down", (shape.E_L, shape.d, shape.F), dt)
    _need(h, "h", (shape.rows, shape.F), dt)
    _need(dy, "dy", (shape.rows, shape.d), dt)
    _need(gu, "gu", (shape.rows, 2 * shape.F), dt)
    _need(dgu, "dgu", (shape.rows, 2 * shape.F), dt)
    _need(dx_rows, "dx_rows", (shape.rows, shape.d), dt)
    _need(dw_gu, "dw_gu", (shape.E_L, 2 * shape.F, shape.d), torch.float32)
    _need(dw_down, "dw_down", (shape.E_L, shape.d, shape.F), torch.float32)
    rc = _abi.load().moe_expert_ffn_bwd(
        ctypes.byref(shape.c()), _ptr(buf), _ptr(offsets), _ptr(w_gu), _ptr(w_down), _ptr(h),
        _ptr(dy), _ptr(gu), _ptr(dgu), _ptr(dx_rows), _ptr(dw_gu), _ptr(dw_down),
        _stream(stream))
    _abi.check("moe_expert_ffn_bwd", rc)


def moe_expert_ffn_bwd_data(shape: MoeShape, buf, offsets, w_gu, w_down, dy, gu, dgu, dx_rows,
                            stream=None) -> None:
    dt = shape.torch_dtype
    _need(buf, "buf", (shape.rows, shape.d), dt)
    _ffn_checks(shape, offsets)
    _need(w_gu, "w_gu", (shape.E_L, 2 * shape.F, shape.d), dt)
    _need(w_down, "w_down", (shape.E_L, shape.d, shape.F), dt)
    _need(dy, "dy", (shape.rows, shape.d), dt)
    _need(gu, "gu", (shape.rows, 2 * shape.F), dt)
    _need(dgu, "dgu", (shape.rows, 2 * shape.F), dt)
    _need(dx_rows, "dx_rows", (shape.rows, shape.d), dt)
    rc = _abi.load().moe_expert_ffn_bwd_data(
        ctypes.byref(shape.c()), _ptr(buf), _ptr(offsets), _ptr(w_gu), _ptr(w_down), _ptr(dy),
        _ptr(gu), _ptr(dgu), _ptr(dx_rows), _stream(stream))
    _abi.check("moe_expert_ffn_bwd_data", rc)


def moe_expert_ffn_bwd_data_saved_gu(shape: MoeShape, offsets, w_gu, w_down, dy, gu, dgu,
                                     dx_rows, stream=None) -> None:
    dt = shape.torch_dtype
    _ffn_checks(shape, offsets)
    _need(w_gu, "w_gu", (shape.E_L, 2 * shape.F, shape.d), dt)
    _need(w_down, "w_down", (shape.E_L, shape.d, shape.F), dt)
    _need(dy, "dy", (shape.rows, shape.d), dt)
    _need(gu, "gu", (shape.rows, 2 * shape.F), dt)
    _need(dgu, "dgu", (shape.rows, 2 * shape.F), dt)
    _need(dx_rows, "dx_rows", (shape.rows, shape.d), dt)
    rc = _abi.load().moe_expert_ffn_bwd_data_saved_gu(
        ctypes.byref(shape.c()), _ptr(offsets), _ptr(w_gu), _ptr(w_down), _ptr(dy), _ptr(gu),
        _ptr(dgu), _ptr(dx_rows), _stream(stream))
    _abi.check("moe_expert_ffn_bwd_data_saved_gu", rc)


def moe_expert_ffn_bwd_weight(shape: MoeShape, buf, offsets, h, dy, dgu, dw_gu, dw_down,
                              stream=None) -> None:
    dt = shape.torch_dtype
    _need(buf, "buf", (shape.rows, shape.d), dt)
    _ffn_checks(shape, offsets)
    _need(h, "h", (shape.rows, shape.F), dt)
    _need(dy, "dy", (shape.rows, shape.d), dt)
    _need(dgu, "dgu", (shape.rows, 2 * shape.F), dt)
    _need(dw_gu, "dw_gu", (shape.E_L, 2 * shape.F, shape.d), torch.float32)
    _need(dw_down, "dw_down", (shape.E_L, shape.d, shape.F), torch.float32)
    rc = _abi.load().moe_expert_ffn_bwd_weight(
        ctypes.byref(shape.c()), _ptr(buf), _ptr(offsets), _ptr(h), _ptr(dy), _ptr(dgu),
        _ptr(dw_gu), _ptr(dw_down), _stream(stream))
    _abi.check("moe_expert_ffn_bwd_weight", rc)


def moe_dispatch_bwd(shape: MoeShape, dx_rows, dest_rank, dest_row, dx, stream=None) -> None:
    dt = shape.torch_dtype
    _need(dx_rows, "dx_rows", (shape.rows, shape.d), dt)
    _need(dest_rank, "dest_rank", (shape.T, shape.K), torch.int32)
    _need(dest_row, "dest_row", (shape.T, shape.K), torch.int32)
    _need(dx, "dx", (shape.T, shape.d), dt)
    rc = _abi.load().moe_dispatch_bwd(ctypes.byref(shape.c()), _ptr(dx_rows), _ptr(dest_rank),
                                      _ptr(dest_row), _ptr(dx), _stream(stream))
    _abi.check("moe_dispatch_bwd", rc)


def moe_route_bwd(shape: MoeShape, topk_idx, topk_w, dw, dlogits, stream=None) -> None:
    _need(topk_idx, "topk_idx", (shape.T, shape.K), torch.int32)
    _need(topk_w, "topk_w", (shape.T, shape.K), torch.float32)
    _need(dw, "dw", (shape.T, shape.K), torch.float32)
    _need(dlogits, "dlogits", (shape.T, shape.N), torch.float32)
    rc = _abi.load().moe_route_bwd(ctypes.byref(shape.c()), _ptr(topk_idx), _ptr(topk_w),
                                   _ptr(dw), _ptr(dlogits), _stream(stream))
    _abi.check("moe_route_bwd", rc)


# ----------------------------------------------------------------- MXFP8
def mx_scale_cols(cols: int) -> int:
    """Bytes per MX scale row of ``cols`` elements: cols / 32 block scales
    rounded up to a multiple of 4 (the rows start 4-byte aligned)."""
    return (cols // 32 + 3) // 4 * 4


def moe_mx_quantize_rows(src, qdata, scales, stream=None) -> None:
    """MX-quantize the rows of a bf16 tensor along its last dimension (a
    multiple of 32): qdata uint8 of src's shape, scales uint8
    [..., mx_scale_cols(cols)] (the first cols/32 bytes of a row are its
    scales)."""
    if not isinstance(src, torch.Tensor) or src.dtype != torch.bfloat16 or src.dim() < 1:
        raise ValueError("src must be a bf16 tensor")
    cols = src.shape[-1]
    rows = src.numel() // cols if cols else 0
    _need(src, "src", tuple(src.shape), torch.bfloat16)
    _need(qdata, "qdata", tuple(src.shape), torch.uint8)
    _need(scales, "scales", tuple(src.shape[:-1]) + (mx_scale_cols(cols),), torch.uint8)
    rc = _abi.load().moe_mx_quantize_rows(rows, cols, _ptr(src), _ptr(qdata), _ptr(scales),
                                          _stream(stream))
    _abi.check("moe_mx_quantize_rows", rc)


def moe_dispatch_rows_mx(shape: MoeShape, x, dest_rank, dest_row, qbuf, sbuf,
                         stream=None) -> None:
    _need(x, "x", (shape.T, shape.d), torch.bfloat16)
    _need(dest_rank, "dest_rank", (shape.T, shape.K), torch.int32)
    _need(dest_row, "dest_row", (shape.T, shape.K), torch.int32)
    _need(qbuf, "qbuf", (shape.rows, shape.d), torch.uint8)
    _need(sbuf, "sbuf", (shape.rows, mx_scale_cols(shape.d)), torch.uint8)
    rc = _abi.load().moe_dispatch_rows_mx(ctypes.byref(shape.c()), _ptr(x), _ptr(dest_rank),
                                          _ptr(dest_row), _ptr(qbuf), _ptr(sbuf), _stream(stream))
    _abi.check("moe_dispatch_rows_mx", rc)


def moe_expert_up_mx(shape: MoeShape, qbuf, sbuf, offsets, w_gu_q, w_gu_s, h_q, h_s,
                     stream=None) -> None:
    u8 = torch.uint8
    _need(qbuf, "qbuf", (shape.rows, shape.d), u8)
    _need(sbuf, "sbuf", (shape.rows, mx_scale_cols(shape.d)), u8)
    _ffn_checks(shape, offsets)
    _need(w_gu_q, "w_gu_q", (shape.E_L, 2 * shape.F, shape.d), u8)
    _need(w_gu_s, "w_gu_s", (shape.E_L, 2 * shape.F, mx_scale_cols(shape.d)), u8)
    _need(h_q, "h_q", (shape.rows, shape.F), u8)
    _need(h_s, "h_s", (shape.rows, mx_scale_cols(shape.F)), u8)
    rc = _abi.load().moe_expert_up_mx(ctypes.byref(shape.c()), _ptr(qbuf), _ptr(sbuf),
                                      _ptr(offsets), _ptr(w_gu_q), _ptr(w_gu_s), _ptr(h_q),
                                      _ptr(h_s), _stream(stream))
    _abi.check("moe_expert_up_mx", rc)


def moe_expert_down_mx(shape: MoeShape, h_q, h_s, offsets, w_d_q, w_d_s, y, stream=None) -> None:
    u8 = torch.uint8
    _need(h_q, "h_q", (shape.rows, shape.F), u8)
    _need(h_s, "h_s", (shape.rows, mx_scale_cols(shape.F)), u8)
    _ffn_checks(shape, offsets)
    _need(w_d_q, "w_d_q", (shape.E_L, shape.d, shape.F), u8)
    _need(w_d_s, "w_d_s", (shape.E_L, shape.d, mx_scale_cols(shape.F)), u8)
    _need(y, "y", (shape.rows, shape.d), torch.bfloat16)
    rc = _abi.load().moe_expert_down_mx(ctypes.byref(shape.c()), _ptr(h_q), _ptr(h_s),
                                        _ptr(offsets), _ptr(w_d_q), _ptr(w_d_s), _ptr(y),
                                        _stream(stream))
    _abi.check("moe_expert_down_mx", rc)


@dataclass
class MxWeights:
    """Expert weights quantized once along their contraction dimension."""
    w_gu_q: torch.Tensor   # [E_L, 2F, d] uint8
    w_gu_s: torch.Tensor   # [E_L, 2F, mx_scale_cols(d)] uint8
    w_d_q: torch.Tensor    # [E_L, d, F] uint8
    w_d_s: torch.Tensor    # [E_L, d, mx_scale_cols(F)] uint8

    @classmethod
    def from_bf16(cls, w_gu: torch.Tensor, w_d: torch.Tensor, stream=None) -> "MxWeights":
        u8 = torch.uint8
        E_L, F2, d = w_gu.shape
        F = F2 // 2
        q = cls(torch.empty(E_L, F2, d, dtype=u8, device=w_gu.device),
                torch.empty(E_L, F2, mx_scale_cols(d), dtype=u8, device=w_gu.device),
                torch.empty(E_L, d, F, dtype=u8, device=w_gu.device),
                torch.empty(E_L, d, mx_scale_cols(F), dtype=u8, device=w_gu.device))
        moe_mx_quantize_rows(w_gu, q.w_gu_q, q.w_gu_s, stream)
        moe_mx_quantize_rows(w_d, q.w_d_q, q.w_d_s, stream)
        return q


# ----------------------------------------------------------------- layer
class MoELayer:
    """Capacity-shaped buffers allocated once; ``forward`` enqueues the four
    calls back to back on the current stream with no host synchronization."""

    def __init__(self, shape: MoeShape, device="cuda", row_src: bool = True):
        _abi.load()
        self.shape = shape
        dt = shape.torch_dtype
        self.route = RouteOut.empty(shape, device, row_src=row_src)
        self.ws = torch.empty(moe_route_workspace_size(shape), dtype=torch.uint8, device=device)
        self.buf = torch.empty(shape.rows, shape.d, dtype=dt, device=device)
        self.h = torch.empty(shape.rows, shape.F, dtype=dt, device=device)
        self.y = torch.empty(shape.rows, shape.d, dtype=dt, device=device)
        self.out = torch.empty(shape.T, shape.d, dtype=dt, device=device)
        # which forward filled the buffers last: "bf16", "mx" or None
        self.last_forward = None

    def route_step(self, logits, stream=None):
        moe_route(self.shape, logits, self.route, self.ws, stream)

    def dispatch_step(self, x, stream=None):
        r = self.route
        moe_dispatch_rows(self.shape, x, r.dest_rank, r.dest_row, self.buf, stream)

    def up_step(self, w_gu, stream=None, save_gu: bool = False):
        if save_gu:
            if not hasattr(self, "gu"):
                self.alloc_backward(self.out.device)
            moe_expert_up_save_gu(self.shape, self.buf, self.route.offsets, w_gu, self.h,
                                  self.gu, stream)
        else:
            moe_expert_up(self.shape, self.buf, self.route.offsets, w_gu, self.h, stream)
        self.gu_saved = save_gu

    def down_step(self, w_d, stream=None):
        moe_expert_down(self.shape, self.h, self.route.offsets, w_d, self.y, stream)

    def combine_step(self, stream=None):
        r = self.route
        moe_combine(self.shape, self.y, r.dest_rank, r.dest_row, r.topk_w, self.out, stream)

    def forward(self, logits, x, w_gu, w_d, stream=None, save_gu: bool = False) -> torch.Tensor:
        """Route, dispatch, expert FFN, combine. ``save_gu`` (training): the up
        GEMM also keeps the pre-activation [G U] rows, so that ``backward``
        reads them instead of recomputing them."""
        self.route_step(logits, stream)
        self.dispatch_step(x, stream)
        self.up_step(w_gu, stream, save_gu)
        self.down_step(w_d, stream)
        self.combine_step(stream)
        self.last_forward = "bf16"
        return self.out

    def alloc_mx(self, device="cuda") -> None:
        """MXFP8 forward buffers, allocated once: quantized dispatch rows and
        the quantized H, each with its scale rows."""
        s = self.shape
        u8 = torch.uint8
        self.qbuf = torch.empty(s.rows, s.d, dtype=u8, device=device)
        self.sbuf = torch.empty(s.rows, mx_scale_cols(s.d), dtype=u8, device=device)
        self.h_q = torch.empty(s.rows, s.F, dtype=u8, device=device)
        self.h_s = torch.empty(s.rows, mx_scale_cols(s.F), dtype=u8, device=device)

    def dispatch_mx_step(self, x, stream=None):
        r = self.route
        moe_dispatch_rows_mx(self.shape, x, r.dest_rank, r.dest_row, self.qbuf, self.sbuf, stream)

    def up_mx_step(self, mxw: "MxWeights", stream=None):
        moe_expert_up_mx(self.shape, self.qbuf, self.sbuf, self.route.offsets, mxw.w_gu_q,
                         mxw.w_gu_s, self.h_q, self.h_s, stream)

    def down_mx_step(self, mxw: "MxWeights", stream=None):
        moe_expert_down_mx(self.shape, self.h_q, self.h_s, self.route.offsets, mxw.w_d_q,
                           mxw.w_d_s, self.y, stream)

    def forward_mx(self, logits, x, mxw: "MxWeights", stream=None) -> torch.Tensor:
        """MXFP8 forward (inference only: ``backward`` refuses to follow it):
        the same routing, quantize-on-dispatch, MXFP8 expert GEMMs on the
        quantized weights, BF16 combine."""
        if not hasattr(self, "qbuf"):
            self.alloc_mx(self.out.device)
        self.gu_saved = False
        self.route_step(logits, stream)
        self.dispatch_mx_step(x, stream)
        self.up_mx_step(mxw, stream)
        self.down_mx_step(mxw, stream)
        self.combine_step(stream)
        self.last_forward = "mx"
        return self.out

    def alloc_backward(self, device="cuda") -> None:
        """Backward buffers, allocated once: dY, [G U] (reused in place for
        [dG dU]), dX rows, dx, the weight and logit gradients."""
        s = self.shape
        dt = s.torch_dtype
        self.dy = torch.empty(s.rows, s.d, dtype=dt, device=device)
        self.gu = torch.empty(s.rows, 2 * s.F, dtype=dt, device=device)
        self.dx_rows = torch.empty(s.rows, s.d, dtype=dt, device=device)
        self.dx = torch.empty(s.T, s.d, dtype=dt, device=device)
        self.dw = torch.empty(s.T, s.K, dtype=torch.float32, device=device)
        self.dw_gu = torch.empty(s.E_L, 2 * s.F, s.d, dtype=torch.float32, device=device)
        self.dw_down = torch.empty(s.E_L, s.d, s.F, dtype=torch.float32, device=device)
        self.dlogits = torch.empty(s.T, s.N, dtype=torch.float32, device=device)

    def backward(self, dout, w_gu, w_d, stream=None):
        """Gradients of the last forward for the output gradient ``dout``:
        returns (dx, dlogits, dw_gu, dw_down), enqueued on the stream with no
        host synchronization. The last forward must be the BF16 ``forward``:
        the MXFP8 forward keeps no BF16 dispatch rows or H, so a backward after
        it (or before any forward) raises instead of differentiating stale
        buffers."""
        if self.last_forward != "bf16":
            raise RuntimeError(
                "MoELayer.backward needs the BF16 forward as the last forward "
                f"(last forward: {self.last_forward!r}; the MXFP8 forward is inference-only)")
        if not hasattr(self, "dy"):
            self.alloc_backward(self.out.device)
        s, r = self.shape, self.route
        moe_combine_bwd(s, dout, self.y, r.dest_rank, r.dest_row, r.topk_w, self.dy, self.dw,
                        stream)
        # row gradients first, so dispatch backward reads dX rows while cached;
        # [G U] from the forward when it kept them, else recomputed (dgu
        # overwrites gu in place either way)
        if getattr(self, "gu_saved", False):
            moe_expert_ffn_bwd_data_saved_gu(s, r.offsets, w_gu, w_d, self.dy, self.gu, self.gu,
                                             self.dx_rows, stream)
            self.gu_saved = False
        else:
            moe_expert_ffn_bwd_data(s, self.buf, r.offsets, w_gu, w_d, self.dy, self.gu,
                                    self.gu, self.dx_rows, stream)
        moe_dispatch_bwd(s, self.dx_rows, r.dest_rank, r.dest_row, self.dx, stream)
        moe_route_bwd(s, r.topk_idx, r.topk_w, self.dw, self.dlogits, stream)
        moe_expert_ffn_bwd_weight(s, self.buf, r.offsets, self.h, self.dy, self.gu, self.dw_gu,
                                  self.dw_down, stream)
        return self.dx, self.dlogits, self.dw_gu, self.dw_down
