"""Seeded synthetic workloads for the routed-expert MoE forward layer.

This module only draws random inputs and states shapes. It holds none of the
layer's arithmetic (no top-K, no softmax, no admission, no expert math), so both
the HIP path and the CPU oracle can consume exactly the same tensors without
sharing any of the method's code.

Recipe (one per named workload):
  * seed = the workload's number; one ``torch.Generator`` on the target device,
    drawn in the fixed order: router input (x then W_r for the tiny layer, raw
    logits otherwise), x, W_gu, W_d.
  * x ~ N(0, 1), rounded to the layer dtype (round-to-nearest-even).
  * expert weights ~ N(0, 0.02^2) in the K-contiguous ``[out, in]`` layout:
    W_gu[j] is [2F, d] (rows 0..F-1 gate, F..2F-1 up), W_d[j] is [d, F].
  * logits are fp32. The tiny layer computes them as x . W_r^T in float64 and
    rounds once to fp32 (the router GEMM sits upstream of the layer boundary,
    so it is part of input synthesis). The larger layers use i.i.d. N(0, 1)
    logits; the skewed layer adds a per-expert Zipf(s) bias (e + 1)^(-s).
  * capacity C = ceil(T * K * cf / N) in exact rational arithmetic; a dropless
    workload takes C = max(T, 1) instead (no expert can receive more than T
    routes, so none is dropped), with buffers of the upper-bound row count.

The shapes follow the pages' workloads: an OLMoE-like layer (64 experts, top-8),
a GPT-OSS-20B-like layer seen from one shard of an 8-way expert split (32
experts, top-4, 4 local), and larger fine-grained layers (Olmo-core MoE report,
Sec. 05 Expert Parallelism; AWS Neuron vLLM Expert Parallelism design,
GPT-OSS-20B case study). No dataset or trained weight is involved.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from fractions import Fraction

import torch


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int          # tokens
    d: int          # hidden size
    N: int          # experts (global)
    K: int          # top-K
    F: int          # expert SwiGLU width
    cf: Fraction    # capacity factor
    dtype: str      # "f32" or "bf16"
    ep_size: int = 1
    ep_rank: int = 0
    logits: str = "gauss"   # "router" | "gauss" | "zipf"
    zipf_s: float = 1.1
    seed: int = 0
    dropless: bool = False  # capacity = T: every route kept (cf unused)

    @property
    def capacity(self) -> int:
        if self.dropless:
            return max(self.T, 1)
        return math.ceil(Fraction(self.T * self.K, self.N) * self.cf)

    @property
    def E_L(self) -> int:
        return self.N // self.ep_size

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


CONFIGS = {
    "tiny_f32": LayerConfig("tiny_f32", T=256, d=128, N=8, K=2, F=256,
                            cf=Fraction(5, 4), dtype="f32", logits="router", seed=1),
    "olmoe_bf16": LayerConfig("olmoe_bf16", T=8192, d=2048, N=64, K=8, F=1024,
                              cf=Fraction(5, 4), dtype="bf16", seed=2),
    "gptoss_shard_bf16": LayerConfig("gptoss_shard_bf16", T=16384, d=2880, N=32, K=4,
                                     F=3072, cf=Fraction(1), dtype="bf16",
                                     ep_size=8, ep_rank=0, seed=3),
    "zipf_skew_bf16": LayerConfig("zipf_skew_bf16", T=32768, d=4096, N=128, K=8, F=1536,
                                  cf=Fraction(5, 4), dtype="bf16", logits="zipf", seed=4),
    "finegrained_shard_bf16": LayerConfig("finegrained_shard_bf16", T=65536, d=4096, N=256,
                                          K=8, F=2048, cf=Fraction(3, 2), dtype="bf16",
                                          ep_size=8, ep_rank=0, seed=5),
    # the skewed layer's inputs, routed dropless into upper-bound buffers
    "zipf_dropless_bf16": LayerConfig("zipf_dropless_bf16", T=32768, d=4096, N=128, K=8,
                                      F=1536, cf=Fraction(1), dtype="bf16", logits="zipf",
                                      seed=4, dropless=True),
}


@dataclass
class LayerInputs:
    cfg: LayerConfig
    logits: torch.Tensor   # [T, N] fp32
    x: torch.Tensor        # [T, d] dtype
    w_gu: torch.Tensor     # [E_L, 2F, d] dtype
    w_d: torch.Tensor      # [E_L, d, F] dtype


def make_inputs(cfg: LayerConfig, device="cpu", with_weights: bool = True) -> LayerInputs:
    """Draw the seeded inputs of ``cfg`` on ``device`` (see module docstring)."""
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed)
    dt = cfg.torch_dtype
    if cfg.logits == "router":
        x32 = torch.randn(cfg.T, cfg.d, generator=g, device=device, dtype=torch.float32)
        w_r = torch.randn(cfg.N, cfg.d, generator=g, device=device, dtype=torch.float32) * 0.02
        x = x32.to(dt)
        logits = (x.double() @ w_r.double().T).float()
    else:
        logits = torch.randn(cfg.T, cfg.N, generator=g, device=device, dtype=torch.float32)
        if cfg.logits == "zipf":
            bias = (torch.arange(cfg.N, device=device, dtype=torch.float64) + 1.0) ** (-cfg.zipf_s)
            logits = (logits.double() + bias[None, :]).float()
        x = torch.randn(cfg.T, cfg.d, generator=g, device=device, dtype=torch.float32).to(dt)
    if with_weights:
        E_L = cfg.E_L
        w_gu = (torch.randn(E_L, 2 * cfg.F, cfg.d, generator=g, device=device,
                            dtype=torch.float32) * 0.02).to(dt)
        w_d = (torch.randn(E_L, cfg.d, cfg.F, generator=g, device=device,
                           dtype=torch.float32) * 0.02).to(dt)
    else:
        w_gu = w_d = None
    return LayerInputs(cfg, logits.contiguous(), x.contiguous(), w_gu, w_d)


def random_rows(rows: int, cols: int, dtype: torch.dtype, seed: int, device="cpu") -> torch.Tensor:
    """N(0,1) matrix in ``dtype`` (used as a stand-in expert output for combine)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32).to(dtype)


def random_ids(T: int, N: int, K: int, seed: int, invalid_frac: float = 0.0) -> torch.Tensor:
    """[T, K] int32 distinct expert ids per token; a fraction replaced by -1 (invalid)."""
    g = torch.Generator()
    g.manual_seed(seed)
    ids = torch.argsort(torch.rand(T, N, generator=g), dim=1)[:, :K].to(torch.int32)
    if invalid_frac > 0:
        mask = torch.rand(T, K, generator=g) < invalid_frac
        ids[mask] = -1
    return ids.contiguous()
