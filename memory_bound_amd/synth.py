"""Seeded synthetic inputs for the fused row kernels.

This module holds none of the method's arithmetic: it only draws random tensors with the
shapes and value distributions of the workloads below, on the CPU, from a seeded
``torch.Generator``, in a fixed order, and casts them to the storage type with IEEE
round-to-nearest-even (torch's ``.to(dtype)``).  The same CPU tensors feed the device (after
``.to('cuda')``) and the CPU oracle, so both see bit-identical inputs.

Distribution parameters ("N(mu, s)" means mean mu and standard deviation s):

* Add+LayerNorm: x, r ~ N(0, 1) of shape [rows, hidden]; gamma ~ U(0.5, 1.5); beta ~ N(0, 0.1);
  eps = 1e-5.
* BiasAdd+GELU+Residual: x ~ N(0, 1); bias[hidden] ~ N(0, 0.02); residual ~ N(0, 1).
* Row softmax of attention scores: x = N(0, 1) * sqrt(d) with d = 128 head size, stored in the
  I/O type; the kernel applies scale = 1/sqrt(d).
* SwiGLU: a[M, K] ~ N(0, 1); b1, b2 [K, N] ~ N(0, 1/sqrt(K)).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _randn(g, *shape):
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def _rand(g, *shape):
    return torch.rand(*shape, generator=g, dtype=torch.float32)


def add_layernorm_inputs(rows: int, hidden: int, dtype: str, seed: int) -> dict:
    """x, residual, gamma, beta (CPU tensors in ``dtype``) and eps."""
    g = _gen(seed)
    t = DTYPES[dtype]
    x = _randn(g, rows, hidden).to(t)
    r = _randn(g, rows, hidden).to(t)
    gamma = (0.5 + _rand(g, hidden)).to(t)
    beta = (0.1 * _randn(g, hidden)).to(t)
    return {"x": x, "residual": r, "gamma": gamma, "beta": beta, "eps": 1e-5}


def bias_gelu_residual_inputs(rows: int, hidden: int, dtype: str, seed: int) -> dict:
    g = _gen(seed)
    t = DTYPES[dtype]
    x = _randn(g, rows, hidden).to(t)
    bias = (0.02 * _randn(g, hidden)).to(t)
    r = _randn(g, rows, hidden).to(t)
    return {"x": x, "bias": bias, "residual": r}


def softmax_inputs(rows: int, cols: int, dtype: str, seed: int, head_dim: int = 128) -> dict:
    g = _gen(seed)
    t = DTYPES[dtype]
    x = (_randn(g, rows, cols) * math.sqrt(head_dim)).to(t)
    return {"x": x, "scale": 1.0 / math.sqrt(head_dim)}


def cumsum_inputs(rows: int, cols: int, dtype: str, seed: int) -> dict:
    """x ~ N(0,1); the scale 1/sqrt(cols) keeps the scaled running sums of order one."""
    g = _gen(seed)
    x = _randn(g, rows, cols).to(DTYPES[dtype])
    return {"x": x, "scale": 1.0 / math.sqrt(cols)}


def gemm_inputs(M: int, N: int, K: int, dtype: str, seed: int) -> dict:
    """x ~ N(0,1); w ~ N(0, 1/sqrt(K)) (standard deviation); bias ~ N(0, 0.02)."""
    g = _gen(seed)
    t = DTYPES[dtype]
    x = _randn(g, M, K).to(t)
    w = (_randn(g, K, N) / math.sqrt(K)).to(t)
    bias = (_randn(g, N) * 0.02).to(t)
    return {"x": x, "w": w, "bias": bias}


def swiglu_inputs(M: int, N: int, K: int, dtype: str, seed: int) -> dict:
    g = _gen(seed)
    t = DTYPES[dtype]
    s = 1.0 / math.sqrt(K)
    a = _randn(g, M, K).to(t)
    b1 = (_randn(g, K, N) * s).to(t)
    b2 = (_randn(g, K, N) * s).to(t)
    return {"a": a, "b1": b1, "b2": b2}


@dataclass(frozen=True)
class Workload:
    """One named workload: the operation, its shape, I/O type and seed."""
    name: str
    op: str
    shape: tuple
    dtype: str
    seed: int
    note: str = ""
    extra: dict = field(default_factory=dict)

    def inputs(self) -> dict:
        if self.op == "add_layernorm":
            return add_layernorm_inputs(*self.shape, self.dtype, self.seed)
        if self.op == "bias_gelu_residual":
            return bias_gelu_residual_inputs(*self.shape, self.dtype, self.seed)
        if self.op == "softmax_rows":
            return softmax_inputs(*self.shape, self.dtype, self.seed)
        if self.op == "swiglu":
            return swiglu_inputs(*self.shape, self.dtype, self.seed)
        if self.op == "cumsum_scale_rows":
            return cumsum_inputs(*self.shape, self.dtype, self.seed)
        if self.op == "gemm_bias_act":
            return gemm_inputs(*self.shape, self.dtype, self.seed)
        raise ValueError(self.op)


# The workloads of the hot path (B*S flattened into rows).
WORKLOADS = {
    w.name: w
    for w in [
        Workload("addln_f32_64x768", "add_layernorm", (64, 768), "f32", 1001,
                 "ResidualAdd+LayerNorm fp32, 64 rows x H=768"),
        Workload("gelu_f16_2048x4096", "bias_gelu_residual", (2048, 4096), "f16", 1002,
                 "BiasAdd+GELU(erf)+Residual fp16, [B,S,H]=[1,2048,4096]"),
        Workload("addln_f16_2048x4096", "add_layernorm", (2048, 4096), "f16", 1003,
                 "ResidualAdd+LayerNorm fp16, [B,S,H]=[1,2048,4096]"),
        Workload("addln_f16_16384x4096", "add_layernorm", (16384, 4096), "f16", 1004,
                 "ResidualAdd+LayerNorm fp16, [B,S,H]=[8,2048,4096]"),
        Workload("softmax_f16_65536x2048", "softmax_rows", (65536, 2048), "f16", 1005,
                 "row softmax fp16, 32 heads x 2048 x 2048 scores"),
        Workload("swiglu_bf16_2048x8960x1536", "swiglu", (2048, 8960, 1536), "bf16", 1006,
                 "SwiGLU dual GEMM bf16, M=2048 N=8960 K=1536"),
        Workload("cumsum_f16_2048x4096", "cumsum_scale_rows", (2048, 4096), "f16", 1007,
                 "row cumsum + scale fp16, [B,S,H]=[1,2048,4096], scale 1/64"),
        Workload("gemm_relu_bf16_2048x8960x1536", "gemm_bias_act", (2048, 8960, 1536), "bf16", 1008,
                 "GEMM + bias + ReLU bf16, x [2048,1536], W [1536,8960] (the SwiGLU layer's shapes)"),
    ]
}
