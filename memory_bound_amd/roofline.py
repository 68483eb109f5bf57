"""Algorithmic work per launch and the MI355X peaks the kernels are measured against.

Algorithmic bytes are the bytes the operation must move between HBM and the chip at minimum:
every input element read once, every output element written once, per-column parameters read
once per launch.  The unfused chains add the intermediates each separate kernel stores and the
next one reloads, at the I/O width (page "算子融合的收益量化", §1 counts them that way: 16 MB per
[1,2048,4096] fp16 tensor, 80 MB unfused versus 48 MB fused for ResidualAdd+LayerNorm).
"""
from __future__ import annotations

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}

# Published MI355X figures (AMD): HBM3E bandwidth and dense matrix-core peaks.
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0, "f32": 157.3, "f64": 78.6}


def _t(kind: str, tensor: int, params: int = 0, scalars: int = 0) -> dict:
    return {"kind": kind, "tensor_bytes": tensor, "param_bytes": params,
            "scalar_bytes": scalars, "bytes": tensor + params + scalars}


def add_layernorm_bytes(rows: int, hidden: int, dtype: str, fused: bool = True) -> dict:
    """Fused: read x and r, write y, read gamma and beta.  Unfused: the add kernel reads x, r and
    writes A; the LayerNorm kernel reads A and writes y (5 tensor passes instead of 3)."""
    e = ELEM_BYTES[dtype]
    t = rows * hidden * e
    passes = 3 if fused else 5
    return _t("fused" if fused else "unfused", passes * t, 2 * hidden * e)


def add_layernorm_ex_bytes(rows: int, hidden: int, dtype: str, fused: bool = True) -> dict:
    """The LayerNorm variants with every extra output: the fused Add+LN traffic plus the stored
    pre-norm sum (one more tensor pass) and the fp32 mean and variance (8 bytes per row).  The
    ReLU adds no traffic."""
    d = add_layernorm_bytes(rows, hidden, dtype, fused)
    e = ELEM_BYTES[dtype]
    return _t("fused", d["tensor_bytes"] + rows * hidden * e, d["param_bytes"], 8 * rows)


def bias_gelu_residual_bytes(rows: int, hidden: int, dtype: str, fused: bool = True) -> dict:
    """Fused: read x and r, write y, read bias.  Unfused: bias kernel (read x, write t), GELU
    kernel (read t, write g), residual kernel (read g and r, write y): 7 tensor passes."""
    e = ELEM_BYTES[dtype]
    t = rows * hidden * e
    passes = 3 if fused else 7
    return _t("fused" if fused else "unfused", passes * t, hidden * e)


def softmax_rows_bytes(rows: int, cols: int, dtype: str, fused: bool = True) -> dict:
    """Fused: read x, write y.  Unfused: row-max kernel (read x, write m), exp kernel (read x and
    m, write E and the row sums s), divide kernel (read E and s, write y); m and s are fp32."""
    e = ELEM_BYTES[dtype]
    t = rows * cols * e
    if fused:
        return _t("fused", 2 * t)
    return _t("unfused", 5 * t, 0, 4 * rows * 4)


def cumsum_scale_rows_bytes(rows: int, cols: int, dtype: str, fused: bool = True) -> dict:
    """Fused: read x, write y.  Unfused: the scan kernel reads x and writes S, the scale kernel
    reads S and writes y (4 tensor passes)."""
    t = rows * cols * ELEM_BYTES[dtype]
    return _t("fused" if fused else "unfused", (2 if fused else 4) * t)


def swiglu_bytes(M: int, N: int, K: int, dtype: str, fused: bool = True) -> dict:
    """Minimum traffic: read a, b1, b2 once, write out once.  Unfused adds c1 and c2 written by the
    GEMM kernel and read back by the element-wise kernel."""
    e = ELEM_BYTES[dtype]
    base = (M * K + 2 * K * N + M * N) * e
    if fused:
        return _t("fused", base)
    return _t("unfused", base + 4 * M * N * e)


def gemm_bias_act_bytes(M: int, N: int, K: int, dtype: str, fused: bool = True) -> dict:
    """Minimum traffic: read x, w and bias once, write y once.  Unfused ([P1] §二.1's three
    kernels): C written and re-read, C + bias written and re-read."""
    e = ELEM_BYTES[dtype]
    base = (M * K + K * N + N + M * N) * e
    return _t("fused", base) if fused else _t("unfused", base + 4 * M * N * e)


def gemm_flops(M: int, N: int, K: int) -> int:
    """One M x N x K product at 2 flops per multiply-add (bias and activation not counted)."""
    return 2 * M * N * K


def swiglu_flops(M: int, N: int, K: int) -> int:
    """Two M x N x K products at 2 flops per multiply-add (the activation is not counted)."""
    return 4 * M * N * K


def workload_work(op: str, shape: tuple, dtype: str, fused: bool = True) -> dict:
    if op == "add_layernorm":
        return add_layernorm_bytes(*shape, dtype, fused)
    if op == "add_layernorm_ex":
        return add_layernorm_ex_bytes(*shape, dtype, fused)
    if op == "bias_gelu_residual":
        return bias_gelu_residual_bytes(*shape, dtype, fused)
    if op == "softmax_rows":
        return softmax_rows_bytes(*shape, dtype, fused)
    if op == "cumsum_scale_rows":
        return cumsum_scale_rows_bytes(*shape, dtype, fused)
    if op == "gemm_bias_act":
        d = gemm_bias_act_bytes(*shape, dtype, fused)
        d["flops"] = gemm_flops(*shape)
        return d
    if op == "swiglu":
        d = swiglu_bytes(*shape, dtype, fused)
        d["flops"] = swiglu_flops(*shape)
        return d
    raise ValueError(op)
