"""CPU oracle for the fused row kernels -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never import, load or call anything here, and this package imports nothing
from them: the two sides share no code, only the seeded input generators of
``memory_bound_amd.synth`` (which hold none of the method's arithmetic).

The arithmetic lives in ``oracle.c`` (plain double-precision loops, built with
gcc, no fast-math, no FP contraction).  This module loads it through ctypes,
widens the exact stored values of the inputs to float64 and returns float64
results.  The unfused variants compose the same routines with the rounding of
each stored intermediate to the I/O type, mirroring the separate kernels of an
unfused chain.

Pages cited (titles abbreviated):
  [P1] "CUDA算子融合优化：提升GPU推理性能的核心机制"
  [P2] "4. 算子融合与Kernel合并…"
  [P3] "算子融合的收益量化：显存带宽瓶颈下的 Kernel 拼接实测"
  [P4] "融合计算范式对比：从分离 Kernel 到算子内融合的 GPU 应用优化实践"

Every function is pinned by ``tests/test_oracle_pins.py`` against closed
forms, textbook values, invariants, brute force and library routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# ORACLE_LIB names another build of oracle.c to load instead (the sanitizer test runs the pins
# against an AddressSanitizer / UndefinedBehaviorSanitizer build this way)
_LIB_OVERRIDE = os.environ.get("ORACLE_LIB")
_lib = None

GCC_CMD = [
    "gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
    "-ffp-contract=off", "-fno-fast-math",
    "-o", _LIB_PATH, _SRC, "-lm",
]


def build() -> str:
    """Compile oracle.c into liboracle.so with gcc; returns the library path."""
    subprocess.run(GCC_CMD, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.oracle_add_layernorm.argtypes = [dp, dp, dp, dp, dp, i64, i64, ctypes.c_double]
    lib.oracle_add_layernorm_ex.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, i64, i64, ctypes.c_double,
                                            ctypes.c_int]
    lib.oracle_bias_gelu_residual.argtypes = [dp, dp, dp, dp, i64, i64]
    lib.oracle_softmax_rows.argtypes = [dp, dp, i64, i64, ctypes.c_double]
    lib.oracle_cumsum_scale_rows.argtypes = [dp, dp, i64, i64, ctypes.c_double]
    lib.oracle_matmul.argtypes = [dp, dp, dp, i64, i64, i64]
    lib.oracle_swiglu.argtypes = [dp, dp, dp, dp, dp, dp, i64, i64, i64]
    lib.oracle_gemm_bias_act.argtypes = [dp, dp, dp, dp, i64, i64, i64, ctypes.c_int]
    lib.oracle_activation.argtypes = [dp, dp, i64, ctypes.c_int]
    lib.oracle_round.argtypes = [dp, dp, i64, ctypes.c_int]
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None
    for name in ("oracle_add_layernorm", "oracle_add_layernorm_ex", "oracle_bias_gelu_residual", "oracle_softmax_rows",
                 "oracle_cumsum_scale_rows",
                 "oracle_matmul", "oracle_swiglu", "oracle_gemm_bias_act", "oracle_activation",
                 "oracle_round"):
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def f64(t) -> np.ndarray:
    """Exact stored values of a tensor/array, widened to a C-contiguous float64 array."""
    if hasattr(t, "detach"):  # torch tensor: widen through float64 on the CPU (exact)
        import torch
        t = t.detach().to("cpu").to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(t, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def threads() -> int:
    """OpenMP threads the oracle's row loops use."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Sets the OpenMP threads of the oracle's row loops (for timing it on one core)."""
    _load().oracle_set_threads(int(n))


# ----------------------------------------------------------------------------------------------
# fused definitions (the exact results the fused kernels approximate)
# ----------------------------------------------------------------------------------------------

def add_layernorm(x, residual, gamma, beta, eps: float) -> np.ndarray:
    """y = LayerNorm(x + residual) * gamma + beta per row; [P3] §1, [P2] §4.2.

    residual=None gives the plain LayerNorm of x.  x is [rows, hidden].
    """
    x = f64(x)
    rows, hidden = x.shape
    r = f64(residual) if residual is not None else None
    g, b = f64(gamma), f64(beta)
    assert g.shape == (hidden,) and b.shape == (hidden,)
    if r is not None:
        assert r.shape == x.shape
    y = np.empty_like(x)
    _load().oracle_add_layernorm(_p(x), _p(r) if r is not None else None, _p(g), _p(b), _p(y),
                                 rows, hidden, float(eps))
    return y


def add_layernorm_ex(x, residual, gamma, beta, eps: float, relu: bool = False):
    """LayerNorm variants; [P1] §二.1 (LayerNorm + ReLU), [P2] §4.4 (multi-output fusion).

    Returns (y, sum, mean, var): y = LN(x + residual) * gamma + beta, clamped below at 0 when
    relu; sum = x + residual; mean and var (population, without eps) per row.
    """
    x = f64(x)
    rows, hidden = x.shape
    r = f64(residual) if residual is not None else None
    g, b = f64(gamma), f64(beta)
    assert g.shape == (hidden,) and b.shape == (hidden,)
    if r is not None:
        assert r.shape == x.shape
    y, sm = np.empty_like(x), np.empty_like(x)
    mean, var = np.empty(rows), np.empty(rows)
    _load().oracle_add_layernorm_ex(_p(x), _p(r) if r is not None else None, _p(g), _p(b), _p(y),
                                    _p(sm), _p(mean), _p(var), rows, hidden, float(eps), int(bool(relu)))
    return y, sm, mean, var


def bias_gelu_residual(x, bias, residual) -> np.ndarray:
    """y = GELU_erf(x + bias[col]) + residual; [P3] intro diagram and §1."""
    x, bias, r = f64(x), f64(bias), f64(residual)
    rows, hidden = x.shape
    assert bias.shape == (hidden,) and r.shape == x.shape
    y = np.empty_like(x)
    _load().oracle_bias_gelu_residual(_p(x), _p(bias), _p(r), _p(y), rows, hidden)
    return y


def softmax_rows(x, scale: float) -> np.ndarray:
    """y = softmax(scale * x) per row; [P1] §二.1 (Softmax + Scale), [P2] §4.3."""
    x = f64(x)
    rows, cols = x.shape
    y = np.empty_like(x)
    _load().oracle_softmax_rows(_p(x), _p(y), rows, cols, float(scale))
    return y


def cumsum_scale_rows(x, scale: float) -> np.ndarray:
    """y = scale * inclusive prefix sum along each row; [P2] §4.4 (Cumsum + Scale)."""
    x = f64(x)
    rows, cols = x.shape
    y = np.empty_like(x)
    _load().oracle_cumsum_scale_rows(_p(x), _p(y), rows, cols, float(scale))
    return y


def matmul(a, b) -> np.ndarray:
    """Plain row-major product a[M,K] . b[K,N] with ascending-k sums."""
    a, b = f64(a), f64(b)
    M, K = a.shape
    K2, N = b.shape
    assert K == K2
    c = np.empty((M, N), dtype=np.float64)
    _load().oracle_matmul(_p(a), _p(b), _p(c), M, N, K)
    return c


def swiglu(a, b1, b2) -> np.ndarray:
    """out = SiLU(a . b1) * (a . b2); [P4] 对比对象定义."""
    a, b1, b2 = f64(a), f64(b1), f64(b2)
    M, K = a.shape
    assert b1.shape == b2.shape and b1.shape[0] == K
    N = b1.shape[1]
    out = np.empty((M, N), dtype=np.float64)
    c1 = np.empty_like(out)
    c2 = np.empty_like(out)
    _load().oracle_swiglu(_p(a), _p(b1), _p(b2), _p(out), _p(c1), _p(c2), M, N, K)
    return out


ACT = {"none": 0, "relu": 1, "gelu": 2, "silu": 3}


def gemm_bias_act(x, w, bias, act: str) -> np.ndarray:
    """y = act(x . W + bias[col]); [P1] §二.1 (GEMM + BiasAdd + Activation)."""
    x, w = f64(x), f64(w)
    M, K = x.shape
    assert w.shape[0] == K
    N = w.shape[1]
    b = f64(bias) if bias is not None else None
    if b is not None:
        assert b.shape == (N,)
    y = np.empty((M, N), dtype=np.float64)
    _load().oracle_gemm_bias_act(_p(x), _p(w), _p(b) if b is not None else None, _p(y), M, N, K, ACT[act])
    return y


def gemm_bias_act_unfused(x, w, bias, act: str, kind: str) -> np.ndarray:
    """[P1] §二.1's unfused pipeline: the GEMM kernel stores C, the bias kernel stores C + b, the
    activation kernel reads that; each stored intermediate rounded to the I/O type."""
    c = round_to(gemm_bias_act(x, w, None, "none"), kind)
    t = round_to(c + (f64(bias)[None, :] if bias is not None else 0.0), kind)
    return activation(t, act)


def activation(t, act: str) -> np.ndarray:
    """The activation alone, element-wise (none, ReLU, GELU erf form, SiLU)."""
    t = f64(t)
    y = np.empty_like(t)
    _load().oracle_activation(_p(t), _p(y), t.size, ACT[act])
    return y


_KIND = {"f32": 0, "fp32": 0, "f16": 1, "fp16": 1, "bf16": 2}


def round_to(v, kind: str) -> np.ndarray:
    """Round-to-nearest-even of float64 values onto the f16 / bf16 grid ('f32' keeps them)."""
    v = f64(v)
    out = np.empty_like(v)
    if kind in ("f32", "fp32"):
        # single precision: numpy's float32 cast is the IEEE RNE conversion
        return v.astype(np.float32).astype(np.float64)
    _load().oracle_round(_p(v), _p(out), v.size, _KIND[kind])
    return out


# ----------------------------------------------------------------------------------------------
# unfused chains: each intermediate a separate kernel would store is rounded to the I/O type
# ([P3] §1 accounts intermediates at the I/O width; [P4] 对比对象定义, scheme A)
# ----------------------------------------------------------------------------------------------

def add_layernorm_unfused(x, residual, gamma, beta, eps: float, kind: str) -> np.ndarray:
    """Add kernel stores A = x + r in the I/O type, then LayerNorm kernel reads A."""
    a = round_to(f64(x) + f64(residual), kind)
    return add_layernorm(a, None, gamma, beta, eps)


def bias_gelu_residual_unfused(x, bias, residual, kind: str) -> np.ndarray:
    """BiasAdd stores t, GELU stores g, Residual adds r: three stored tensors."""
    t = round_to(f64(x) + f64(bias)[None, :], kind)
    zeros_bias = np.zeros(t.shape[1])
    zeros_res = np.zeros_like(t)
    g = round_to(bias_gelu_residual(t, zeros_bias, zeros_res), kind)
    return g + f64(residual)


def softmax_rows_unfused(x, scale: float, kind: str) -> np.ndarray:
    """Row max kernel; exp kernel stores E = exp(z - m) in the I/O type and the row sum of the
    unrounded terms; divide kernel reads E.  y = E / s.  [P2] §4.3 lists the three steps."""
    x = f64(x)
    z = scale * x
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=1, keepdims=True)
    return round_to(e, kind) / s


def cumsum_scale_rows_unfused(x, scale: float, kind: str) -> np.ndarray:
    """Scan kernel stores the prefix sums S in the I/O type; scale kernel reads S: y = scale * S."""
    return float(scale) * round_to(cumsum_scale_rows(x, 1.0), kind)


def swiglu_unfused(a, b1, b2, kind: str) -> np.ndarray:
    """Scheme A of [P4]: a GEMM kernel stores c1 and c2 in the I/O type, then an element-wise
    kernel computes SiLU(c1) * c2."""
    c1 = round_to(matmul(a, b1), kind)
    c2 = round_to(matmul(a, b2), kind)
    return c1 / (1.0 + np.exp(-c1)) * c2
