"""Python binding of the libfuse C ABI (include/libfuse.h): argument marshalling only.

Every function has the name of the C entry point it calls and takes torch tensors that already
live on the GPU; it passes their data pointers, sizes and the current torch stream, and raises
``FuseError`` on a non-OK status.  All computation happens in the HIP kernels of libfuse.so; if
the library is not built this module raises instead of computing anything another way.

torch is imported before libfuse.so is loaded so that both share torch's HIP runtime.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfuse.so")

FUSE_F32, FUSE_F16, FUSE_BF16 = 0, 1, 2
_DTYPE_CODE = {torch.float32: FUSE_F32, torch.float16: FUSE_F16, torch.bfloat16: FUSE_BF16}

FUSE_LN_RELU = 1

FUSE_OP_ADD_LAYERNORM, FUSE_OP_BIAS_GELU_RESIDUAL, FUSE_OP_SOFTMAX_ROWS, FUSE_OP_SWIGLU = 0, 1, 2, 3
FUSE_OP_CUMSUM_SCALE, FUSE_OP_GEMM_BIAS_ACT = 4, 5
FUSE_ACT = {"none": 0, "relu": 1, "gelu": 2, "silu": 3}

STATUS = {0: "FUSE_OK", 1: "FUSE_ERR_NULL_PTR", 2: "FUSE_ERR_BAD_SHAPE", 3: "FUSE_ERR_BAD_DTYPE",
          4: "FUSE_ERR_BAD_VALUE", 5: "FUSE_ERR_ALIAS", 6: "FUSE_ERR_UNSUPPORTED",
          7: "FUSE_ERR_WORKSPACE", 8: "FUSE_ERR_MISALIGNED", 9: "FUSE_ERR_HIP"}

# Every symbol include/libfuse.h declares.
EXPORTS = [
    "fuse_add_layernorm", "fuse_add_layernorm_ex", "fuse_bias_gelu_residual", "fuse_softmax_rows",
    "fuse_cumsum_scale_rows", "fuse_swiglu_dualgemm", "fuse_gemm_bias_act", "fuse_unfused_gemm_bias_act",
    "fuse_auto_splits", "fuse_auto_workspace_bytes", "fuse_swiglu_auto", "fuse_gemm_bias_act_auto",
    "fuse_swiglu_auto_noalloc",
    "fuse_unfused_workspace_bytes", "fuse_unfused_add_layernorm", "fuse_unfused_bias_gelu_residual",
    "fuse_unfused_softmax_rows", "fuse_unfused_cumsum_scale_rows", "fuse_unfused_swiglu", "fuse_copy", "fuse_empty_kernels",
    "fuse_mfma_ceiling",
    "fuse_status_string", "fuse_last_hip_error", "fuse_version",
]


class FuseError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        lib = _lib
        msg = lib.fuse_status_string(status).decode() if lib else STATUS.get(status, str(status))
        if status == 9 and lib:
            msg += f" (hipError_t {lib.fuse_last_hip_error()})"
        super().__init__(f"{what}: {msg}")


_lib = None


def load() -> ctypes.CDLL:
    """Load libfuse.so (built by memory_bound_amd.build); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m memory_bound_amd.build` "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, f32, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    sig = {
        "fuse_add_layernorm": [vp, vp, vp, vp, vp, i64, i64, f32, i32, vp],
        "fuse_add_layernorm_ex": [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, f32, ctypes.c_uint, i32, vp],
        "fuse_bias_gelu_residual": [vp, vp, vp, vp, i64, i64, i32, vp],
        "fuse_softmax_rows": [vp, vp, i64, i64, f32, i32, vp],
        "fuse_cumsum_scale_rows": [vp, vp, i64, i64, f32, i32, vp],
        "fuse_unfused_cumsum_scale_rows": [vp, vp, i64, i64, f32, i32, vp, sz, vp],
        "fuse_swiglu_dualgemm": [vp, vp, vp, vp, i64, i64, i64, i32, vp],
        "fuse_gemm_bias_act": [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp],
        "fuse_swiglu_auto": [vp, vp, vp, vp, i64, i64, i64, i32, vp, sz, vp],
        "fuse_swiglu_auto_noalloc": [vp, vp, vp, vp, i64, i64, i64, i32, vp],
        "fuse_gemm_bias_act_auto": [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, sz, vp],
        "fuse_auto_splits": [i32, i64, i64, i64],
        "fuse_unfused_gemm_bias_act": [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, sz, vp],
        "fuse_unfused_add_layernorm": [vp, vp, vp, vp, vp, i64, i64, f32, i32, vp, sz, vp],
        "fuse_unfused_bias_gelu_residual": [vp, vp, vp, vp, i64, i64, i32, vp, sz, vp],
        "fuse_unfused_softmax_rows": [vp, vp, i64, i64, f32, i32, vp, sz, vp],
        "fuse_unfused_swiglu": [vp, vp, vp, vp, i64, i64, i64, i32, vp, sz, vp],
        "fuse_copy": [vp, vp, sz, vp],
        "fuse_empty_kernels": [i64, vp],
        "fuse_mfma_ceiling": [i64, i64, vp, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.fuse_unfused_workspace_bytes.argtypes = [i32, i64, i64, i64, i32]
    lib.fuse_unfused_workspace_bytes.restype = sz
    lib.fuse_auto_workspace_bytes.argtypes = [i32, i64, i64, i64, i32]
    lib.fuse_auto_workspace_bytes.restype = sz
    lib.fuse_status_string.argtypes = [i32]
    lib.fuse_status_string.restype = ctypes.c_char_p
    lib.fuse_last_hip_error.argtypes = []
    lib.fuse_last_hip_error.restype = ctypes.c_int
    lib.fuse_version.argtypes = []
    lib.fuse_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ------------------------------------------------------------------------------------------------
# marshalling helpers
# ------------------------------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dt(t) -> int:
    if t.dtype not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DTYPE_CODE[t.dtype]


def _check(t, name, dtype=None, shape=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}; the kernels run on cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _rows_cols(x):
    h = x.shape[-1] if x.dim() else 1
    return (x.numel() // h if h else 0), h


def _ok(status: int, what: str):
    if status != 0:
        raise FuseError(status, what)


def _torch_stream(stream):
    """The torch stream object for a stream argument (None = the current stream)."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream))


def _scratch(n, device, stream):
    """n bytes of device memory whose base is rounded up to a 256-byte boundary.  The kernels
    that use it are enqueued on `stream`, which may not be torch's current stream: the block is
    marked as used there, so the caching allocator does not hand it out again (after this
    wrapper drops it) before the work already enqueued on that stream has finished."""
    buf = torch.empty(n + 256, dtype=torch.uint8, device=device)
    buf.record_stream(_torch_stream(stream))
    off = (-buf.data_ptr()) % 256
    return buf, ctypes.c_void_p(buf.data_ptr() + off), n


def _workspace(op, d0, d1, d2, dtype_code, device, stream=None):
    return _scratch(load().fuse_unfused_workspace_bytes(op, d0, d1, d2, dtype_code), device, stream)


def _caller_workspace(workspace):
    """The `workspace` argument of the entry points that take one: None (allocate one for this
    call), a contiguous GPU tensor whose bytes are the workspace (at least what the matching
    fuse_*_workspace_bytes call returns, 256-byte aligned; the library checks both), or what
    _workspace / _auto_workspace return."""
    if workspace is None or isinstance(workspace, tuple):
        return workspace
    _check(workspace, "workspace")
    return workspace, ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


# ------------------------------------------------------------------------------------------------
# fused entry points
# ------------------------------------------------------------------------------------------------

def fuse_add_layernorm(x, residual, gamma, beta, eps=1e-5, y=None, stream=None):
    """y = LayerNorm(x + residual) * gamma + beta over the last dim (residual may be None)."""
    rows, hidden = _rows_cols(x)
    _check(x, "x")
    _check(residual, "residual", x.dtype, x.shape)
    _check(gamma, "gamma", x.dtype, (hidden,))
    _check(beta, "beta", x.dtype, (hidden,))
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.dtype, x.shape)
    _ok(load().fuse_add_layernorm(_ptr(x), _ptr(residual), _ptr(gamma), _ptr(beta), _ptr(y), rows, hidden,
                                  float(eps), _dt(x), _stream(stream)), "fuse_add_layernorm")
    return y


def fuse_add_layernorm_ex(x, residual, gamma, beta, eps=1e-5, relu=False, want_sum=False, want_stats=False,
                          y=None, sum_out=None, mean_out=None, var_out=None, stream=None):
    """LayerNorm variants in one pass: y (clamped at 0 when relu) and, on request, the pre-norm
    sum x + residual and the per-row fp32 mean and population variance.  Returns
    (y, sum, mean, var), None for an output not requested."""
    rows, hidden = _rows_cols(x)
    _check(x, "x")
    _check(residual, "residual", x.dtype, x.shape)
    _check(gamma, "gamma", x.dtype, (hidden,))
    _check(beta, "beta", x.dtype, (hidden,))
    if y is None:
        y = torch.empty_like(x)
    if want_sum and sum_out is None:
        sum_out = torch.empty_like(x)
    if want_stats and mean_out is None:
        mean_out = torch.empty(rows, dtype=torch.float32, device=x.device)
    if want_stats and var_out is None:
        var_out = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check(y, "y", x.dtype, x.shape)
    _check(sum_out, "sum_out", x.dtype, x.shape)
    _check(mean_out, "mean_out", torch.float32, (rows,))
    _check(var_out, "var_out", torch.float32, (rows,))
    _ok(load().fuse_add_layernorm_ex(_ptr(x), _ptr(residual), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(sum_out),
                                     _ptr(mean_out), _ptr(var_out), rows, hidden, float(eps),
                                     FUSE_LN_RELU if relu else 0, _dt(x), _stream(stream)),
        "fuse_add_layernorm_ex")
    return y, sum_out, mean_out, var_out


def fuse_bias_gelu_residual(x, bias, residual, y=None, stream=None):
    """y = GELU_erf(x + bias) + residual over the last dim."""
    rows, hidden = _rows_cols(x)
    _check(x, "x")
    _check(bias, "bias", x.dtype, (hidden,))
    _check(residual, "residual", x.dtype, x.shape)
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.dtype, x.shape)
    _ok(load().fuse_bias_gelu_residual(_ptr(x), _ptr(bias), _ptr(residual), _ptr(y), rows, hidden, _dt(x),
                                       _stream(stream)), "fuse_bias_gelu_residual")
    return y


def fuse_softmax_rows(x, scale=1.0, y=None, stream=None):
    """y = softmax(scale * x) over the last dim."""
    rows, cols = _rows_cols(x)
    _check(x, "x")
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.dtype, x.shape)
    _ok(load().fuse_softmax_rows(_ptr(x), _ptr(y), rows, cols, float(scale), _dt(x), _stream(stream)),
        "fuse_softmax_rows")
    return y


def fuse_cumsum_scale_rows(x, scale=1.0, y=None, stream=None):
    """y = scale * cumsum(x) over the last dim (inclusive running sum)."""
    rows, cols = _rows_cols(x)
    _check(x, "x")
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.dtype, x.shape)
    _ok(load().fuse_cumsum_scale_rows(_ptr(x), _ptr(y), rows, cols, float(scale), _dt(x), _stream(stream)),
        "fuse_cumsum_scale_rows")
    return y


def fuse_swiglu_dualgemm(a, b1, b2, out=None, stream=None):
    """out = SiLU(a @ b1) * (a @ b2); a [M,K], b1 and b2 [K,N], bf16."""
    M, K = a.shape
    N = b1.shape[1]
    _check(a, "a")
    _check(b1, "b1", a.dtype, (K, N))
    _check(b2, "b2", a.dtype, (K, N))
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    _check(out, "out", a.dtype, (M, N))
    _ok(load().fuse_swiglu_dualgemm(_ptr(a), _ptr(b1), _ptr(b2), _ptr(out), M, N, K, _dt(a), _stream(stream)),
        "fuse_swiglu_dualgemm")
    return out


def fuse_gemm_bias_act(x, w, bias=None, act="relu", y=None, stream=None):
    """y = act(x @ w + bias); x [M,K], w [K,N], bias [N] or None, bf16; act none/relu/gelu/silu."""
    M, K = x.shape
    N = w.shape[1]
    _check(x, "x")
    _check(w, "w", x.dtype, (K, N))
    _check(bias, "bias", x.dtype, (N,))
    if y is None:
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check(y, "y", x.dtype, (M, N))
    _ok(load().fuse_gemm_bias_act(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), M, N, K, FUSE_ACT[act], _dt(x),
                                  _stream(stream)), "fuse_gemm_bias_act")
    return y


def _auto_workspace(op, M, N, K, device, stream=None):
    n = load().fuse_auto_workspace_bytes(op, M, N, K, FUSE_BF16)
    if n == 0:
        return None, None, 0
    return _scratch(n, device, stream)


def fuse_auto_splits(op, M, N, K) -> int:
    """K splits the shape-dependent plan uses on the current device (1 = single fused kernel)."""
    return load().fuse_auto_splits(op, M, N, K)


def fuse_swiglu_auto(a, b1, b2, out=None, workspace=None, stream=None):
    """fuse_swiglu_dualgemm, or its split-K form when the tiles cannot fill the GPU."""
    M, K = a.shape
    N = b1.shape[1]
    _check(a, "a")
    _check(b1, "b1", a.dtype, (K, N))
    _check(b2, "b2", a.dtype, (K, N))
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    _check(out, "out", a.dtype, (M, N))
    ws = _caller_workspace(workspace) or _auto_workspace(FUSE_OP_SWIGLU, M, N, K, a.device, stream)
    _ok(load().fuse_swiglu_auto(_ptr(a), _ptr(b1), _ptr(b2), _ptr(out), M, N, K, _dt(a), ws[1], ws[2],
                                _stream(stream)), "fuse_swiglu_auto")
    return out


def fuse_swiglu_auto_noalloc(a, b1, b2, out=None, stream=None):
    """fuse_swiglu_auto without a workspace: the split-K partials go to the library's fixed
    per-device array (calls that overlap on one device race on it)."""
    M, K = a.shape
    N = b1.shape[1]
    _check(a, "a")
    _check(b1, "b1", a.dtype, (K, N))
    _check(b2, "b2", a.dtype, (K, N))
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    _check(out, "out", a.dtype, (M, N))
    _ok(load().fuse_swiglu_auto_noalloc(_ptr(a), _ptr(b1), _ptr(b2), _ptr(out), M, N, K, _dt(a), _stream(stream)),
        "fuse_swiglu_auto_noalloc")
    return out


def fuse_gemm_bias_act_auto(x, w, bias=None, act="relu", y=None, workspace=None, stream=None):
    """fuse_gemm_bias_act, or its split-K form when the tiles cannot fill the GPU."""
    M, K = x.shape
    N = w.shape[1]
    _check(x, "x")
    _check(w, "w", x.dtype, (K, N))
    _check(bias, "bias", x.dtype, (N,))
    if y is None:
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check(y, "y", x.dtype, (M, N))
    ws = _caller_workspace(workspace) or _auto_workspace(FUSE_OP_GEMM_BIAS_ACT, M, N, K, x.device, stream)
    _ok(load().fuse_gemm_bias_act_auto(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), M, N, K, FUSE_ACT[act], _dt(x),
                                       ws[1], ws[2], _stream(stream)), "fuse_gemm_bias_act_auto")
    return y


# ------------------------------------------------------------------------------------------------
# unfused baselines (the workspace is allocated here unless given as (tensor, ptr, bytes))
# ------------------------------------------------------------------------------------------------

def fuse_unfused_add_layernorm(x, residual, gamma, beta, eps=1e-5, y=None, workspace=None, stream=None):
    rows, hidden = _rows_cols(x)
    _check(x, "x")
    _check(residual, "residual", x.dtype, x.shape)
    _check(gamma, "gamma", x.dtype, (hidden,))
    _check(beta, "beta", x.dtype, (hidden,))
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.dtype, x.shape)
    ws = _caller_workspace(workspace) or _workspace(FUSE_OP_ADD_LAYERNORM, rows, hidden, 0, _dt(x), x.device, stream)
    _ok(load().fuse_unfused_add_layernorm(_ptr(x), _ptr(residual), _ptr(gamma), _ptr(beta), _ptr(y), rows,
                                          hidden, float(eps), _dt(x), ws[1], ws[2], _stream(stream)),
        "fuse_unfused_add_layernorm")
    return y


def fuse_unfused_bias_gelu_residual(x, bias, residual, y=None, workspace=None, stream=None):
    rows, hidden = _rows_cols(x)
    _check(x, "x")
    _check(bias, "bias", x.dtype, (hidden,))
    _check(residual, "residual", x.dtype, x.shape)
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.dtype, x.shape)
    ws = _caller_workspace(workspace) or _workspace(FUSE_OP_BIAS_GELU_RESIDUAL, rows, hidden, 0, _dt(x), x.device, stream)
    _ok(load().fuse_unfused_bias_gelu_residual(_ptr(x), _ptr(bias), _ptr(residual), _ptr(y), rows, hidden,
                                               _dt(x), ws[1], ws[2], _stream(stream)),
        "fuse_unfused_bias_gelu_residual")
    return y


def fuse_unfused_softmax_rows(x, scale=1.0, y=None, workspace=None, stream=None):
    rows, cols = _rows_cols(x)
    _check(x, "x")
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.dtype, x.shape)
    ws = _caller_workspace(workspace) or _workspace(FUSE_OP_SOFTMAX_ROWS, rows, cols, 0, _dt(x), x.device, stream)
    _ok(load().fuse_unfused_softmax_rows(_ptr(x), _ptr(y), rows, cols, float(scale), _dt(x), ws[1], ws[2],
                                         _stream(stream)), "fuse_unfused_softmax_rows")
    return y


def fuse_unfused_cumsum_scale_rows(x, scale=1.0, y=None, workspace=None, stream=None):
    rows, cols = _rows_cols(x)
    _check(x, "x")
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.dtype, x.shape)
    ws = _caller_workspace(workspace) or _workspace(FUSE_OP_CUMSUM_SCALE, rows, cols, 0, _dt(x), x.device, stream)
    _ok(load().fuse_unfused_cumsum_scale_rows(_ptr(x), _ptr(y), rows, cols, float(scale), _dt(x), ws[1], ws[2],
                                              _stream(stream)), "fuse_unfused_cumsum_scale_rows")
    return y


def fuse_unfused_swiglu(a, b1, b2, out=None, workspace=None, stream=None):
    M, K = a.shape
    N = b1.shape[1]
    _check(a, "a")
    _check(b1, "b1", a.dtype, (K, N))
    _check(b2, "b2", a.dtype, (K, N))
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    _check(out, "out", a.dtype, (M, N))
    ws = _caller_workspace(workspace) or _workspace(FUSE_OP_SWIGLU, M, N, K, _dt(a), a.device, stream)
    _ok(load().fuse_unfused_swiglu(_ptr(a), _ptr(b1), _ptr(b2), _ptr(out), M, N, K, _dt(a), ws[1], ws[2],
                                   _stream(stream)), "fuse_unfused_swiglu")
    return out


def fuse_unfused_workspace_bytes(op: int, d0: int, d1: int, d2: int, dtype) -> int:
    code = _DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(load().fuse_unfused_workspace_bytes(op, d0, d1, d2, code))


def fuse_unfused_gemm_bias_act(x, w, bias=None, act="relu", y=None, workspace=None, stream=None):
    M, K = x.shape
    N = w.shape[1]
    _check(x, "x")
    _check(w, "w", x.dtype, (K, N))
    _check(bias, "bias", x.dtype, (N,))
    if y is None:
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check(y, "y", x.dtype, (M, N))
    ws = _caller_workspace(workspace) or _workspace(FUSE_OP_GEMM_BIAS_ACT, M, N, K, _dt(x), x.device, stream)
    _ok(load().fuse_unfused_gemm_bias_act(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), M, N, K, FUSE_ACT[act], _dt(x),
                                          ws[1], ws[2], _stream(stream)), "fuse_unfused_gemm_bias_act")
    return y


def fuse_copy(src, dst, stream=None):
    """Byte copy of src into dst (same byte size); roofline calibration kernel."""
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("src and dst differ in size")
    _check(src, "src")
    _check(dst, "dst")
    _ok(load().fuse_copy(_ptr(src), _ptr(dst), nb, _stream(stream)), "fuse_copy")
    return dst


def fuse_mfma_ceiling(workgroups, iters, out, stream=None):
    """Matrix-core calibration kernel: `workgroups` x 4 waves x `iters` rounds of 8 bf16 32x32x16
    MFMAs from registers; out (fp32, >= workgroups * 256 values) receives 2048 * iters per thread."""
    if out.dtype != torch.float32 or out.numel() < int(workgroups) * 256:
        raise ValueError("out must be fp32 with at least workgroups * 256 values")
    _check(out, "out")
    _ok(load().fuse_mfma_ceiling(int(workgroups), int(iters), _ptr(out), _stream(stream)), "fuse_mfma_ceiling")
    return out


def fuse_empty_kernels(count, stream=None):
    """Enqueue `count` launches of the empty probe kernel (launch-cost measurement)."""
    _ok(load().fuse_empty_kernels(int(count), _stream(stream)), "fuse_empty_kernels")


def fuse_version() -> str:
    return load().fuse_version().decode()
