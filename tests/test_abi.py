"""The C-ABI library without a GPU: it loads, exports every symbol the header declares, and
rejects bad arguments with the documented status before touching any device.

Only argument combinations that fail validation (or are documented no-ops) are passed here, so
nothing is ever launched.  The fake pointer values are never dereferenced: validation compares
addresses only.
"""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "libfuse.h")

OK, NULL, SHAPE, DTYPE, VALUE, ALIAS, UNSUP, WS, MISAL, HIP = range(10)
F32, F16, BF16 = 0, 1, 2
P = 1 << 20  # fake, 256-byte aligned "device" addresses; never dereferenced


@pytest.fixture(scope="module")
def lib():
    from memory_bound_amd import api as libfuse
    if not os.path.exists(libfuse.LIB_PATH):
        import memory_bound_amd.build as b
        b.build()
    return libfuse.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fuse_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_operations():
    names = declared_functions()
    for n in ("fuse_add_layernorm", "fuse_bias_gelu_residual", "fuse_softmax_rows", "fuse_swiglu_dualgemm"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from memory_bound_amd import api as libfuse
    names = declared_functions()
    assert set(names) == set(libfuse.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_header_is_c99_and_every_symbol_links(tmp_path, lib):
    # a plain C program (no C++, no HIP headers) compiled against the header with -pedantic and
    # linked against the library: it takes the address of every declared entry point and makes
    # calls that validation answers or that are documented no-ops, so nothing is launched
    import shutil
    import subprocess
    from memory_bound_amd import api as libfuse
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    names = declared_functions()
    src = "\n".join([
        "#include <stdio.h>", "#include <string.h>", '#include "libfuse.h"',
        "typedef void (*fn_t)(void);",
        "static const fn_t every_entry_point[] = {" + ", ".join(f"(fn_t){n}" for n in names) + "};",
        "int main(void) {",
        "    int bad = 0;",
        "    if (sizeof every_entry_point / sizeof every_entry_point[0] != %d) bad |= 1;" % len(names),
        '    if (strstr(fuse_version(), "gfx950") == NULL) bad |= 2;',
        "    if (fuse_add_layernorm(NULL, NULL, NULL, NULL, NULL, 4, 64, 1e-5f, FUSE_F16, NULL)",
        "        != FUSE_ERR_NULL_PTR) bad |= 4;",
        "    if (fuse_add_layernorm(NULL, NULL, NULL, NULL, NULL, 0, 64, 1e-5f, FUSE_F16, NULL) != FUSE_OK) bad |= 8;",
        "    if (fuse_softmax_rows(NULL, NULL, 4, 0, 1.0f, FUSE_F16, NULL) != FUSE_ERR_BAD_SHAPE) bad |= 16;",
        "    if (fuse_swiglu_dualgemm(NULL, NULL, NULL, NULL, 64, 64, 64, FUSE_F16, NULL) != FUSE_ERR_BAD_DTYPE)",
        "        bad |= 32;",
        '    if (strncmp(fuse_status_string(FUSE_ERR_ALIAS), "FUSE_ERR_ALIAS", 14) != 0) bad |= 64;',
        '    printf("bad=%d\\n", bad);',
        "    return bad;",
        "}", ""])
    (tmp_path / "abi.c").write_text(src)
    libdir = os.path.dirname(libfuse.LIB_PATH)
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.dirname(HEADER),
           str(tmp_path / "abi.c"), "-L", libdir, "-lfuse", f"-Wl,-rpath,{libdir}",
           "-Wl,-rpath-link,/opt/rocm/lib", "-o", str(tmp_path / "abi")]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stderr
    r = subprocess.run([str(tmp_path / "abi")], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr


def test_status_strings_and_version(lib):
    for code in range(10):
        s = lib.fuse_status_string(code).decode()
        assert s.startswith("FUSE_")
    assert b"gfx950" in lib.fuse_version()
    assert lib.fuse_last_hip_error() == 0


def v(x):
    return ctypes.c_void_p(x)


def ln(lib, x=P, r=2 * P, g=3 * P, b=4 * P, y=5 * P, rows=4, hidden=64, eps=1e-5, dt=F16):
    return lib.fuse_add_layernorm(v(x), v(r), v(g), v(b), v(y), rows, hidden, eps, dt, None)


def test_add_layernorm_validation(lib):
    H = 1 << 12  # bytes per 64-element... spacing between fake buffers is 1 MiB, large enough
    assert ln(lib, x=0) == NULL
    assert ln(lib, g=0) == NULL
    assert ln(lib, b=0) == NULL
    assert ln(lib, y=0) == NULL
    assert ln(lib, rows=-1) == SHAPE
    assert ln(lib, hidden=0) == SHAPE
    assert ln(lib, hidden=16385) == UNSUP
    assert ln(lib, dt=7) == DTYPE
    assert ln(lib, eps=float("nan")) == VALUE
    assert ln(lib, eps=float("inf")) == VALUE
    assert ln(lib, eps=-1.0) == VALUE
    assert ln(lib, x=P + 1) == MISAL
    assert ln(lib, y=P + 2) == ALIAS            # partial overlap with x
    assert ln(lib, y=3 * P + 64) == ALIAS       # overlaps gamma
    assert ln(lib, y=3 * P) == ALIAS            # equals gamma: still not allowed
    assert ln(lib, rows=0) == OK                # no-op, nothing launched
    assert ln(lib, rows=0, x=0, y=0) == OK
    assert ln(lib, rows=1 << 31) == SHAPE
    assert H


def ln_ex(lib, x=P, r=2 * P, g=3 * P, b=4 * P, y=5 * P, s=6 * P, m=7 * P, var=8 * P, rows=4, hidden=64,
          eps=1e-5, flags=1, dt=F16):
    return lib.fuse_add_layernorm_ex(v(x), v(r), v(g), v(b), v(y), v(s), v(m), v(var), rows, hidden, eps, flags,
                                     dt, None)


def test_add_layernorm_ex_validation(lib):
    # the checks of the plain entry point first
    assert ln_ex(lib, x=0) == NULL
    assert ln_ex(lib, hidden=16385) == UNSUP
    assert ln_ex(lib, eps=float("nan")) == VALUE
    assert ln_ex(lib, y=P + 2) == ALIAS
    # then the variants' own arguments
    assert ln_ex(lib, flags=2) == VALUE
    assert ln_ex(lib, flags=0xFFFFFFFF) == VALUE
    assert ln_ex(lib, s=5 * P) == ALIAS          # sum_out equal to y
    assert ln_ex(lib, s=5 * P + 128) == ALIAS    # sum_out overlapping y
    assert ln_ex(lib, s=3 * P) == ALIAS          # sum_out on gamma
    assert ln_ex(lib, s=P + 64) == ALIAS         # sum_out partially over x
    assert ln_ex(lib, s=6 * P + 1) == MISAL
    assert ln_ex(lib, m=7 * P + 2) == MISAL
    assert ln_ex(lib, m=P) == ALIAS              # mean_out inside x
    assert ln_ex(lib, var=5 * P + 256) == ALIAS  # var_out inside y
    assert ln_ex(lib, var=7 * P + 8) == ALIAS    # var_out overlapping mean_out
    assert ln_ex(lib, m=6 * P) == ALIAS          # mean_out inside sum_out
    assert ln_ex(lib, rows=0) == OK              # no-op, nothing launched
    assert ln_ex(lib, rows=0, flags=4) == VALUE  # flags are checked even for an empty call


def test_bias_gelu_residual_validation(lib):
    def call(x=P, bias=2 * P, r=3 * P, y=4 * P, rows=4, hidden=64, dt=F16):
        return lib.fuse_bias_gelu_residual(v(x), v(bias), v(r), v(y), rows, hidden, dt, None)
    assert call(bias=0) == NULL
    assert call(r=0) == NULL
    assert call(hidden=0) == SHAPE
    assert call(dt=5) == DTYPE
    assert call(y=2 * P) == ALIAS               # writes over the bias
    assert call(y=3 * P + 16) == ALIAS          # partial overlap with residual
    assert call(rows=1 << 20, hidden=1 << 14) == SHAPE  # 2^34 elements
    assert call(rows=0) == OK


def test_softmax_validation(lib):
    def call(x=P, y=2 * P, rows=4, cols=64, scale=1.0, dt=F16):
        return lib.fuse_softmax_rows(v(x), v(y), rows, cols, scale, dt, None)
    assert call(x=0) == NULL
    assert call(cols=0) == SHAPE
    assert call(cols=16385) == UNSUP
    assert call(scale=float("inf")) == VALUE
    assert call(scale=float("nan")) == VALUE
    assert call(y=P + 64) == ALIAS
    assert call(x=P + 1) == MISAL
    assert call(dt=3) == DTYPE
    assert call(rows=0) == OK


def test_cumsum_validation(lib):
    def call(x=P, y=2 * P, rows=4, cols=64, scale=0.5, dt=F16):
        return lib.fuse_cumsum_scale_rows(v(x), v(y), rows, cols, scale, dt, None)
    assert call(x=0) == NULL
    assert call(y=0) == NULL
    assert call(cols=0) == SHAPE
    assert call(rows=-2) == SHAPE
    assert call(cols=16385) == UNSUP
    assert call(dt=5) == DTYPE
    assert call(scale=float("inf")) == VALUE
    assert call(scale=float("nan")) == VALUE
    assert call(y=P + 2) == ALIAS
    assert call(x=P + 1) == MISAL
    assert call(rows=0) == OK
    n = lib.fuse_unfused_workspace_bytes(4, 4, 64, 0, F16)
    assert n == 512
    assert lib.fuse_unfused_cumsum_scale_rows(v(P), v(2 * P), 4, 64, 0.5, F16, v(0), n, None) == WS
    assert lib.fuse_unfused_cumsum_scale_rows(v(P), v(2 * P), 4, 64, 0.5, F16, v(3 * P), n - 1, None) == WS
    assert lib.fuse_unfused_cumsum_scale_rows(v(P), v(2 * P), 4, 64, 0.5, F16, v(3 * P + 16), n, None) == WS
    assert lib.fuse_unfused_cumsum_scale_rows(v(P), v(2 * P), 4, 64, 0.5, F16, v(P), n, None) == WS


def test_swiglu_validation(lib):
    def call(a=P, b1=8 * P, b2=16 * P, out=24 * P, M=128, N=128, K=64, dt=BF16):
        return lib.fuse_swiglu_dualgemm(v(a), v(b1), v(b2), v(out), M, N, K, dt, None)
    assert call(dt=F16) == DTYPE
    assert call(dt=F32) == DTYPE
    assert call(a=0) == NULL
    assert call(N=0) == SHAPE
    assert call(K=0) == SHAPE
    assert call(M=-1) == SHAPE
    assert call(M=1 << 31) == SHAPE
    assert call(out=8 * P) == ALIAS             # out over b1
    assert call(out=P) == ALIAS                 # out over a (in-place is not allowed here)
    assert call(b1=8 * P + 1) == MISAL
    assert call(M=0) == OK


def test_gemm_bias_act_validation(lib):
    def call(x=P, w=2 * P, b=3 * P, y=4 * P, M=256, N=256, K=64, act=1, dt=BF16):
        return lib.fuse_gemm_bias_act(v(x), v(w), v(b), v(y), M, N, K, act, dt, None)
    assert call(x=0) == NULL
    assert call(w=0) == NULL
    assert call(y=0) == NULL
    assert call(b=0, M=0) == OK         # no bias is allowed (M = 0: nothing launched)
    assert call(b=0, dt=F16) == DTYPE
    assert call(dt=F16) == DTYPE
    assert call(act=4) == VALUE
    assert call(act=-1) == VALUE
    assert call(N=0) == SHAPE
    assert call(M=-1) == SHAPE
    assert call(K=(1 << 21) + 1) == UNSUP
    assert call(y=2 * P + 64) == ALIAS      # y over w
    assert call(y=3 * P) == ALIAS           # y over bias
    assert call(b=3 * P + 1) == MISAL
    assert call(M=0) == OK
    n = lib.fuse_unfused_workspace_bytes(5, 256, 256, 64, BF16)
    assert n == 2 * 256 * 256 * 2
    assert lib.fuse_unfused_workspace_bytes(5, 256, 256, 64, F16) == 0
    assert lib.fuse_unfused_gemm_bias_act(v(P), v(2 * P), v(3 * P), v(4 * P), 256, 256, 64, 1, BF16, v(0), n,
                                          None) == WS
    assert lib.fuse_unfused_gemm_bias_act(v(P), v(2 * P), v(3 * P), v(4 * P), 256, 256, 64, 1, BF16, v(5 * P),
                                          n - 256, None) == WS


def test_auto_plan_and_validation(lib):
    # Plans depend only on the shape and the CU count (256 here when no device answers, as on the
    # MI355X): below half the CUs in tiles, the split count the library's cost model prices
    # cheapest (the values below are that model's choices for 256 CUs).
    SW, GM = 3, 5
    assert lib.fuse_auto_splits(SW, 2048, 8960, 1536) == 1               # 560 tiles: single kernel
    assert lib.fuse_auto_splits(GM, 2048, 8960, 1536) == 1               # 280 tiles: single kernel
    assert lib.fuse_auto_splits(SW, 300, 512, 1536) == 1                 # ragged M: single kernel
    assert lib.fuse_auto_splits(SW, 256, 512, 1536) == 8                 # 4 tiles, 48 K steps
    assert lib.fuse_auto_splits(SW, 256, 512, 96) == 1                   # 3 K steps: too short to split
    assert lib.fuse_auto_splits(SW, 512, 2048, 1536) == 3                # 32 tiles
    assert lib.fuse_auto_splits(SW, 1024, 2048, 1536) == 1               # 64 tiles, 48 K steps: not worth it
    assert lib.fuse_auto_splits(SW, 2048, 1024, 4096) == 4               # 64 tiles, 128 K steps
    assert lib.fuse_auto_splits(GM, 2048, 2048, 2048) == 3               # 64 tiles of 256 x 256
    assert lib.fuse_auto_splits(GM, 2048, 2048, 512) == 1                # 16 K steps: not worth it
    assert lib.fuse_auto_splits(SW, 2048, 2048, 4096) == 1               # 128 tiles: half the CUs
    assert lib.fuse_auto_splits(GM, 256, 512, 1536) == 12                # 2 tiles of 256 x 256
    assert lib.fuse_auto_splits(SW, 0, 512, 1536) == 0
    assert lib.fuse_auto_workspace_bytes(SW, 256, 512, 1536, BF16) == 8 * 2 * 256 * 512 * 4
    assert lib.fuse_auto_workspace_bytes(GM, 256, 512, 1536, BF16) == 12 * 256 * 512 * 4
    assert lib.fuse_auto_workspace_bytes(SW, 2048, 8960, 1536, BF16) == 0
    assert lib.fuse_auto_workspace_bytes(SW, 256, 512, 1536, F16) == 0
    Q = 16 * P  # 16 MiB apart: the operands of these shapes do not overlap each other
    sw = lambda ws, n, **k: lib.fuse_swiglu_auto(v(Q), v(2 * Q), v(3 * Q), v(4 * Q), k.get("M", 256), 512, 1536,
                                                 k.get("dt", BF16), v(ws), n, None)
    assert sw(0, 0) == WS                       # split plan needs a workspace
    assert sw(5 * Q, 1000) == WS                # too small
    assert sw(5 * Q + 16, 1 << 24) == WS        # not 256-byte aligned
    assert sw(Q, 1 << 24) == WS                 # overlaps a
    assert sw(0, 0, dt=F16) == DTYPE
    assert sw(0, 0, M=0) == OK
    gm = lambda ws, n, act=1: lib.fuse_gemm_bias_act_auto(v(Q), v(2 * Q), v(3 * Q), v(4 * Q), 256, 512, 1536, act,
                                                          BF16, v(ws), n, None)
    assert gm(0, 0) == WS
    assert gm(0, 0, act=9) == VALUE
    assert gm(4 * Q, 1 << 24) == WS             # overlaps y


def test_swiglu_noalloc_validation(lib, monkeypatch):
    SW = 3
    Q = 16 * P
    def call(a=Q, M=256, N=512, K=1536, dt=BF16):
        return lib.fuse_swiglu_auto_noalloc(v(a), v(2 * Q), v(3 * Q), v(4 * Q), M, N, K, dt, None)
    assert call(dt=F16) == DTYPE
    assert call(a=0) == NULL
    assert call(M=0) == OK                      # no-op
    assert call(M=0, a=0) == OK
    assert call(K=(1 << 21) + 1) == UNSUP
    assert call(a=Q + 1) == MISAL
    # a plan whose partials exceed the fixed 64 MiB array is refused before anything is launched
    monkeypatch.setenv("FUSE_SPLITK", "48")
    assert lib.fuse_auto_workspace_bytes(SW, 1024, 1024, 1536, BF16) == 48 * 2 * 1024 * 1024 * 4
    Q2 = 64 * P
    assert lib.fuse_swiglu_auto_noalloc(v(Q2), v(2 * Q2), v(3 * Q2), v(4 * Q2), 1024, 1024, 1536, BF16, None) == WS


def test_unfused_workspace_bytes(lib):
    f = lib.fuse_unfused_workspace_bytes
    t = 2048 * 4096 * 2
    assert f(0, 2048, 4096, 0, F16) == t
    assert f(1, 2048, 4096, 0, F16) == 2 * t
    assert f(2, 65536, 2048, 0, F16) == 65536 * 2048 * 2 + 2 * 65536 * 4
    assert f(3, 2048, 8960, 1536, BF16) == 2 * 2048 * 8960 * 2
    assert f(3, 2048, 8960, 1536, F16) == 0
    assert f(0, -1, 4096, 0, F16) == 0
    assert f(9, 1, 1, 1, F16) == 0


def test_unfused_validation(lib):
    need = lib.fuse_unfused_workspace_bytes(0, 4, 64, 0, F16)
    ws = 40 * P
    args = [v(P), v(2 * P), v(3 * P), v(4 * P), v(5 * P), 4, 64, 1e-5, F16]
    assert lib.fuse_unfused_add_layernorm(*args, v(0), need, None) == WS
    assert lib.fuse_unfused_add_layernorm(*args, v(ws), need - 1, None) == WS
    assert lib.fuse_unfused_add_layernorm(*args, v(ws + 16), need, None) == WS   # not 256-aligned
    assert lib.fuse_unfused_add_layernorm(*args, v(P), need, None) == WS         # overlaps x
    no_res = [v(P), v(0), v(3 * P), v(4 * P), v(5 * P), 4, 64, 1e-5, F16]
    assert lib.fuse_unfused_add_layernorm(*no_res, v(ws), need, None) == NULL
    sw = lib.fuse_unfused_workspace_bytes(3, 128, 128, 64, BF16)
    assert lib.fuse_unfused_swiglu(v(P), v(8 * P), v(16 * P), v(24 * P), 128, 128, 64, BF16, v(ws),
                                   sw - 256, None) == WS


def test_copy_validation(lib):
    assert lib.fuse_copy(v(P), v(P + 8), 64, None) == ALIAS
    assert lib.fuse_copy(v(0), v(P), 64, None) == NULL
    assert lib.fuse_copy(v(P), v(2 * P), 0, None) == OK
    assert lib.fuse_copy(v(P), v(2 * P), (1 << 40) + 1, None) == SHAPE


def test_mfma_ceiling_validation(lib):
    assert lib.fuse_mfma_ceiling(0, 16, v(P), None) == SHAPE
    assert lib.fuse_mfma_ceiling(65537, 16, v(P), None) == SHAPE
    assert lib.fuse_mfma_ceiling(8, 0, v(P), None) == SHAPE
    assert lib.fuse_mfma_ceiling(8, (1 << 24) + 1, v(P), None) == SHAPE
    assert lib.fuse_mfma_ceiling(8, 16, v(0), None) == NULL
    assert lib.fuse_mfma_ceiling(8, 16, v(P + 2), None) == MISAL


def test_empty_kernels_validation(lib):
    assert lib.fuse_empty_kernels(-1, None) == SHAPE
    assert lib.fuse_empty_kernels((1 << 20) + 1, None) == SHAPE
    assert lib.fuse_empty_kernels(0, None) == OK  # nothing enqueued


def test_python_binding_refuses_cpu_tensors():
    import torch
    from memory_bound_amd import api as libfuse
    x = torch.zeros(4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        libfuse.fuse_add_layernorm(x, x, x[0], x[0])


class _GpuStandIn:
    """Looks like a contiguous GPU tensor to the binding's checks; taking its pointer fails the
    test, so any call that gets past the checks is caught before it reaches the library."""
    is_cuda = True

    def __init__(self, shape, dtype, index=0):
        import torch
        self.shape, self.dtype, self.device = torch.Size(shape), dtype, torch.device("cuda", index)

    def is_contiguous(self):
        return True

    def dim(self):
        return len(self.shape)

    def numel(self):
        n = 1
        for d in self.shape:
            n *= d
        return n

    def element_size(self):
        return 4 if str(self.dtype) == "torch.float32" else 2

    def data_ptr(self):
        raise AssertionError("a pointer was taken before every operand was checked")


def _binding_cases():
    import torch
    h, b, f = torch.float16, torch.bfloat16, torch.float32
    R, H, M, N, K = 4, 64, 32, 48, 16
    row = dict(x=((R, H), h), y=((R, H), h))
    ln = dict(x=((R, H), h), residual=((R, H), h), gamma=((H,), h), beta=((H,), h), y=((R, H), h))
    gelu = dict(x=((R, H), h), bias=((H,), h), residual=((R, H), h), y=((R, H), h))
    sw = dict(a=((M, K), b), b1=((K, N), b), b2=((K, N), b), out=((M, N), b))
    gm = dict(x=((M, K), b), w=((K, N), b), bias=((N,), b), y=((M, N), b))
    return [
        ("fuse_add_layernorm", ln, {}),
        ("fuse_add_layernorm_ex", dict(ln, sum_out=((R, H), h), mean_out=((R,), f), var_out=((R,), f)), {}),
        ("fuse_bias_gelu_residual", gelu, {}),
        ("fuse_softmax_rows", row, {}),
        ("fuse_cumsum_scale_rows", row, {}),
        ("fuse_swiglu_dualgemm", sw, {}),
        ("fuse_swiglu_auto", sw, {"workspace": (None, None, 0)}),
        ("fuse_swiglu_auto_noalloc", sw, {}),
        ("fuse_gemm_bias_act", gm, {}),
        ("fuse_gemm_bias_act_auto", gm, {"workspace": (None, None, 0)}),
        ("fuse_unfused_add_layernorm", ln, {"workspace": (None, None, 0)}),
        ("fuse_unfused_bias_gelu_residual", gelu, {"workspace": (None, None, 0)}),
        ("fuse_unfused_softmax_rows", row, {"workspace": (None, None, 0)}),
        ("fuse_unfused_cumsum_scale_rows", row, {"workspace": (None, None, 0)}),
        ("fuse_unfused_swiglu", sw, {"workspace": (None, None, 0)}),
        ("fuse_unfused_gemm_bias_act", gm, {"workspace": (None, None, 0)}),
        ("fuse_copy", dict(src=((R, H), h), dst=((R, H), h)), {}),
    ]


@pytest.mark.parametrize("case", _binding_cases(), ids=lambda c: c[0])
def test_python_binding_checks_every_operand(monkeypatch, case):
    # one operand at a time is a CPU tensor, or a GPU tensor on another device than the current
    # one: the wrapper must raise before taking any pointer, whichever operand it is
    import torch
    from memory_bound_amd import api as libfuse
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    monkeypatch.setattr(libfuse, "load", lambda: pytest.fail("the library was called"))
    name, ops, extra = case
    fn = getattr(libfuse, name)
    for bad in ops:
        for kind in ("cpu", "other device"):
            args = {}
            for k, (shape, dt) in ops.items():
                if k != bad:
                    args[k] = _GpuStandIn(shape, dt)
                elif kind == "cpu":
                    args[k] = torch.zeros(shape, dtype=dt)
                else:
                    args[k] = _GpuStandIn(shape, dt, index=1)
            with pytest.raises(ValueError):
                fn(**args, **extra)
