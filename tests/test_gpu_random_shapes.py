"""Seeded random shapes for every fused operation (GPU required): row lengths across the whole
supported range, odd row counts, every storage type, with and without the residual, random
activations and LayerNorm-variant outputs, and tensors that start one element past a 16-byte
boundary (the per-element paths), and whole-tile dual-product shapes (the persistent kernel, its
last-round slices, the split-K plans).  Each result is compared with the CPU oracle element by
element under the operation's rule.  The shapes are drawn once from a fixed seed, so a failure
names a case that can be rerun alone.
"""
import numpy as np
import pytest
import torch

import oracle
from memory_bound_amd import api, synth
from oracle.tolerance import assert_close

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f16", "bf16"]


def _cases(seed, n, draw):
    rng = np.random.default_rng(seed)
    return [draw(rng) for _ in range(n)]


def _row_case(rng, max_cols):
    return (int(rng.integers(1, 40)), int(rng.integers(1, max_cols + 1)), DTYPES[int(rng.integers(0, 3))],
            int(rng.integers(0, 2)))


def _place(t, offset):
    """The tensor on the GPU, starting `offset` elements into a fresh allocation."""
    flat = torch.empty(t.numel() + offset, dtype=t.dtype, device="cuda")
    view = flat[offset:offset + t.numel()].view(t.shape)
    view.copy_(t.to("cuda"))
    return view


def _out_like(t, offset):
    flat = torch.empty(t.numel() + offset, dtype=t.dtype, device="cuda")
    return flat[offset:offset + t.numel()].view(t.shape)


def announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


LN_CASES = _cases(20261203, 16, lambda r: _row_case(r, 16384) + (bool(r.integers(0, 2)),))


@pytest.mark.parametrize("rows,hidden,dtype,offset,res", LN_CASES)
def test_add_layernorm_random(rows, hidden, dtype, offset, res):
    announce(f"add_layernorm random {rows}x{hidden} {dtype} offset={offset} residual={res}")
    d = synth.add_layernorm_inputs(rows, hidden, dtype, seed=rows * 31 + hidden)
    x = _place(d["x"], offset)
    r = _place(d["residual"], offset) if res else None
    y = _out_like(d["x"], offset)
    api.fuse_add_layernorm(x, r, d["gamma"].cuda(), d["beta"].cuda(), d["eps"], y=y)
    ref = oracle.add_layernorm(d["x"], d["residual"] if res else None, d["gamma"], d["beta"], np.float32(d["eps"]))
    assert_close(y, ref, dtype, f"ln {rows}x{hidden} {dtype} off={offset} res={res}")


GELU_CASES = _cases(20261204, 12, lambda r: _row_case(r, 20000))


@pytest.mark.parametrize("rows,hidden,dtype,offset", GELU_CASES)
def test_bias_gelu_residual_random(rows, hidden, dtype, offset):
    announce(f"bias_gelu_residual random {rows}x{hidden} {dtype} offset={offset}")
    d = synth.bias_gelu_residual_inputs(rows, hidden, dtype, seed=rows * 37 + hidden)
    y = _out_like(d["x"], offset)
    api.fuse_bias_gelu_residual(_place(d["x"], offset), d["bias"].cuda(), _place(d["residual"], offset), y=y)
    assert_close(y, oracle.bias_gelu_residual(d["x"], d["bias"], d["residual"]), dtype,
                 f"gelu {rows}x{hidden} {dtype} off={offset}")


SOFTMAX_CASES = _cases(20261205, 14, lambda r: _row_case(r, 16384) + (float(r.uniform(-2.0, 2.0)),))


@pytest.mark.parametrize("rows,cols,dtype,offset,scale", SOFTMAX_CASES)
def test_softmax_random(rows, cols, dtype, offset, scale):
    announce(f"softmax random {rows}x{cols} {dtype} offset={offset} scale={scale:.4f}")
    d = synth.softmax_inputs(rows, cols, dtype, seed=rows * 41 + cols)
    y = _out_like(d["x"], offset)
    api.fuse_softmax_rows(_place(d["x"], offset), scale, y=y)
    assert_close(y, oracle.softmax_rows(d["x"], np.float32(scale)), dtype,
                 f"softmax {rows}x{cols} {dtype} off={offset} scale={scale}")


CUMSUM_CASES = _cases(20261206, 14, lambda r: _row_case(r, 16384))


@pytest.mark.parametrize("rows,cols,dtype,offset", CUMSUM_CASES)
def test_cumsum_random(rows, cols, dtype, offset):
    announce(f"cumsum random {rows}x{cols} {dtype} offset={offset}")
    d = synth.cumsum_inputs(rows, cols, dtype, seed=rows * 43 + cols)
    y = _out_like(d["x"], offset)
    api.fuse_cumsum_scale_rows(_place(d["x"], offset), d["scale"], y=y)
    assert_close(y, oracle.cumsum_scale_rows(d["x"], np.float32(d["scale"])), dtype,
                 f"cumsum {rows}x{cols} {dtype} off={offset}")


def _mnk(rng):
    return (int(rng.integers(1, 300)), int(rng.integers(1, 400)), int(rng.integers(1, 300)), int(rng.integers(0, 2)))


SWIGLU_CASES = _cases(20261207, 10, _mnk)


@pytest.mark.parametrize("M,N,K,offset", SWIGLU_CASES)
def test_swiglu_random(M, N, K, offset):
    announce(f"swiglu random {M}x{N}x{K} offset={offset}")
    d = synth.swiglu_inputs(M, N, K, "bf16", seed=M + 3 * N + 7 * K)
    out = torch.empty(M * N + offset, dtype=torch.bfloat16, device="cuda")[offset:].view(M, N)
    api.fuse_swiglu_dualgemm(_place(d["a"], offset), _place(d["b1"], offset), _place(d["b2"], offset), out=out)
    assert_close(out, oracle.swiglu(d["a"], d["b1"], d["b2"]), "bf16", f"swiglu {M}x{N}x{K} off={offset}")


GEMM_CASES = _cases(20261208, 10, lambda r: _mnk(r) + (["none", "relu", "gelu", "silu"][int(r.integers(0, 4))],))


@pytest.mark.parametrize("M,N,K,offset,act", GEMM_CASES)
def test_gemm_bias_act_random(M, N, K, offset, act):
    announce(f"gemm_bias_act random {M}x{N}x{K} offset={offset} {act}")
    d = synth.gemm_inputs(M, N, K, "bf16", seed=M + 5 * N + 11 * K)
    y = torch.empty(M * N + offset, dtype=torch.bfloat16, device="cuda")[offset:].view(M, N)
    api.fuse_gemm_bias_act(_place(d["x"], offset), _place(d["w"], offset), d["bias"].cuda(), act, y=y)
    assert_close(y, oracle.gemm_bias_act(d["x"], d["w"], d["bias"], act), "bf16",
                 f"gemm {M}x{N}x{K} off={offset} {act}")


LN_EX_CASES = _cases(20261209, 12, lambda r: (int(r.integers(1, 40)), int(r.integers(2, 16385)),
                                              DTYPES[int(r.integers(0, 3))], bool(r.integers(0, 2)),
                                              bool(r.integers(0, 2)), bool(r.integers(0, 2))))


@pytest.mark.parametrize("rows,hidden,dtype,relu,want_sum,want_stats", LN_EX_CASES)
def test_add_layernorm_ex_random(rows, hidden, dtype, relu, want_sum, want_stats):
    from test_gpu_parity import _check_ln_ex
    announce(f"add_layernorm_ex random {rows}x{hidden} {dtype} relu={relu} sum={want_sum} stats={want_stats}")
    d = synth.add_layernorm_inputs(rows, hidden, dtype, seed=rows * 47 + hidden)
    outs = api.fuse_add_layernorm_ex(d["x"].cuda(), d["residual"].cuda(), d["gamma"].cuda(), d["beta"].cuda(),
                                     d["eps"], relu=relu, want_sum=want_sum, want_stats=want_stats)
    assert (outs[1] is not None) == want_sum and (outs[2] is not None) == want_stats
    _check_ln_ex(outs, d, relu, dtype, f"ln_ex {rows}x{hidden} {dtype} relu={relu} sum={want_sum} stats={want_stats}")


def _full_tile_case(rng):
    gemm = bool(rng.integers(0, 2))
    return (256 * int(rng.integers(1, 9)), (256 if gemm else 128) * int(rng.integers(1, 37 if gemm else 73)),
            32 * int(rng.integers(1, 65)), gemm, bool(rng.integers(0, 2)), ["none", "relu", "gelu", "silu"][int(rng.integers(0, 4))])


FULL_TILE_CASES = _cases(20261210, 12, _full_tile_case)


@pytest.mark.parametrize("M,N,K,gemm,auto,act", FULL_TILE_CASES)
def test_dual_product_full_tile_random(M, N, K, gemm, auto, act):
    """Shapes made of whole 256-row tiles: the full-tile kernels (one workgroup per CU walking its
    units when they outnumber the CUs, last-round slices) and, through the *_auto entry points,
    the split-K plans; 12 sampled rows against the oracle."""
    op = api.FUSE_OP_GEMM_BIAS_ACT if gemm else api.FUSE_OP_SWIGLU
    splits = api.fuse_auto_splits(op, M, N, K) if auto else 1
    announce(f"{'gemm ' + act if gemm else 'swiglu'} full tiles {M}x{N}x{K} auto={auto} splits={splits}")
    rows = torch.from_numpy(np.sort(np.random.default_rng(M + N + K).choice(M, size=12, replace=False)))
    if gemm:
        d = synth.gemm_inputs(M, N, K, "bf16", seed=M + 3 * N + 5 * K)
        x, w, bias = d["x"].cuda(), d["w"].cuda(), d["bias"].cuda()
        y = api.fuse_gemm_bias_act_auto(x, w, bias, act) if auto else api.fuse_gemm_bias_act(x, w, bias, act)
        assert_close(y[rows.cuda()], oracle.gemm_bias_act(d["x"][rows], d["w"], d["bias"], act), "bf16",
                     f"gemm {M}x{N}x{K} {act} auto={auto}")
    else:
        d = synth.swiglu_inputs(M, N, K, "bf16", seed=M + 3 * N + 5 * K)
        a, b1, b2 = d["a"].cuda(), d["b1"].cuda(), d["b2"].cuda()
        out = api.fuse_swiglu_auto(a, b1, b2) if auto else api.fuse_swiglu_dualgemm(a, b1, b2)
        assert_close(out[rows.cuda()], oracle.swiglu(d["a"][rows], d["b1"], d["b2"]), "bf16",
                     f"swiglu {M}x{N}x{K} auto={auto}")
