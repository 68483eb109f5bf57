"""Parity of the HIP kernels with the CPU oracle, through the C ABI (GPU required).

Small and medium shapes are compared element by element on every output; the full workload
shapes run in the launch configuration the benchmark times and are compared on every output
where the oracle is fast (Add+LayerNorm, GELU chain) and on a seeded sample of whole rows
otherwise (softmax, SwiGLU), plus properties that hold for every row.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from memory_bound_amd import api, synth
from oracle.tolerance import assert_close, compare

pytestmark = pytest.mark.gpu

KIND = {"f32": "f32", "f16": "f16", "bf16": "bf16"}


def cuda(d):
    return {k: (v.to("cuda") if torch.is_tensor(v) else v) for k, v in d.items()}


def announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


def stratified_rows(n, group, per_group, seed):
    """Seeded sample of whole rows: per_group distinct rows out of every block of `group`
    consecutive rows (all of a short last block), sorted."""
    rng = np.random.default_rng(seed)
    picks = []
    for g0 in range(0, n, group):
        size = min(group, n - g0)
        picks.append(g0 + np.sort(rng.choice(size, min(per_group, size), replace=False)))
    return np.concatenate(picks)


# ------------------------------------------------------------------------------------------------
# ResidualAdd + LayerNorm
# ------------------------------------------------------------------------------------------------

LN_SHAPES = [
    (64, 768, "f32"),      # small fp32 workload
    (37, 4096, "f16"),     # odd row count: last workgroup partly empty
    (130, 4096, "bf16"),
    (5, 1000, "f16"),      # row not a whole number of 16-byte words: per-element path
    (3, 7, "f32"),
    (2, 1, "f16"),         # one-element rows: output is beta
    (4, 8, "f16"),         # one chunk per row
    (7, 16384, "f16"),     # longest row
    (6, 16384, "f32"),
    (9, 8192, "bf16"),
    (11, 12288, "f16"),    # 3 x 4096: the last chunk group of each lane partly outside the row
    (3, 4097, "f32"),      # per-element path with several waves per row
    (33, 2048, "f32"),
]


@pytest.mark.parametrize("rows,hidden,dtype", LN_SHAPES)
def test_add_layernorm_parity(rows, hidden, dtype):
    announce(f"add_layernorm {rows}x{hidden} {dtype}")
    d = synth.add_layernorm_inputs(rows, hidden, dtype, seed=rows * 131 + hidden)
    g = cuda(d)
    y = api.fuse_add_layernorm(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"])
    ref = oracle.add_layernorm(d["x"], d["residual"], d["gamma"], d["beta"], np.float32(d["eps"]))
    assert_close(y, ref, KIND[dtype], f"add_layernorm {rows}x{hidden} {dtype}")


@pytest.mark.parametrize("name", ["addln_f32_64x768", "addln_f16_2048x4096", "addln_f16_16384x4096"])
def test_add_layernorm_workloads_full(name):
    w = synth.WORKLOADS[name]
    announce(f"add_layernorm workload {name}")
    d = w.inputs()
    g = cuda(d)
    y = api.fuse_add_layernorm(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"])
    ref = oracle.add_layernorm(d["x"], d["residual"], d["gamma"], d["beta"], np.float32(d["eps"]))
    r = assert_close(y, ref, KIND[w.dtype], name)
    print(f"  max_abs={r['max_abs']:.3e}", flush=True)


def test_add_layernorm_no_residual_and_inplace():
    announce("add_layernorm residual=None and in-place")
    d = synth.add_layernorm_inputs(64, 4096, "f16", seed=5)
    g = cuda(d)
    y = api.fuse_add_layernorm(g["x"], None, g["gamma"], g["beta"], d["eps"])
    assert_close(y, oracle.add_layernorm(d["x"], None, d["gamma"], d["beta"], np.float32(d["eps"])), "f16", "no residual")
    x = g["x"].clone()
    api.fuse_add_layernorm(x, g["residual"], g["gamma"], g["beta"], d["eps"], y=x)  # y == x
    ref = oracle.add_layernorm(d["x"], d["residual"], d["gamma"], d["beta"], np.float32(d["eps"]))
    assert_close(x, ref, "f16", "in place over x")
    r = g["residual"].clone()
    api.fuse_add_layernorm(g["x"], r, g["gamma"], g["beta"], d["eps"], y=r)  # y == residual
    assert_close(r, ref, "f16", "in place over residual")


def test_add_layernorm_misaligned_pointers():
    announce("add_layernorm misaligned views")
    rows, hidden = 6, 4096
    d = synth.add_layernorm_inputs(rows, hidden, "f16", seed=6)
    # views that start one element into a larger buffer: not 16-byte aligned
    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
        v = buf[1:].view(t.shape)
        v.copy_(t.to("cuda"))
        return v
    x, r, gm, bt = shifted(d["x"]), shifted(d["residual"]), shifted(d["gamma"]), shifted(d["beta"])
    y = shifted(torch.zeros(rows, hidden, dtype=torch.float16))
    api.fuse_add_layernorm(x, r, gm, bt, d["eps"], y=y)
    ref = oracle.add_layernorm(d["x"], d["residual"], d["gamma"], d["beta"], np.float32(d["eps"]))
    assert_close(y, ref, "f16", "misaligned")


# LayerNorm variants: ReLU epilogue, pre-norm sum, per-row mean and variance

_FROM_D = object()


def _check_ln_ex(outs, d, relu, kind, what, residual=_FROM_D):
    y, sm, mean, var = outs
    x = d["x"]
    residual = d["residual"] if residual is _FROM_D else residual
    ry, rs, rm, rv = oracle.add_layernorm_ex(x, residual, d["gamma"], d["beta"], np.float32(d["eps"]), relu)
    assert_close(y, ry, kind, f"{what} y")
    if sm is not None:
        # x + r is exact in fp32 for fp16/bf16 inputs and correctly rounded for fp32 ones, so
        # the stored sum is the round-to-nearest-even of the exact sum: bit-exact
        exp = oracle.round_to(rs, kind)
        got = sm.float().cpu().numpy().astype(np.float64)
        assert np.array_equal(got, exp), f"{what} sum: max diff {np.nanmax(np.abs(got - exp))}"
    if mean is not None:
        # fp32 tree sums of H terms: allow 1e-5 of the mean magnitude, 2e-5 of the variance
        absmean = np.abs(oracle.f64(x) + (oracle.f64(residual) if residual is not None else 0)).mean(axis=1)
        gm, gv = mean.cpu().numpy().astype(np.float64), var.cpu().numpy().astype(np.float64)
        assert (np.abs(gm - rm) <= 1e-5 * absmean + 1e-30).all(), f"{what} mean: {np.abs(gm - rm).max()}"
        assert (np.abs(gv - rv) <= 2e-5 * rv + 1e-30).all(), f"{what} var: {(np.abs(gv - rv) / rv).max()}"


@pytest.mark.parametrize("rows,hidden,dtype", [s for s in LN_SHAPES if s[1] != 1])
@pytest.mark.parametrize("relu", [False, True])
def test_add_layernorm_ex_parity(rows, hidden, dtype, relu):
    announce(f"add_layernorm_ex {rows}x{hidden} {dtype} relu={relu}")
    d = synth.add_layernorm_inputs(rows, hidden, dtype, seed=rows * 17 + hidden)
    g = cuda(d)
    outs = api.fuse_add_layernorm_ex(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"], relu=relu,
                                     want_sum=True, want_stats=True)
    _check_ln_ex(outs, d, relu, KIND[dtype], f"ln_ex {rows}x{hidden} {dtype} relu={relu}")


def test_add_layernorm_ex_workload_full(monkeypatch):
    w = synth.WORKLOADS["addln_f16_2048x4096"]
    announce("add_layernorm_ex workload 2048x4096 fp16, relu and every output")
    d = w.inputs()
    g = cuda(d)
    outs = api.fuse_add_layernorm_ex(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"], relu=True,
                                     want_sum=True, want_stats=True)
    _check_ln_ex(outs, d, True, "f16", "ln_ex workload")
    # under one launch plan (the plain kernel's 4 waves per row, and the 8 a call storing the sum
    # takes by default): the same y as the plain fused kernel before the clamp, the same
    # statistics with or without the sum, and only the requested outputs
    for wpr in ("4", "8"):
        monkeypatch.setenv("FUSE_ROW_WPR", wpr)
        full = api.fuse_add_layernorm_ex(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"], relu=True,
                                         want_sum=True, want_stats=True)
        y0 = api.fuse_add_layernorm(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"])
        assert torch.equal(full[0], torch.where(y0 < 0, torch.zeros_like(y0), y0)), wpr
        assert torch.equal(full[1], outs[1]), wpr  # the sum is exact whatever the plan
        y1, s1, m1, v1 = api.fuse_add_layernorm_ex(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"])
        assert torch.equal(y1, y0) and s1 is None and m1 is None and v1 is None, wpr
        _, s2, m2, v2 = api.fuse_add_layernorm_ex(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"],
                                                  want_stats=True)
        assert s2 is None and torch.equal(m2, full[2]) and torch.equal(v2, full[3]), wpr


def test_add_layernorm_ex_inplace_sum_and_nan():
    announce("add_layernorm_ex sum_out over x, NaN row, no residual")
    d = synth.add_layernorm_inputs(24, 1024, "bf16", seed=41)
    d["x"][5, 100] = float("nan")
    g = cuda(d)
    x = g["x"].clone()
    y, sm, mean, var = api.fuse_add_layernorm_ex(x, g["residual"], g["gamma"], g["beta"], d["eps"], relu=True,
                                                 sum_out=x, want_stats=True)
    assert sm is x
    ok = [i for i in range(24) if i != 5]
    dd = {k: (v[ok] if torch.is_tensor(v) and v.dim() == 2 else v) for k, v in d.items()}
    _check_ln_ex((y[ok], sm[ok], mean[ok], var[ok]), dd, True, "bf16", "ln_ex in place")
    assert torch.isnan(y[5].float()).all() and torch.isnan(mean[5]) and torch.isnan(var[5])
    outs = api.fuse_add_layernorm_ex(g["x"][ok].contiguous(), None, g["gamma"], g["beta"], d["eps"],
                                     want_sum=True, want_stats=True)
    _check_ln_ex(outs, dd, False, "bf16", "ln_ex no residual", residual=None)


@pytest.mark.parametrize("rows,hidden,dtype", [(2048, 4096, "f16"), (2047, 4096, "f16"), (1000, 1024, "bf16"),
                                               (4096, 2048, "f16"), (513, 1024, "f32"), (3, 4096, "bf16"),
                                               (130, 4000, "f16"), (777, 256, "f16")])
def test_add_layernorm_steps_bit_identical(monkeypatch, rows, hidden, dtype):
    # workgroups that walk 1, 2 or 4 row blocks with the next block's loads in flight run the same
    # arithmetic per row: every output of every LayerNorm entry point must be bit-identical, for
    # ragged row counts (steps past the last row); rows that leave chunks of the slice empty
    # (H = 4000, 256) always take one step, whatever the override
    announce(f"add_layernorm steps 1/2/4 {rows}x{hidden} {dtype}")
    d = synth.add_layernorm_inputs(rows, hidden, dtype, seed=47 + rows)
    g = cuda(d)
    outs = {}
    for st in ("1", "2", "4"):
        monkeypatch.setenv("FUSE_ROW_STEPS", st)
        y = api.fuse_add_layernorm(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"])
        yn = api.fuse_add_layernorm(g["x"], None, g["gamma"], g["beta"], d["eps"])
        ex = api.fuse_add_layernorm_ex(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"], relu=True,
                                       want_sum=True, want_stats=True)
        outs[st] = (y, yn) + tuple(ex)
    for st in ("2", "4"):
        for a, b in zip(outs["1"], outs[st]):
            assert torch.equal(a, b), f"steps {st}"
    monkeypatch.delenv("FUSE_ROW_STEPS")
    y = api.fuse_add_layernorm(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"])
    assert torch.equal(y, outs["1"][0])
    assert_close(y, oracle.add_layernorm(d["x"], d["residual"], d["gamma"], d["beta"], d["eps"]), dtype,
                 f"steps default {rows}x{hidden}")


@pytest.mark.parametrize("steps", ["1", "2", "4"])
def test_add_layernorm_steps_in_place(monkeypatch, steps):
    # y over x, y over the residual, and the ReLU variant's pre-norm sum over x, on the workload
    # shape where several row blocks per workgroup are in flight: bit-identical to out of place
    monkeypatch.setenv("FUSE_ROW_STEPS", steps)
    announce(f"add_layernorm in place, steps {steps}")
    d = synth.add_layernorm_inputs(2048, 4096, "f16", seed=53)
    g = cuda(d)
    y = api.fuse_add_layernorm(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"])
    x = g["x"].clone()
    assert api.fuse_add_layernorm(x, g["residual"], g["gamma"], g["beta"], d["eps"], y=x) is x
    assert torch.equal(x, y)
    r = g["residual"].clone()
    api.fuse_add_layernorm(g["x"], r, g["gamma"], g["beta"], d["eps"], y=r)
    assert torch.equal(r, y)
    ref = api.fuse_add_layernorm_ex(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"], relu=True, want_sum=True)
    x = g["x"].clone()
    got = api.fuse_add_layernorm_ex(x, g["residual"], g["gamma"], g["beta"], d["eps"], relu=True, sum_out=x)
    assert got[1] is x
    assert torch.equal(got[0], ref[0]) and torch.equal(x, ref[1])


def test_add_layernorm_relu_f16_tiny_negatives_become_plus_zero():
    # gamma at the smallest f16 subnormal and beta 0: every output lies within one subnormal of
    # zero, and the negative ones round to -0 or -2^-24 before the clamp.  The clamp must store
    # +0 for all of them (the oracle clamps first, then rounds), never the bit pattern of -0.
    announce("add_layernorm_ex relu f16 tiny negatives")
    d = synth.add_layernorm_inputs(16, 2048, "f16", seed=43)
    d["gamma"] = torch.full((2048,), 2.0 ** -24, dtype=torch.float16)
    d["beta"] = torch.zeros(2048, dtype=torch.float16)
    g = cuda(d)
    y = api.fuse_add_layernorm_ex(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"], relu=True)[0].cpu()
    bits = y.view(torch.int16)
    assert not (bits == -32768).any(), "a -0 was stored"
    assert (y.float() >= 0).all()
    ref = oracle.add_layernorm_ex(d["x"], d["residual"], d["gamma"], d["beta"], d["eps"], relu=True)[0]
    assert_close(y, ref, "f16", "relu tiny")


def test_add_layernorm_large_mean_rows():
    # mean 1e4, spread 1: the statistics must not lose the variance to cancellation
    announce("add_layernorm mean 1e4 fp32")
    gen = torch.Generator().manual_seed(7)
    x = (1e4 + torch.randn(16, 4096, generator=gen)).float()
    r = torch.randn(16, 4096, generator=gen).float()
    gm = torch.ones(4096)
    bt = torch.zeros(4096)
    y = api.fuse_add_layernorm(x.cuda(), r.cuda(), gm.cuda(), bt.cuda(), 1e-5)
    ref = oracle.add_layernorm(x, r, gm, bt, np.float32(1e-5))
    # fp32 inputs near 1e4 carry 1e-3 absolute quantum; the bound below is the fp32 rule scaled
    # by the row's condition number (mean / std ~ 1e4)
    err = np.abs(y.cpu().double().numpy() - ref).max()
    assert err < 2e-3, err


def test_add_layernorm_constant_rows_give_beta():
    announce("add_layernorm constant rows")
    x = torch.full((8, 768), 3.0, dtype=torch.float16)
    r = torch.full((8, 768), -1.5, dtype=torch.float16)
    gm = torch.rand(768).half()
    bt = torch.randn(768).half()
    y = api.fuse_add_layernorm(x.cuda(), r.cuda(), gm.cuda(), bt.cuda(), 1e-5)
    assert torch.equal(y.cpu(), bt.expand(8, 768))


def test_add_layernorm_zero_rows_is_noop():
    x = torch.empty(0, 4096, dtype=torch.float16, device="cuda")
    g = torch.ones(4096, dtype=torch.float16, device="cuda")
    y = api.fuse_add_layernorm(x, x, g, g, 1e-5)
    assert y.shape == (0, 4096)


def test_add_layernorm_deterministic():
    announce("add_layernorm determinism")
    g = cuda(synth.add_layernorm_inputs(2048, 4096, "f16", seed=9))
    y1 = api.fuse_add_layernorm(g["x"], g["residual"], g["gamma"], g["beta"], 1e-5)
    y2 = api.fuse_add_layernorm(g["x"], g["residual"], g["gamma"], g["beta"], 1e-5)
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("wpr", [1, 2, 4, 8])
def test_add_layernorm_every_waves_per_row(monkeypatch, wpr):
    # the tuning override picks other compiled launch shapes; all must agree with the oracle
    announce(f"add_layernorm FUSE_ROW_WPR={wpr}")
    monkeypatch.setenv("FUSE_ROW_WPR", str(wpr))
    d = synth.add_layernorm_inputs(67, 4096, "f16", seed=10 + wpr)
    g = cuda(d)
    y = api.fuse_add_layernorm(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"])
    ref = oracle.add_layernorm(d["x"], d["residual"], d["gamma"], d["beta"], np.float32(d["eps"]))
    assert_close(y, ref, "f16", f"wpr={wpr}")


# ------------------------------------------------------------------------------------------------
# BiasAdd + GELU + Residual
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("rows,hidden,dtype", [
    (2048, 4096, "f16"),   # the full workload
    (33, 768, "f32"),
    (17, 4096, "bf16"),
    (5, 1001, "f16"),      # per-element path
    (1, 3, "f32"),
    (300, 520, "f16"),     # chunk count not a multiple of the workgroup's
])
def test_bias_gelu_residual_parity(rows, hidden, dtype):
    announce(f"bias_gelu_residual {rows}x{hidden} {dtype}")
    d = synth.bias_gelu_residual_inputs(rows, hidden, dtype, seed=1002 if rows == 2048 else rows + hidden)
    g = cuda(d)
    y = api.fuse_bias_gelu_residual(g["x"], g["bias"], g["residual"])
    ref = oracle.bias_gelu_residual(d["x"], d["bias"], d["residual"])
    assert_close(y, ref, KIND[dtype], f"gelu {rows}x{hidden} {dtype}")


def test_gelu_exhaustive_fp16_domain():
    # every finite fp16 value t as x with bias 0 and residual 0: the kernel's GELU before the
    # output rounding is held to the 1e-4 relative rule for approximate math; after rounding to
    # fp32 output the comparison is direct
    announce("gelu exhaustive fp16")
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    t = bits.view(torch.float16)
    t = t[torch.isfinite(t)].float()
    n = t.numel()
    hidden = 64
    rows = (n + hidden - 1) // hidden
    x = torch.zeros(rows * hidden)
    x[:n] = t
    x = x.view(rows, hidden)
    zb = torch.zeros(hidden)
    zr = torch.zeros(rows, hidden)
    y = api.fuse_bias_gelu_residual(x.cuda(), zb.cuda(), zr.cuda()).cpu().double().numpy().ravel()[:n]
    ref = oracle.bias_gelu_residual(x, zb, zr).ravel()[:n]
    rel = np.abs(y - ref) / np.maximum(np.abs(ref), 1e-30)
    small = np.abs(ref) < 1e-30  # GELU underflows: require an absolute 1e-30
    assert np.all(np.abs(y - ref)[small] < 1e-30)
    assert rel[~small].max() < 1e-4, rel[~small].max()


def test_bias_gelu_residual_inplace_and_deterministic():
    announce("gelu in place")
    d = synth.bias_gelu_residual_inputs(64, 4096, "f16", seed=3)
    g = cuda(d)
    ref = oracle.bias_gelu_residual(d["x"], d["bias"], d["residual"])
    y1 = api.fuse_bias_gelu_residual(g["x"], g["bias"], g["residual"])
    y2 = api.fuse_bias_gelu_residual(g["x"], g["bias"], g["residual"])
    assert torch.equal(y1, y2)
    x = g["x"].clone()
    api.fuse_bias_gelu_residual(x, g["bias"], g["residual"], y=x)
    assert_close(x, ref, "f16", "gelu in place")


# ------------------------------------------------------------------------------------------------
# Row softmax
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("rows,cols,dtype,scale", [
    (256, 2048, "f16", 1 / math.sqrt(128)),
    (37, 2048, "bf16", 1 / math.sqrt(128)),
    (19, 768, "f32", 0.5),
    (8, 16384, "f16", 1 / math.sqrt(128)),   # longest row
    (5, 1000, "f16", 1.0),                   # per-element path
    (3, 1, "f16", 1.0),                      # one column: exactly 1
    (6, 333, "f32", -0.7),                   # negative scale
    (12, 4096, "f16", 1 / math.sqrt(128)),
    (64, 2048, "f16", -1 / math.sqrt(128)),  # negative scale on full rows (max of -x)
    (33, 1024, "bf16", -0.3),
    (16, 2048, "f16", 0.0),                  # scale 0: every row uniform, 1/cols
    (7, 4000, "f16", -0.25),                 # 128-bit path, chunks past the row, negative scale
])
def test_softmax_parity(rows, cols, dtype, scale):
    announce(f"softmax {rows}x{cols} {dtype} scale={scale}")
    d = synth.softmax_inputs(rows, cols, dtype, seed=rows * 7 + cols)
    y = api.fuse_softmax_rows(d["x"].cuda(), scale)
    ref = oracle.softmax_rows(d["x"], np.float32(scale))
    assert_close(y, ref, KIND[dtype], f"softmax {rows}x{cols}")


def test_softmax_workload_all_rows():
    w = synth.WORKLOADS["softmax_f16_65536x2048"]
    announce("softmax workload 65536x2048, every row")
    d = w.inputs()
    y = api.fuse_softmax_rows(d["x"].cuda(), d["scale"])
    # every row: sum of the stored fp16 outputs within 2e-3 of one (emulated error ~3e-5)
    sums = y.float().sum(dim=1)
    assert (sums - 1).abs().max().item() < 2e-3
    y = y.cpu()
    step = 8192  # element-wise against the oracle, all 65536 rows, in blocks to bound host memory
    for r0 in range(0, w.shape[0], step):
        ref = oracle.softmax_rows(d["x"][r0:r0 + step], np.float32(d["scale"]))
        assert_close(y[r0:r0 + step], ref, "f16", f"softmax rows {r0}..{r0 + step - 1}")


def test_softmax_constant_rows_and_inplace():
    announce("softmax constant rows")
    x = torch.full((4, 2048), 2.5, dtype=torch.float16, device="cuda")
    y = api.fuse_softmax_rows(x, 0.3)
    assert torch.all(y == 2.0 ** -11)
    d = synth.softmax_inputs(64, 2048, "f16", seed=4)
    ref = oracle.softmax_rows(d["x"], np.float32(d["scale"]))
    x = d["x"].cuda()
    api.fuse_softmax_rows(x, d["scale"], y=x)
    assert_close(x, ref, "f16", "softmax in place")


@pytest.mark.parametrize("dtype,cols", [("f16", 2048), ("f32", 1000), ("bf16", 4096), ("f16", 333)])
def test_softmax_masked_rows(dtype, cols):
    # causal-style masks: row r keeps its first r * cols / rows + 1 entries and the rest are -inf;
    # masked entries come out exactly 0 and the kept ones match the oracle
    rows = 48
    announce(f"softmax masked rows {rows}x{cols} {dtype}")
    d = synth.softmax_inputs(rows, cols, dtype, seed=cols + 5)
    x = d["x"].clone()
    mask = torch.zeros(rows, cols, dtype=torch.bool)
    for r in range(rows):
        mask[r, (r * cols) // rows + 1:] = True
    x[mask] = float("-inf")
    y = api.fuse_softmax_rows(x.cuda(), d["scale"])
    assert_close(y, oracle.softmax_rows(x, np.float32(d["scale"])), KIND[dtype], f"masked softmax {dtype}")
    assert bool((y.cpu()[mask] == 0).all())


def test_softmax_nan_propagates():
    x = torch.randn(2, 2048).half()
    x[1, 100] = float("nan")
    y = api.fuse_softmax_rows(x.cuda(), 1.0).cpu()
    assert torch.isfinite(y[0]).all()
    assert torch.isnan(y[1]).all()


# ------------------------------------------------------------------------------------------------
# Row cumsum + scale
# ------------------------------------------------------------------------------------------------

CUMSUM_SHAPES = [
    (37, 4096, "f16"), (64, 768, "f32"), (130, 4096, "bf16"), (5, 1000, "f16"), (3, 7, "f32"),
    (2, 1, "f16"), (4, 8, "f16"), (9, 64, "f32"), (7, 16384, "f16"), (6, 16384, "f32"), (9, 8192, "bf16"),
    (11, 12288, "f16"), (3, 4097, "f32"), (33, 2048, "f32"), (17, 520, "bf16"),
]


@pytest.mark.parametrize("rows,cols,dtype", CUMSUM_SHAPES)
def test_cumsum_parity(rows, cols, dtype):
    announce(f"cumsum_scale {rows}x{cols} {dtype}")
    d = synth.cumsum_inputs(rows, cols, dtype, seed=rows * 7 + cols)
    y = api.fuse_cumsum_scale_rows(d["x"].cuda(), d["scale"])
    assert_close(y, oracle.cumsum_scale_rows(d["x"], np.float32(d["scale"])), KIND[dtype],
                 f"cumsum {rows}x{cols} {dtype}")


@pytest.mark.parametrize("wpr", [1, 2, 4, 8])
def test_cumsum_exact_counts_every_wpr(monkeypatch, wpr):
    # integer inputs make every partial sum exact in fp32, so any misplaced carry between chunks,
    # lanes, DPP rows or waves shows up as an exact mismatch
    monkeypatch.setenv("FUSE_ROW_WPR", str(wpr))
    announce(f"cumsum exact counts FUSE_ROW_WPR={wpr}")
    for cols in (4096, 2048, 1000):
        x = torch.ones(6, cols, dtype=torch.float32)
        x[1] = torch.arange(cols) % 5 - 2.0
        x[2] = -1.0
        x[3, ::64] = 7.0
        y = api.fuse_cumsum_scale_rows(x.cuda(), 1.0).cpu()
        assert torch.equal(y, torch.cumsum(x.double(), dim=1).float()), f"cols={cols} wpr={wpr}"


@pytest.mark.parametrize("rows,cols,dtype", [(2048, 4096, "f16"), (2047, 4096, "f16"), (4096, 2048, "bf16"),
                                             (1000, 1024, "f32"), (3, 4096, "f16"), (130, 4000, "f16")])
def test_cumsum_steps_bit_identical(monkeypatch, rows, cols, dtype):
    # workgroups that walk 1, 2 or 4 row blocks (the next block's loads in flight, block totals in
    # LDS alternating by step parity) run the same arithmetic per row: bit-identical outputs for
    # ragged row counts (steps past the last row) and in place; rows that leave chunks of the
    # slice empty (4000 columns) take one step whatever the override.  Integer-valued rows make
    # every partial sum exact, so a carry taken from the wrong step's totals is an exact mismatch.
    announce(f"cumsum steps 1/2/4 {rows}x{cols} {dtype}")
    d = synth.cumsum_inputs(rows, cols, dtype, seed=61 + rows)
    x = d["x"].cuda()
    ints = ((torch.arange(rows * cols) * 7 % 9) - 4.0).reshape(rows, cols)
    ints[rows // 2] = 1.0
    exact = torch.cumsum(ints.double(), dim=1).to(x.dtype)
    ints = ints.to(x.dtype).cuda()
    outs = {}
    for st in ("1", "2", "4"):
        monkeypatch.setenv("FUSE_ROW_STEPS", st)
        outs[st] = api.fuse_cumsum_scale_rows(x, d["scale"])
        xi = x.clone()
        assert api.fuse_cumsum_scale_rows(xi, d["scale"], y=xi) is xi
        assert torch.equal(xi, outs[st]), f"in place, steps {st}"
        assert torch.equal(api.fuse_cumsum_scale_rows(ints, 1.0).cpu(), exact), f"exact carries, steps {st}"
    for st in ("2", "4"):
        assert torch.equal(outs["1"], outs[st]), f"steps {st}"
    monkeypatch.delenv("FUSE_ROW_STEPS")
    y = api.fuse_cumsum_scale_rows(x, d["scale"])
    assert torch.equal(y, outs["1"])
    assert_close(y, oracle.cumsum_scale_rows(d["x"], np.float32(d["scale"])), KIND[dtype],
                 f"cumsum steps default {rows}x{cols} {dtype}")


def test_cumsum_workload_full_and_inplace():
    w = synth.WORKLOADS["cumsum_f16_2048x4096"]
    announce("cumsum workload 2048x4096 fp16")
    d = w.inputs()
    ref = oracle.cumsum_scale_rows(d["x"], np.float32(d["scale"]))
    x = d["x"].cuda()
    y = api.fuse_cumsum_scale_rows(x, d["scale"])
    r = assert_close(y, ref, "f16", "cumsum workload")
    print(f"  max_abs={r['max_abs']:.3e}", flush=True)
    y2 = api.fuse_cumsum_scale_rows(x, d["scale"], y=x)  # in place
    assert torch.equal(y2, y)
    yn = api.fuse_cumsum_scale_rows(d["x"].cuda(), -2.0)
    assert_close(yn, oracle.cumsum_scale_rows(d["x"], -2.0), "f16", "cumsum scale -2")


# ------------------------------------------------------------------------------------------------
# SwiGLU dual GEMM
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [
    (128, 128, 64),     # one tile, one K step
    (256, 384, 192),    # several tiles and K steps
    (130, 200, 136),    # ragged M, N, K (aligned rows: K, N multiples of 8)
    (100, 72, 70),      # K not a multiple of 8: per-element loads
    (1, 8, 16),
    (64, 1000, 1536),   # the workload's K with a ragged N tile
])
def test_swiglu_parity(M, N, K):
    announce(f"swiglu {M}x{N}x{K}")
    d = synth.swiglu_inputs(M, N, K, "bf16", seed=M + N + K)
    out = api.fuse_swiglu_dualgemm(d["a"].cuda(), d["b1"].cuda(), d["b2"].cuda())
    ref = oracle.swiglu(d["a"], d["b1"], d["b2"])
    r = assert_close(out, ref, "bf16", f"swiglu {M}x{N}x{K}")
    print(f"  max_abs={r['max_abs']:.3e}", flush=True)


@pytest.mark.parametrize("env", [{"FUSE_SWIGLU_STAGES": "3"}, {"FUSE_SWIGLU_STAGES": "4"},
                                 {"FUSE_SWIGLU_STAGES": "5"}, {"FUSE_SWIGLU_GENERAL": "1"}])
def test_swiglu_full_tile_paths(monkeypatch, env):
    # full tiles (N = 384, 640) take the direct-to-LDS kernel with a ring of 3 to 5 stages unless
    # the general kernel is forced; N = 480 is not a multiple of the tile width and takes the
    # general kernel
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    announce(f"swiglu full-tile path {env}")
    for N in (384, 480, 640):
        for K in (320, 64, 32, 96):  # several steps, and rings longer than the K loop
            d = synth.swiglu_inputs(512, N, K, "bf16", seed=21 + K + N)
            out = api.fuse_swiglu_dualgemm(d["a"].cuda(), d["b1"].cuda(), d["b2"].cuda())
            assert_close(out, oracle.swiglu(d["a"], d["b1"], d["b2"]), "bf16", f"swiglu N={N} K={K} {env}")


def test_swiglu_full_tile_stores_match_general_kernel(monkeypatch):
    # the full-tile kernel stores each 4 x 4 quad of lanes as four 8-byte rows, the general kernel
    # one element per lane; both sum the same 16-deep k slices in ascending order, so every output
    # (SwiGLU, and GEMM + bias + activation) must be bit-identical, and a value stored at the
    # wrong row or column cannot hide
    announce("swiglu full-tile quad stores vs general kernel")
    for M, N, K in ((512, 384, 320), (256, 640, 96), (512, 8960 // 35 * 3, 1536)):
        d = synth.swiglu_inputs(M, N, K, "bf16", seed=5 + N)
        a, b1, b2 = d["a"].cuda(), d["b1"].cuda(), d["b2"].cuda()
        direct = api.fuse_swiglu_dualgemm(a, b1, b2)
        monkeypatch.setenv("FUSE_SWIGLU_GENERAL", "1")
        general = api.fuse_swiglu_dualgemm(a, b1, b2)
        monkeypatch.delenv("FUSE_SWIGLU_GENERAL")
        assert torch.equal(direct, general), f"{M}x{N}x{K}"
    # the GEMM epilogue (bias, activation) on the same two kernels
    d = synth.gemm_inputs(512, 768, 320, "bf16", seed=7)
    x, w, bias = d["x"].cuda(), d["w"].cuda(), d["bias"].cuda()
    for act in ("none", "relu", "gelu", "silu"):
        direct = api.fuse_gemm_bias_act(x, w, bias, act)
        monkeypatch.setenv("FUSE_SWIGLU_GENERAL", "1")
        general = api.fuse_gemm_bias_act(x, w, bias, act)
        monkeypatch.delenv("FUSE_SWIGLU_GENERAL")
        assert torch.equal(direct, general), f"gemm {act}"


def test_swiglu_last_round_slices(monkeypatch):
    # 5 x 53 = 265 tiles on 256 CUs: the last 9 tiles run as 64-row quarters by default, as 128-row
    # halves with FUSE_SWIGLU_TAIL=2, whole with =0.  Same k order per element every way, so the
    # results are bit-identical; checked against the oracle on every fourth row.
    M, N, K = 1280, 6784, 256
    announce(f"swiglu {M}x{N}x{K} last-round slices")
    d = synth.swiglu_inputs(M, N, K, "bf16", seed=29)
    a, b1, b2 = d["a"].cuda(), d["b1"].cuda(), d["b2"].cuda()
    out = api.fuse_swiglu_dualgemm(a, b1, b2)
    rows = torch.arange(0, M, 4)
    assert_close(out[rows.cuda()], oracle.swiglu(d["a"][rows], d["b1"], d["b2"]), "bf16", "quarters")
    for tail in ("2", "0"):
        monkeypatch.setenv("FUSE_SWIGLU_TAIL", tail)
        assert torch.equal(out, api.fuse_swiglu_dualgemm(a, b1, b2)), f"tail {tail}"
    d = synth.gemm_inputs(M, 2 * N, K, "bf16", seed=30)  # the same tile grid for the GEMM
    x, w, bias = d["x"].cuda(), d["w"].cuda(), d["bias"].cuda()
    y0 = api.fuse_gemm_bias_act(x, w, bias, "gelu")
    monkeypatch.setenv("FUSE_SWIGLU_TAIL", "2")
    assert torch.equal(y0, api.fuse_gemm_bias_act(x, w, bias, "gelu")), "gemm halves"
    monkeypatch.delenv("FUSE_SWIGLU_TAIL")
    y1 = api.fuse_gemm_bias_act(x, w, bias, "gelu")
    assert torch.equal(y0, y1), "gemm quarters"
    assert_close(y1[rows.cuda()], oracle.gemm_bias_act(d["x"][rows], d["w"], d["bias"], "gelu"), "bf16", "gemm quarters")


@pytest.mark.parametrize("M,N", [(2048, 8960), (2048, 5248)])
def test_swiglu_tail_slices_at_full_grids(monkeypatch, M, N):
    # 560 tiles on 256 CUs leave 48 for a last round run as 64-row quarters (the workload's tile
    # grid), 328 tiles leave 72 run as 128-row halves; by default one resident workgroup per CU
    # walks its units.  The k order per element is the same every way: bit-identical to whole
    # tiles, to halves and to one workgroup per unit, and checked against the oracle on sampled
    # rows.
    K = 256
    announce(f"swiglu {M}x{N}x{K} tail slices")
    d = synth.swiglu_inputs(M, N, K, "bf16", seed=N)
    a, b1, b2 = d["a"].cuda(), d["b1"].cuda(), d["b2"].cuda()
    out = api.fuse_swiglu_dualgemm(a, b1, b2)
    for tail in ("2", "0"):
        monkeypatch.setenv("FUSE_SWIGLU_TAIL", tail)
        assert torch.equal(out, api.fuse_swiglu_dualgemm(a, b1, b2)), f"tail {tail}"
    monkeypatch.delenv("FUSE_SWIGLU_TAIL")
    # one workgroup per unit instead of one resident workgroup per CU walking its units
    monkeypatch.setenv("FUSE_SWIGLU_PERSIST", "0")
    assert torch.equal(out, api.fuse_swiglu_dualgemm(a, b1, b2)), "one workgroup per unit"
    monkeypatch.delenv("FUSE_SWIGLU_PERSIST")
    rows = torch.arange(3, M, 29)
    assert_close(out[rows.cuda()], oracle.swiglu(d["a"][rows], d["b1"], d["b2"]), "bf16", f"swiglu {M}x{N} tail")


@pytest.mark.parametrize("stages", [None, "3", "5"])
def test_swiglu_workload_sampled_rows(monkeypatch, stages):
    # the default ring depth and the shallowest and deepest rings at the full size
    if stages:
        monkeypatch.setenv("FUSE_SWIGLU_STAGES", stages)
    w = synth.WORKLOADS["swiglu_bf16_2048x8960x1536"]
    announce(f"swiglu workload 2048x8960x1536 stages {stages or 'default'}")
    d = w.inputs()
    out = api.fuse_swiglu_dualgemm(d["a"].cuda(), d["b1"].cuda(), d["b2"].cuda()).cpu()
    # 8 seeded rows from each block of 64 (256 rows): every 64-row slice of every tile, whole
    # or cut into the last round's quarters, is compared on all of its columns
    rows = torch.from_numpy(stratified_rows(w.shape[0], 64, 8, 1006))
    assert len(rows) == 256
    print(f"  comparing {len(rows)} full rows", flush=True)
    ref = oracle.swiglu(d["a"][rows], d["b1"], d["b2"])
    r = assert_close(out[rows], ref, "bf16", "swiglu sampled rows")
    nw = float(np.abs(out[rows].double().numpy() - ref).max() / np.abs(ref).max())
    print(f"  max_abs={r['max_abs']:.3e} normwise={nw:.2e}", flush=True)
    assert nw < 5e-3
    out2 = api.fuse_swiglu_dualgemm(d["a"].cuda(), d["b1"].cuda(), d["b2"].cuda()).cpu()
    assert torch.equal(out, out2)


# ------------------------------------------------------------------------------------------------
# GEMM + bias + activation
# ------------------------------------------------------------------------------------------------

GEMM_SHAPES = [
    (256, 256, 64),     # one full 256 x 256 tile, two K steps
    (512, 768, 320),    # several full tiles (direct path)
    (300, 384, 96),     # ragged M; N not a multiple of 256: the second half of the last tile empty
    (130, 200, 136),    # ragged M, N, K
    (64, 100, 40),      # N below 128: the shifted second half has no columns at all
    (33, 136, 37),      # K not a multiple of 8: per-element loads
    (256, 512, 1536),   # long K
]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
@pytest.mark.parametrize("act", ["none", "relu", "gelu", "silu"])
def test_gemm_bias_act_parity(M, N, K, act):
    announce(f"gemm_bias_act {M}x{N}x{K} {act}")
    d = synth.gemm_inputs(M, N, K, "bf16", seed=M + N + K)
    y = api.fuse_gemm_bias_act(d["x"].cuda(), d["w"].cuda(), d["bias"].cuda(), act)
    assert_close(y, oracle.gemm_bias_act(d["x"], d["w"], d["bias"], act), "bf16", f"gemm {M}x{N}x{K} {act}")


def test_gemm_no_bias_and_stages(monkeypatch):
    announce("gemm without bias, every ring depth, general kernel forced")
    d = synth.gemm_inputs(512, 512, 160, "bf16", seed=3)
    ref = oracle.gemm_bias_act(d["x"], d["w"], None, "relu")
    x, w = d["x"].cuda(), d["w"].cuda()
    assert_close(api.fuse_gemm_bias_act(x, w, None, "relu"), ref, "bf16", "no bias")
    for env in ({"FUSE_SWIGLU_STAGES": "3"}, {"FUSE_SWIGLU_STAGES": "5"}, {"FUSE_SWIGLU_GENERAL": "1"}):
        with monkeypatch.context() as m:
            for k, v in env.items():
                m.setenv(k, v)
            assert_close(api.fuse_gemm_bias_act(x, w, None, "relu"), ref, "bf16", f"no bias {env}")


def test_gemm_workload_sampled_rows():
    w_ = synth.WORKLOADS["gemm_relu_bf16_2048x8960x1536"]
    announce("gemm + bias + relu workload 2048x8960x1536")
    d = w_.inputs()
    y = api.fuse_gemm_bias_act(d["x"].cuda(), d["w"].cuda(), d["bias"].cuda(), "relu").cpu()
    rows = torch.from_numpy(stratified_rows(w_.shape[0], 64, 8, 1008))  # 256 rows, every 64-row block
    assert len(rows) == 256
    print(f"  comparing {len(rows)} full rows", flush=True)
    ref = oracle.gemm_bias_act(d["x"][rows], d["w"], d["bias"], "relu")
    r = assert_close(y[rows], ref, "bf16", "gemm sampled rows")
    print(f"  max_abs={r['max_abs']:.3e}", flush=True)
    assert (y >= 0).all()
    y2 = api.fuse_gemm_bias_act(d["x"].cuda(), d["w"].cuda(), d["bias"].cuda(), "relu").cpu()
    assert torch.equal(y, y2)


@pytest.mark.parametrize("act", ["relu", "gelu"])
def test_gemm_tail_slices_at_full_grid(monkeypatch, act):
    # 2048x8960 in 256x256 tiles is 280 tiles: one round on 256 CUs and 24 tiles left, run as
    # 64-row quarters ahead of the whole tiles, the 352 units walked by one resident workgroup per
    # CU.  The k order per
    # element does not depend on how the tiles are cut or launched: bit-identical to whole tiles
    # and to one workgroup per unit, and checked against the oracle on sampled rows.
    M, N, K = 2048, 8960, 256
    announce(f"gemm_bias_act {M}x{N}x{K} {act} tail slices")
    d = synth.gemm_inputs(M, N, K, "bf16", seed=77)
    x, w, bias = d["x"].cuda(), d["w"].cuda(), d["bias"].cuda()
    y = api.fuse_gemm_bias_act(x, w, bias, act)
    for env in ({"FUSE_SWIGLU_TAIL": "0"}, {"FUSE_SWIGLU_PERSIST": "0"}):
        with monkeypatch.context() as m:
            for k, v in env.items():
                m.setenv(k, v)
            assert torch.equal(y, api.fuse_gemm_bias_act(x, w, bias, act)), f"{env}"
    rows = torch.arange(5, M, 31)
    assert_close(y[rows.cuda()], oracle.gemm_bias_act(d["x"][rows], d["w"], d["bias"], act), "bf16",
                 f"gemm {M}x{N}x{K} {act} tail")


# ------------------------------------------------------------------------------------------------
# Shape-dependent plans: split K for shapes whose tiles cannot fill the GPU
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,force", [
    (256, 512, 1536, None),   # 4 tiles: split by the plan
    (1024, 1024, 1536, None), # 32 tiles
    (512, 256, 320, None),    # short K: too few steps to pay for a reduction pass, not split
    (256, 512, 1536, "2"), (256, 512, 1536, "5"), (256, 512, 1536, "48"),  # uneven and one step per split
    (2048, 1024, 64, None),   # 64 tiles, two K steps: no split
    (1024, 2048, 2048, None), # 64 tiles, 64 K steps: split by the cost model (3 on 256 CUs)
    (2048, 1024, 4096, None), # 64 tiles, 128 K steps (4 on 256 CUs)
])
def test_swiglu_auto_parity(monkeypatch, M, N, K, force):
    if force:
        monkeypatch.setenv("FUSE_SPLITK", force)
    splits = api.fuse_auto_splits(api.FUSE_OP_SWIGLU, M, N, K)
    announce(f"swiglu auto {M}x{N}x{K} splits={splits}")
    d = synth.swiglu_inputs(M, N, K, "bf16", seed=M + 3 * N + K)
    a, b1, b2 = d["a"].cuda(), d["b1"].cuda(), d["b2"].cuda()
    out = api.fuse_swiglu_auto(a, b1, b2)
    rows = torch.arange(0, M, max(1, M // 64))
    assert_close(out[rows.cuda()], oracle.swiglu(d["a"][rows], d["b1"], d["b2"]), "bf16", f"auto {M}x{N}x{K} s={splits}")
    assert torch.equal(out, api.fuse_swiglu_auto(a, b1, b2))  # fixed summation order
    if force is None and M * N <= 256 * 512 and K >= 1536:
        assert splits > 1


@pytest.mark.parametrize("act", ["none", "relu", "gelu", "silu"])
def test_gemm_auto_parity(monkeypatch, act):
    for M, N, K, force in ((256, 512, 1536, None), (512, 768, 640, "3"), (256, 256, 64, "2")):
        with monkeypatch.context() as m:
            if force:
                m.setenv("FUSE_SPLITK", force)
            splits = api.fuse_auto_splits(api.FUSE_OP_GEMM_BIAS_ACT, M, N, K)
            announce(f"gemm auto {M}x{N}x{K} {act} splits={splits}")
            assert splits > 1
            d = synth.gemm_inputs(M, N, K, "bf16", seed=M + N + K + 1)
            y = api.fuse_gemm_bias_act_auto(d["x"].cuda(), d["w"].cuda(), d["bias"].cuda(), act)
            assert_close(y, oracle.gemm_bias_act(d["x"], d["w"], d["bias"], act), "bf16", f"gemm auto {M}x{N}x{K} {act}")
            y = api.fuse_gemm_bias_act_auto(d["x"].cuda(), d["w"].cuda(), None, act)
            assert_close(y, oracle.gemm_bias_act(d["x"], d["w"], None, act), "bf16", f"gemm auto no bias {act}")


@pytest.mark.parametrize("M,N,K,act", [(2048, 2048, 2048, "gelu"), (256, 8960, 1536, "silu")])
def test_gemm_auto_large_parity(M, N, K, act):
    """Larger shapes the cost model splits (3 splits each on 256 CUs: 64 tiles over a deep K, 35
    tiles of a wide N): sampled rows against the oracle, with and without bias, and the same bits
    on a second call."""
    splits = api.fuse_auto_splits(api.FUSE_OP_GEMM_BIAS_ACT, M, N, K)
    announce(f"gemm auto {M}x{N}x{K} {act} splits={splits}")
    d = synth.gemm_inputs(M, N, K, "bf16", seed=M + 7 * N + K)
    x, w, bias = d["x"].cuda(), d["w"].cuda(), d["bias"].cuda()
    rows = torch.arange(0, M, max(1, M // 48))
    for b, bref in ((bias, d["bias"]), (None, None)):
        y = api.fuse_gemm_bias_act_auto(x, w, b, act)
        assert_close(y[rows.cuda()], oracle.gemm_bias_act(d["x"][rows], d["w"], bref, act), "bf16",
                     f"gemm auto {M}x{N}x{K} {act} bias={b is not None} s={splits}")
        assert torch.equal(y, api.fuse_gemm_bias_act_auto(x, w, b, act))


# ------------------------------------------------------------------------------------------------
# Unfused baselines against the oracle with rounded intermediates (twice the fp16 / bf16 rule:
# an intermediate that sits on a rounding boundary may round the other way in fp32)
# ------------------------------------------------------------------------------------------------

def _loose(y, ref, kind, what):
    r = compare(y, ref, kind)
    if not r["ok"]:
        assert r["max_excess"] <= 2.0, f"{what}: {r}"


def test_unfused_add_layernorm():
    announce("unfused add_layernorm")
    d = synth.add_layernorm_inputs(2048, 4096, "f16", seed=1003)
    g = cuda(d)
    y = api.fuse_unfused_add_layernorm(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"])
    ref = oracle.add_layernorm_unfused(d["x"], d["residual"], d["gamma"], d["beta"], np.float32(d["eps"]), "f16")
    _loose(y, ref, "f16", "unfused add_layernorm")


def test_unfused_bias_gelu_residual():
    announce("unfused gelu chain")
    d = synth.bias_gelu_residual_inputs(512, 4096, "f16", seed=1002)
    g = cuda(d)
    y = api.fuse_unfused_bias_gelu_residual(g["x"], g["bias"], g["residual"])
    ref = oracle.bias_gelu_residual_unfused(d["x"], d["bias"], d["residual"], "f16")
    _loose(y, ref, "f16", "unfused gelu")


def test_unfused_softmax():
    announce("unfused softmax")
    d = synth.softmax_inputs(512, 2048, "f16", seed=1005)
    y = api.fuse_unfused_softmax_rows(d["x"].cuda(), d["scale"])
    ref = oracle.softmax_rows_unfused(d["x"], np.float32(d["scale"]), "f16")
    _loose(y, ref, "f16", "unfused softmax")


def test_unfused_cumsum():
    announce("unfused cumsum + scale")
    d = synth.cumsum_inputs(300, 4096, "f16", seed=1007)
    y = api.fuse_unfused_cumsum_scale_rows(d["x"].cuda(), d["scale"])
    ref = oracle.cumsum_scale_rows_unfused(d["x"], np.float32(d["scale"]), "f16")
    _loose(y, ref, "f16", "unfused cumsum")


def test_unfused_swiglu():
    announce("unfused swiglu")
    d = synth.swiglu_inputs(256, 384, 192, "bf16", seed=11)
    out = api.fuse_unfused_swiglu(d["a"].cuda(), d["b1"].cuda(), d["b2"].cuda())
    ref = oracle.swiglu_unfused(d["a"], d["b1"], d["b2"], "bf16")
    _loose(out, ref, "bf16", "unfused swiglu")


@pytest.mark.parametrize("act", ["none", "relu", "gelu"])
def test_unfused_gemm_bias_act(act):
    announce(f"unfused gemm + bias + {act}")
    d = synth.gemm_inputs(300, 384, 192, "bf16", seed=15)
    y = api.fuse_unfused_gemm_bias_act(d["x"].cuda(), d["w"].cuda(), d["bias"].cuda(), act)
    _loose(y, oracle.gemm_bias_act_unfused(d["x"], d["w"], d["bias"], act, "bf16"), "bf16", f"unfused gemm {act}")
    y = api.fuse_unfused_gemm_bias_act(d["x"].cuda(), d["w"].cuda(), None, act)
    _loose(y, oracle.gemm_bias_act_unfused(d["x"], d["w"], None, act, "bf16"), "bf16", f"unfused gemm {act} no bias")


def test_caller_workspace_tensors():
    # a plain device tensor as the workspace gives the same result as the one the binding
    # allocates; a too small or misaligned one is refused with nothing launched
    announce("caller-owned workspace tensors: split-K SwiGLU plan, unfused Add+LayerNorm")
    lib = api.load()
    M, N, K = 256, 512, 1536
    d = synth.swiglu_inputs(M, N, K, "bf16", seed=17)
    a, b1, b2 = d["a"].cuda(), d["b1"].cuda(), d["b2"].cuda()
    need = lib.fuse_auto_workspace_bytes(api.FUSE_OP_SWIGLU, M, N, K, api.FUSE_BF16)
    assert need > 0
    ref = api.fuse_swiglu_auto(a, b1, b2)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    assert torch.equal(api.fuse_swiglu_auto(a, b1, b2, workspace=ws), ref)
    out = torch.full_like(ref, 7.0)
    with pytest.raises(api.FuseError) as e:
        api.fuse_swiglu_auto(a, b1, b2, out=out, workspace=ws[:need - 256])
    assert e.value.status == 7 and torch.equal(out, torch.full_like(ref, 7.0))
    big = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
    with pytest.raises(api.FuseError) as e:
        api.fuse_swiglu_auto(a, b1, b2, out=out, workspace=big[16:16 + need])
    assert e.value.status == 7
    d = synth.add_layernorm_inputs(64, 4096, "f16", seed=18)
    g = cuda(d)
    y0 = api.fuse_unfused_add_layernorm(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"])
    n = lib.fuse_unfused_workspace_bytes(api.FUSE_OP_ADD_LAYERNORM, 64, 4096, 0, api.FUSE_F16)
    ws = torch.empty(n // 2, dtype=torch.float16, device="cuda")
    y1 = api.fuse_unfused_add_layernorm(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"], workspace=ws)
    assert torch.equal(y0, y1)


def test_internal_workspaces_on_a_side_stream():
    # The wrappers allocate the split-K partials and the unfused intermediates themselves when no
    # workspace is given, and enqueue the kernels on the caller's stream.  Run each on a stream
    # that is not torch's current one, with a spin kernel ahead of it so the work is still queued
    # when the wrapper returns and drops its workspace; allocations made meanwhile on the current
    # stream must not receive that memory.  Results must equal the current-stream results.
    announce("internal workspaces on a non-current stream")
    side = torch.cuda.Stream()
    d = synth.swiglu_inputs(256, 512, 1536, "bf16", seed=21)
    a, b1, b2 = d["a"].cuda(), d["b1"].cuda(), d["b2"].cuda()
    g = synth.gemm_inputs(256, 512, 1536, "bf16", seed=22)
    x, w, bias = g["x"].cuda(), g["w"].cuda(), g["bias"].cuda()
    ln = cuda(synth.add_layernorm_inputs(512, 4096, "f16", seed=23))
    sm = synth.softmax_inputs(512, 2048, "f16", seed=24)["x"].cuda()
    cs = synth.cumsum_inputs(512, 4096, "f16", seed=25)["x"].cuda()
    ge = cuda(synth.bias_gelu_residual_inputs(512, 4096, "f16", seed=26))
    calls = {
        "swiglu_auto": lambda s: api.fuse_swiglu_auto(a, b1, b2, stream=s),
        "gemm_auto": lambda s: api.fuse_gemm_bias_act_auto(x, w, bias, "gelu", stream=s),
        "unfused_swiglu": lambda s: api.fuse_unfused_swiglu(a, b1, b2, stream=s),
        "unfused_gemm": lambda s: api.fuse_unfused_gemm_bias_act(x, w, bias, "relu", stream=s),
        "unfused_add_layernorm": lambda s: api.fuse_unfused_add_layernorm(ln["x"], ln["residual"], ln["gamma"],
                                                                          ln["beta"], 1e-5, stream=s),
        "unfused_softmax": lambda s: api.fuse_unfused_softmax_rows(sm, 0.1, stream=s),
        "unfused_cumsum": lambda s: api.fuse_unfused_cumsum_scale_rows(cs, 0.5, stream=s),
        "unfused_gelu": lambda s: api.fuse_unfused_bias_gelu_residual(ge["x"], ge["bias"], ge["residual"], stream=s),
    }
    assert api.fuse_auto_splits(api.FUSE_OP_SWIGLU, 256, 512, 1536) > 1
    for name, call in calls.items():
        want = call(None)
        torch.cuda.synchronize()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            torch.cuda._sleep(1_000_000)  # keeps the side stream busy past the wrapper's return
        got = call(side)
        # memory churn on the current stream while the side stream's kernels are still queued
        junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(16)]
        del junk
        side.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(got, want), name


# ------------------------------------------------------------------------------------------------
# Captured graphs: the benchmark times every kernel as launches captured in a HIP graph over
# rotating buffer sets
# ------------------------------------------------------------------------------------------------

def _graph_op(op, seed):
    """(inputs on the GPU, launch(inputs, outs) -> outs, fresh outputs) for one fused operation."""
    if op in ("add_layernorm", "add_layernorm_ex"):
        rows = 2048 if op == "add_layernorm" else 512
        d = cuda(synth.add_layernorm_inputs(rows, 4096, "f16", seed))
        if op == "add_layernorm":
            run = lambda d, o: (api.fuse_add_layernorm(d["x"], d["residual"], d["gamma"], d["beta"], d["eps"],
                                                       y=o[0]),)
        else:
            run = lambda d, o: api.fuse_add_layernorm_ex(d["x"], d["residual"], d["gamma"], d["beta"], d["eps"],
                                                         relu=True, want_sum=True, want_stats=True, y=o[0],
                                                         sum_out=o[1], mean_out=o[2], var_out=o[3])
    elif op == "bias_gelu_residual":
        d = cuda(synth.bias_gelu_residual_inputs(512, 4096, "f16", seed))
        run = lambda d, o: (api.fuse_bias_gelu_residual(d["x"], d["bias"], d["residual"], y=o[0]),)
    elif op == "softmax":
        d = cuda(synth.softmax_inputs(1024, 2048, "f16", seed))
        run = lambda d, o: (api.fuse_softmax_rows(d["x"], d["scale"], y=o[0]),)
    elif op == "cumsum":
        d = cuda(synth.cumsum_inputs(2048, 4096, "f16", seed))
        run = lambda d, o: (api.fuse_cumsum_scale_rows(d["x"], d["scale"], y=o[0]),)
    elif op in ("swiglu", "swiglu_auto"):
        M, N, K = (512, 768, 256) if op == "swiglu" else (256, 256, 1536)
        d = cuda(synth.swiglu_inputs(M, N, K, "bf16", seed))
        if op == "swiglu":
            run = lambda d, o: (api.fuse_swiglu_dualgemm(d["a"], d["b1"], d["b2"], out=o[0]),)
        else:
            d["ws"] = api._auto_workspace(api.FUSE_OP_SWIGLU, M, N, K, d["a"].device)
            assert api.fuse_auto_splits(api.FUSE_OP_SWIGLU, M, N, K) > 1
            run = lambda d, o: (api.fuse_swiglu_auto(d["a"], d["b1"], d["b2"], out=o[0], workspace=d["ws"]),)
    else:  # GEMM + bias + ReLU
        d = cuda(synth.gemm_inputs(512, 1024, 256, "bf16", seed))
        run = lambda d, o: (api.fuse_gemm_bias_act(d["x"], d["w"], d["bias"], "relu", y=o[0]),)
    return d, run


@pytest.mark.parametrize("op", ["add_layernorm", "add_layernorm_ex", "bias_gelu_residual", "softmax", "cumsum",
                                "swiglu", "swiglu_auto", "gemm_relu"])
def test_fused_ops_in_a_replayed_graph(op):
    # three launches on three buffer sets captured in one graph, replayed three times with eager
    # work and cleared outputs in between: every replay equals the eager launches bit for bit
    announce(f"graph replay {op}")
    sets, eager = [], []
    for seed in (3, 4, 5):
        d, run = _graph_op(op, seed)
        sets.append(d)
        e = run(d, (None, None, None, None))
        eager.append(tuple(t for t in e if t is not None))
    outs = [tuple(torch.empty_like(t) for t in e) for e in eager]
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for d, o in zip(sets, outs):
            run(d, o + (None,) * (4 - len(o)))
    for rep in range(3):
        for o in outs:
            for t in o:
                t.zero_()
        run(sets[0], (None, None, None, None))  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (e, o) in enumerate(zip(eager, outs)):
            for a, b in zip(e, o):
                assert torch.equal(a, b), f"{op}: replay {rep}, buffer set {i}"
    if op == "add_layernorm":
        d = synth.add_layernorm_inputs(2048, 4096, "f16", 3)
        assert_close(outs[0][0], oracle.add_layernorm(d["x"], d["residual"], d["gamma"], d["beta"], d["eps"]),
                     "f16", "graph replay add_layernorm")


def test_copy_kernel():
    announce("copy")
    src = torch.randint(0, 255, ((1 << 20) + 7,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    api.fuse_copy(src, dst)
    assert torch.equal(src, dst)
    s2 = src[3:]
    d2 = torch.zeros_like(s2)
    api.fuse_copy(s2, d2)
    assert torch.equal(s2, d2)


def test_mfma_ceiling_kernel():
    # every accumulator element is a sum of 16 * iters products of ones: exact in fp32
    announce("mfma ceiling")
    wgs, iters = 2 * torch.cuda.get_device_properties(0).multi_processor_count, 64
    out = torch.full((wgs * 256,), -1.0, dtype=torch.float32, device="cuda")
    api.fuse_mfma_ceiling(wgs, iters, out)
    assert torch.equal(out, torch.full_like(out, 2048.0 * iters))
    part = torch.full((300,), -1.0, dtype=torch.float32, device="cuda")
    api.fuse_mfma_ceiling(1, 8192, part)  # the largest iteration count that stays exact
    assert torch.equal(part[:256], torch.full((256,), 2048.0 * 8192, device="cuda"))
    assert torch.equal(part[256:], torch.full((44,), -1.0, device="cuda"))


def test_empty_kernels_eager_and_captured():
    # the launch-cost probe runs to completion eagerly and inside a captured graph
    announce("empty kernels")
    api.fuse_empty_kernels(1000)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        api.fuse_empty_kernels(50)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
    api.fuse_empty_kernels(0)


def test_empty_inputs_launch_nothing():
    # rows == 0 / M == 0 are valid no-ops for every entry point (nothing is enqueued)
    announce("empty inputs")
    e16 = torch.empty(0, 4096, dtype=torch.float16, device="cuda")
    p16 = torch.zeros(4096, dtype=torch.float16, device="cuda")
    assert api.fuse_add_layernorm(e16, e16, p16, p16).shape == (0, 4096)
    y, s, m, v = api.fuse_add_layernorm_ex(e16, None, p16, p16, relu=True, want_sum=True, want_stats=True)
    assert y.numel() == 0 and s.numel() == 0 and m.numel() == 0 and v.numel() == 0
    assert api.fuse_bias_gelu_residual(e16, p16, e16).numel() == 0
    assert api.fuse_softmax_rows(e16, 0.5).numel() == 0
    assert api.fuse_cumsum_scale_rows(e16, 0.5).numel() == 0
    a = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(64, 128, dtype=torch.bfloat16, device="cuda")
    assert api.fuse_swiglu_dualgemm(a, b, b).shape == (0, 128)
    assert api.fuse_gemm_bias_act(a, b, None, "relu").shape == (0, 128)
    assert api.fuse_swiglu_auto(a, b, b).shape == (0, 128)
    torch.cuda.synchronize()


def test_swiglu_gemm_largest_k_and_n():
    # K and N at their limit (2^21): the 32-bit offsets inside a tile and a K step stay in range
    announce("swiglu K = 2^21")
    K = 1 << 21
    d = synth.swiglu_inputs(256, 128, K, "bf16", seed=31)
    out = api.fuse_swiglu_dualgemm(d["a"].cuda(), d["b1"].cuda(), d["b2"].cuda())
    rows = torch.tensor([0, 77, 128, 255])
    assert_close(out[rows.cuda()], oracle.swiglu(d["a"][rows], d["b1"], d["b2"]), "bf16", "K = 2^21")
    announce("gemm N = 2^21")
    N = 1 << 21
    d = synth.gemm_inputs(256, N, 32, "bf16", seed=32)
    y = api.fuse_gemm_bias_act(d["x"].cuda(), d["w"].cuda(), d["bias"].cuda(), "relu")
    rows = torch.tensor([3, 200])
    assert_close(y[rows.cuda()], oracle.gemm_bias_act(d["x"][rows], d["w"], d["bias"], "relu"), "bf16", "N = 2^21")


def test_binding_reports_status_errors():
    x = torch.zeros(4, 64, dtype=torch.float16, device="cuda")
    with pytest.raises(api.FuseError):
        api.fuse_softmax_rows(x, float("inf"))
