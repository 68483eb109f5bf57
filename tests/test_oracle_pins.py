"""Pins of the CPU oracle against things other than itself (no GPU).

Each op is checked against closed forms built into the input, textbook values stored under
tests/golden/, invariants the definition implies, brute force on tiny inputs, and library
routines (torch / numpy in float64).  The cases are chosen so that a dropped term, a wrong sign,
a wrong divisor, a wrong index or a transposed operand in the oracle fails at least one.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from conftest import read_golden

EPS = 1e-5


# ------------------------------------------------------------------------------------------------
# ResidualAdd + LayerNorm
# ------------------------------------------------------------------------------------------------

def _alternating(n, a, c):
    """Row c + (a, -a, a, -a, ...): mean c, population variance a^2 (n even)."""
    return c + a * np.where(np.arange(n) % 2 == 0, 1.0, -1.0)


@pytest.mark.parametrize("n,a,c", [(2, 1.0, 2.0), (8, 0.5, -3.0), (768, 2.0, 100.0), (4096, 0.25, 0.0)])
def test_ln_alternating_row_closed_form(n, a, c):
    # v = x + r is c +/- a; split it so that neither x nor r alone has that structure.
    rng = np.random.default_rng(n)
    d = np.round(rng.standard_normal(n) * 64) / 64  # dyadic, so x + r is exact
    v = _alternating(n, a, c)
    x, r = (v - d)[None, :], d[None, :]
    y = oracle.add_layernorm(x, r, np.ones(n), np.zeros(n), EPS)
    expect = np.where(np.arange(n) % 2 == 0, 1.0, -1.0) * a / math.sqrt(a * a + EPS)
    np.testing.assert_allclose(y[0], expect, rtol=0, atol=1e-12)
    # mean 0 and variance sigma^2 / (sigma^2 + eps) before the affine step
    assert abs(y.mean()) < 1e-12
    assert abs(y.var() - a * a / (a * a + EPS)) < 1e-12


def test_ln_two_element_hand_formula():
    # v = [1, 3]: mean 2, population variance 1 (an n-1 divisor would give 2)
    y = oracle.add_layernorm(np.array([[1.0, 3.0]]), None, np.ones(2), np.zeros(2), EPS)
    s = 1.0 / math.sqrt(1.0 + EPS)
    np.testing.assert_allclose(y[0], [-s, s], rtol=0, atol=1e-15)


# LayerNorm variants ([P1] §二.1 LayerNorm + ReLU; [P2] §4.4 multi-output: mean and var)

@pytest.mark.parametrize("n,a,d", [(7, -3.0, 0.5), (64, 10.0, -0.25), (4096, 0.0, 1.0)])
def test_ln_ex_stats_of_arithmetic_progression(n, a, d):
    # v_i = a + d i: mean a + d (n-1)/2, population variance d^2 (n^2 - 1) / 12 (closed forms;
    # an n-1 divisor or a missing mean term fails)
    i = np.arange(n, dtype=np.float64)
    v = a + d * i
    h = np.round(np.sin(i) * 64) / 64  # dyadic split, x + r exact
    y, sm, mean, var = oracle.add_layernorm_ex((v - h)[None, :], h[None, :], np.ones(n), np.zeros(n), EPS)
    mu, sig2 = a + d * (n - 1) / 2, d * d * (n * n - 1) / 12
    assert abs(mean[0] - mu) <= 1e-12 * max(1.0, abs(mu))
    assert abs(var[0] - sig2) <= 1e-12 * sig2
    np.testing.assert_array_equal(sm[0], v)  # the pre-norm sum, exactly x + r
    np.testing.assert_allclose(y[0], (v - mu) / math.sqrt(sig2 + EPS), rtol=0, atol=1e-11)


def test_ln_ex_relu_closed_form():
    # symmetric row: the lower half of the normalised values is negative and clamps to 0, the
    # upper half keeps the closed form; beta shifts the threshold column by column
    n = 10
    i = np.arange(n, dtype=np.float64)
    v = (i - 4.5)[None, :]
    sig2 = (n * n - 1) / 12
    xhat = (i - 4.5) / math.sqrt(sig2 + EPS)
    y, _, _, _ = oracle.add_layernorm_ex(v, None, np.ones(n), np.zeros(n), EPS, relu=True)
    np.testing.assert_allclose(y[0], np.where(i < 5, 0.0, xhat), rtol=0, atol=1e-14)
    beta = np.full(n, 0.3)
    y, _, _, _ = oracle.add_layernorm_ex(v, None, np.full(n, 2.0), beta, EPS, relu=True)
    np.testing.assert_allclose(y[0], np.maximum(2.0 * xhat + 0.3, 0.0), rtol=0, atol=1e-14)
    assert (y[0][:5] == 0).all() and y[0][5] > 0  # 2 * (-0.5 / sqrt(8.25)) + 0.3 < 0 still


def test_ln_ex_matches_plain_ln_and_keeps_nan():
    rng = np.random.default_rng(5)
    x, r = rng.standard_normal((6, 48)), rng.standard_normal((6, 48))
    g, b = rng.uniform(0.5, 1.5, 48), rng.normal(0, 0.1, 48)
    y, _, _, _ = oracle.add_layernorm_ex(x, r, g, b, EPS)
    np.testing.assert_array_equal(y, oracle.add_layernorm(x, r, g, b, EPS))
    yr, _, _, _ = oracle.add_layernorm_ex(x, r, g, b, EPS, relu=True)
    np.testing.assert_array_equal(yr, np.where(y < 0, 0.0, y))
    x[2, 7] = np.nan
    yr, _, mean, var = oracle.add_layernorm_ex(x, r, g, b, EPS, relu=True)
    assert np.isnan(yr[2]).all() and np.isnan(mean[2]) and np.isnan(var[2])
    assert not np.isnan(yr[[0, 1, 3, 4, 5]]).any()


def test_ln_gamma_beta_indexed_by_column():
    n = 16
    v = _alternating(n, 1.0, 0.0)[None, :]
    gamma = np.arange(1, n + 1, dtype=np.float64)
    beta = -np.arange(n, dtype=np.float64) / 8
    y = oracle.add_layernorm(v, np.zeros_like(v), gamma, beta, EPS)
    xhat = np.where(np.arange(n) % 2 == 0, 1.0, -1.0) / math.sqrt(1 + EPS)
    np.testing.assert_allclose(y[0], gamma * xhat + beta, rtol=0, atol=1e-13)


def test_ln_constant_row_gives_beta_exactly():
    n = 64
    x = np.full((3, n), 5.25)
    r = -x.copy()
    r[1] = 2.0  # row 1 constant 7.25, row 0 and 2 constant 0
    beta = np.linspace(-1, 1, n)
    y = oracle.add_layernorm(x, r, np.full(n, 3.0), beta, EPS)
    for row in range(3):
        assert np.array_equal(y[row], beta)


def test_ln_scale_shift_invariance_without_eps():
    rng = np.random.default_rng(7)
    v = rng.standard_normal((4, 300))
    g, b = rng.uniform(0.5, 1.5, 300), rng.normal(0, 0.1, 300)
    y0 = oracle.add_layernorm(v, None, g, b, 0.0)
    y1 = oracle.add_layernorm(3.5 * v + 11.0, None, g, b, 0.0)
    np.testing.assert_allclose(y1, y0, rtol=0, atol=1e-12)


def test_ln_matches_torch_layer_norm_fp64():
    rng = np.random.default_rng(3)
    rows, n = 9, 768
    # rows with different means and spreads, so a wrong row stride shows
    x = rng.standard_normal((rows, n)) * np.arange(1, rows + 1)[:, None] + np.arange(rows)[:, None] * 10
    r = rng.standard_normal((rows, n))
    g, b = rng.uniform(0.5, 1.5, n), rng.normal(0, 0.1, n)
    y = oracle.add_layernorm(x, r, g, b, EPS)
    ref = F.layer_norm(torch.from_numpy(x + r), (n,), torch.from_numpy(g), torch.from_numpy(b), EPS)
    np.testing.assert_allclose(y, ref.numpy(), rtol=0, atol=1e-12)


def test_ln_residual_is_added():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 32))
    r = rng.standard_normal((2, 32))
    g, b = np.ones(32), np.zeros(32)
    y = oracle.add_layernorm(x, r, g, b, EPS)
    y_norm_only = oracle.add_layernorm(x, None, g, b, EPS)
    assert np.abs(y - y_norm_only).max() > 0.1


# ------------------------------------------------------------------------------------------------
# BiasAdd + GELU(erf) + Residual
# ------------------------------------------------------------------------------------------------

def _gelu_only(t):
    t = np.atleast_2d(np.asarray(t, dtype=np.float64))
    return oracle.bias_gelu_residual(t, np.zeros(t.shape[1]), np.zeros_like(t))


def test_gelu_zero_is_zero():
    assert _gelu_only([0.0])[0, 0] == 0.0


def test_gelu_against_erf_table():
    rows = read_golden("erf_table.txt")
    u = np.array([float(r[0]) for r in rows])
    erf_u = np.array([float(r[1]) for r in rows])
    t = math.sqrt(2.0) * u
    expect = 0.5 * t * (1.0 + erf_u)
    np.testing.assert_allclose(_gelu_only(t)[0], expect, rtol=0, atol=2e-10)


def test_gelu_against_normal_cdf_table():
    for t_s, phi_s in read_golden("normal_cdf.txt"):
        t, phi = float(t_s), float(phi_s)
        got = _gelu_only([t, -t])[0]
        assert abs(got[0] - t * phi) < 1e-14
        assert abs(got[1] - (-t) * (1.0 - phi)) < 1e-14


def test_gelu_odd_part_identity_and_tails():
    t = np.linspace(-6, 6, 97)
    g = _gelu_only(np.concatenate([t, -t]))[0]
    # GELU(t) - GELU(-t) = t * (Phi(t) + Phi(-t)) = t
    np.testing.assert_allclose(g[:97] - g[97:], t, rtol=0, atol=1e-14)
    big = _gelu_only([12.0, -12.0])[0]
    assert big[0] == 12.0 and abs(big[1]) < 1e-30


@pytest.mark.parametrize("t", [-5.0, -8.0, -8.5, -10.0, -12.0, -20.0, -30.0])
def test_gelu_negative_tail_within_mills_bounds(t):
    # For u > 0 the normal tail Q(u) = Phi(-u) satisfies the textbook Mills-ratio bounds
    # phi(u)/u * (1 - 1/u^2) < Q(u) < phi(u)/u, phi(u) = exp(-u^2/2)/sqrt(2 pi).  GELU(t)/t = Phi(t)
    # must stay inside them: an evaluation through 1 + erf(t/sqrt 2) collapses to 0 here.
    u = -t
    phi = math.exp(-u * u / 2) / math.sqrt(2 * math.pi)
    lo, hi = phi / u * (1 - 1 / (u * u)), phi / u
    q = _gelu_only([t])[0, 0] / t
    assert lo < q < hi, (t, q, lo, hi)


def test_gelu_bias_by_column_and_residual_after():
    rng = np.random.default_rng(5)
    rows, n = 3, 40
    bias = rng.normal(0, 0.5, n)
    r = rng.standard_normal((rows, n))
    # x = -bias makes the GELU argument zero in every column, so y = r exactly
    y = oracle.bias_gelu_residual(np.tile(-bias, (rows, 1)), bias, r)
    assert np.array_equal(y, r)


def test_gelu_chain_matches_torch_fp64():
    rng = np.random.default_rng(6)
    rows, n = 7, 257
    x = rng.standard_normal((rows, n)) * 3
    bias = rng.normal(0, 0.3, n)
    r = rng.standard_normal((rows, n))
    y = oracle.bias_gelu_residual(x, bias, r)
    ref = F.gelu(torch.from_numpy(x) + torch.from_numpy(bias), approximate="none") + torch.from_numpy(r)
    np.testing.assert_allclose(y, ref.numpy(), rtol=0, atol=1e-14)


# ------------------------------------------------------------------------------------------------
# Row softmax with scale
# ------------------------------------------------------------------------------------------------

def test_softmax_hand_values():
    y = oracle.softmax_rows(np.array([[0.0, math.log(2.0), math.log(4.0)]]), 1.0)
    np.testing.assert_allclose(y[0], [1 / 7, 2 / 7, 4 / 7], rtol=0, atol=1e-15)


def test_softmax_scale_applied_before_max_including_negative():
    # scale -1 turns [0, -ln 2] into [0, ln 2]
    y = oracle.softmax_rows(np.array([[0.0, -math.log(2.0)]]), -1.0)
    np.testing.assert_allclose(y[0], [1 / 3, 2 / 3], rtol=0, atol=1e-15)
    y2 = oracle.softmax_rows(np.array([[0.0, math.log(2.0) / 4]]), 4.0)
    np.testing.assert_allclose(y2[0], [1 / 3, 2 / 3], rtol=0, atol=1e-15)


def test_softmax_masked_entries():
    # -inf entries (an attention mask) get exactly 0 and the rest renormalise:
    # [0, -inf, ln 2] -> [1/3, 0, 2/3]; a row with one finite entry puts all its mass there
    y = oracle.softmax_rows(np.array([[0.0, -math.inf, math.log(2.0)], [-math.inf, 5.0, -math.inf]]), 1.0)
    np.testing.assert_allclose(y[0], [1 / 3, 0.0, 2 / 3], rtol=0, atol=1e-15)
    assert y[0, 1] == 0.0
    assert list(y[1]) == [0.0, 1.0, 0.0]


def test_softmax_constant_row_and_single_column():
    y = oracle.softmax_rows(np.full((2, 2048), 3.7), 0.5)
    assert np.all(y == 2.0 ** -11)
    y1 = oracle.softmax_rows(np.array([[5.0], [-800.0]]), 1.0)
    assert np.all(y1 == 1.0)


def test_softmax_large_values_need_max_subtraction():
    y = oracle.softmax_rows(np.array([[1000.0, 1000.0, 999.0]]), 1.0)
    e = math.exp(-1.0)
    np.testing.assert_allclose(y[0], [1 / (2 + e), 1 / (2 + e), e / (2 + e)], rtol=1e-15)


def test_softmax_rows_sum_to_one_and_shift_invariance():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 2048)) * math.sqrt(128)
    y = oracle.softmax_rows(x, 1 / math.sqrt(128))
    np.testing.assert_allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    y2 = oracle.softmax_rows(x + 37.0, 1 / math.sqrt(128))
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-18)


def test_softmax_matches_torch_fp64():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, 333)) * 4
    y = oracle.softmax_rows(x, 0.37)
    ref = torch.softmax(torch.from_numpy(x) * 0.37, dim=1)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13, atol=1e-17)


# ------------------------------------------------------------------------------------------------
# Row cumsum + scale ([P2] §4.4 Scan-Elementwise)
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 7, 768, 4096])
def test_cumsum_closed_forms(n):
    j = np.arange(n, dtype=np.float64)
    x = np.stack([np.ones(n), j, np.where(j % 2 == 0, 1.0, -1.0), (-1.0) ** j * (j + 1)])
    y = oracle.cumsum_scale_rows(x, 0.5)
    np.testing.assert_array_equal(y[0], 0.5 * (j + 1))              # running count
    np.testing.assert_array_equal(y[1], 0.5 * j * (j + 1) / 2)      # triangular numbers
    np.testing.assert_array_equal(y[2], 0.5 * (j % 2 == 0))         # 1, 0, 1, 0, ...
    # 1 - 2 + 3 - 4 ...: (j + 2) / 2 after an even index j, -(j + 1) / 2 after an odd one
    np.testing.assert_array_equal(y[3], 0.5 * np.where(j % 2 == 0, (j + 2) / 2, -(j + 1) / 2))


def test_cumsum_library_and_properties():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 300))
    y = oracle.cumsum_scale_rows(x, -0.125)
    np.testing.assert_allclose(y, -0.125 * np.cumsum(x, axis=1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(y[:, -1], -0.125 * x.sum(axis=1), rtol=0, atol=1e-12)  # last = scaled total
    np.testing.assert_allclose(np.diff(y, axis=1), -0.125 * x[:, 1:], rtol=0, atol=1e-12)  # differences
    np.testing.assert_array_equal(y[:, 0], -0.125 * x[:, 0])
    # each row independently: permuting rows permutes the output
    np.testing.assert_array_equal(oracle.cumsum_scale_rows(x[::-1], -0.125), y[::-1])
    t = torch.from_numpy(x)
    np.testing.assert_allclose(y, (-0.125 * torch.cumsum(t, dim=1)).numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# SwiGLU dual GEMM
# ------------------------------------------------------------------------------------------------

def test_silu_table_values():
    for c_s, s_s in read_golden("logistic.txt"):
        c, s = float(c_s), float(s_s)
        out = oracle.swiglu(np.array([[1.0]]), np.array([[c]]), np.array([[1.0]]))
        assert abs(out[0, 0] - s) < 1e-15


def test_swiglu_brute_force_tiny():
    rng = np.random.default_rng(10)
    M, N, K = 3, 5, 4
    a, b1, b2 = rng.standard_normal((M, K)), rng.standard_normal((K, N)), rng.standard_normal((K, N))
    out = oracle.swiglu(a, b1, b2)
    for i in range(M):
        for j in range(N):
            c1 = sum(a[i, k] * b1[k, j] for k in range(K))
            c2 = sum(a[i, k] * b2[k, j] for k in range(K))
            assert abs(out[i, j] - c1 / (1 + math.exp(-c1)) * c2) < 1e-13


def test_swiglu_identity_a_reduces_to_elementwise():
    rng = np.random.default_rng(11)
    K = N = 6
    b1, b2 = rng.standard_normal((K, N)), rng.standard_normal((K, N))
    out = oracle.swiglu(np.eye(K), b1, b2)
    ref = F.silu(torch.from_numpy(b1)) * torch.from_numpy(b2)
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-15)


def test_swiglu_rank_one_and_linear_in_b2():
    rng = np.random.default_rng(12)
    a, b1, b2 = rng.standard_normal((4, 1)), rng.standard_normal((1, 7)), rng.standard_normal((1, 7))
    out = oracle.swiglu(a, b1, b2)
    c1, c2 = a * b1, a * b2  # outer products
    np.testing.assert_allclose(out, c1 / (1 + np.exp(-c1)) * c2, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(oracle.swiglu(a, b1, -2.5 * b2), -2.5 * out, rtol=1e-14, atol=1e-15)


def test_swiglu_matches_torch_fp64_nonsquare():
    rng = np.random.default_rng(13)
    M, N, K = 17, 29, 11  # all different: a transposed operand cannot pass
    a, b1, b2 = rng.standard_normal((M, K)), rng.standard_normal((K, N)), rng.standard_normal((K, N))
    out = oracle.swiglu(a, b1, b2)
    ta, tb1, tb2 = map(torch.from_numpy, (a, b1, b2))
    ref = F.silu(ta @ tb1) * (ta @ tb2)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.matmul(a, b1), a @ b1, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------------------------------------
# Rounding onto the fp16 / bf16 grid (used by the unfused chains)
# ------------------------------------------------------------------------------------------------

def _f32_exact_values(rng):
    """Values exactly representable in fp32: random, ties between fp16 and bf16 neighbours,
    subnormals, overflow boundaries and signed zeros."""
    v = [rng.standard_normal(20000).astype(np.float32),
         (rng.standard_normal(5000) * 1e4).astype(np.float32),
         (rng.standard_normal(5000) * 1e-6).astype(np.float32)]
    h = rng.standard_normal(5000).astype(np.float16)
    up = np.nextafter(h, np.float16(np.inf))
    v.append(((h.astype(np.float32) + up.astype(np.float32)) / 2).astype(np.float32))  # fp16 ties
    bf = torch.from_numpy(rng.standard_normal(5000).astype(np.float32)).to(torch.bfloat16)
    bf32 = bf.to(torch.float32).numpy()
    step = np.abs(bf32) * 2.0 ** -8
    v.append((bf32 + step).astype(np.float32))  # bf16 ties (half a bf16 spacing above)
    v.append(np.array([0.0, -0.0, 65504.0, 65519.0, 65520.0, 7e4, -65520.0, 2.0 ** -24, 2.0 ** -25,
                       3 * 2.0 ** -26, 2.0 ** -26, 1e-8, -1e-8, 3.0e38, 3.4e38, 1.0e-40],
                      dtype=np.float32))
    return np.concatenate(v).astype(np.float64)


def test_round_f16_matches_numpy():
    rng = np.random.default_rng(14)
    v = _f32_exact_values(rng)
    got = oracle.round_to(v, "f16")
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(15)
    v = _f32_exact_values(rng)
    got = oracle.round_to(v, "bf16")
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------------------------------------
# Unfused chains: equal to the fused definition when no intermediate needs rounding, and
# different by exactly the rounding when one does
# ------------------------------------------------------------------------------------------------

def test_unfused_addln_exact_intermediate_equals_fused():
    rng = np.random.default_rng(16)
    x = np.round(rng.standard_normal((4, 64)) * 16) / 16  # x + r exact in fp16
    r = np.round(rng.standard_normal((4, 64)) * 16) / 16
    g, b = rng.uniform(0.5, 1.5, 64), rng.normal(0, 0.1, 64)
    np.testing.assert_array_equal(oracle.add_layernorm_unfused(x, r, g, b, EPS, "f16"),
                                  oracle.add_layernorm(x, r, g, b, EPS))


def test_unfused_addln_rounds_the_stored_sum():
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    r = np.array([[2.0 ** -12, 0.0, 0.0, 0.0]])  # 1 + 2^-12 is not an fp16 value: A[0] = 1
    y = oracle.add_layernorm_unfused(x, r, np.ones(4), np.zeros(4), EPS, "f16")
    np.testing.assert_array_equal(y, oracle.add_layernorm(x, None, np.ones(4), np.zeros(4), EPS))


def test_unfused_gelu_chain_structure():
    # every intermediate exactly representable: t = x + bias = 0 => g = 0 => y = r
    rng = np.random.default_rng(17)
    bias = np.round(rng.normal(0, 1, 32) * 8) / 8
    r = np.round(rng.standard_normal((2, 32)) * 8) / 8
    y = oracle.bias_gelu_residual_unfused(np.tile(-bias, (2, 1)), bias, r, "f16")
    np.testing.assert_array_equal(y, r)
    # t = 3: GELU(3) stored in fp16 before the residual add
    y3 = oracle.bias_gelu_residual_unfused(np.array([[3.0]]), np.array([0.0]), np.array([[0.0]]), "f16")
    phi3 = float(read_golden("normal_cdf.txt")[2][1])
    assert y3[0, 0] == float(np.float16(3.0 * phi3))


def test_unfused_softmax_equals_rounded_terms_over_sum():
    # max 0: terms 1 and 1/4 are fp16 values, sum 5/4
    y = oracle.softmax_rows_unfused(np.array([[0.0, -math.log(4.0)]]), 1.0, "f16")
    np.testing.assert_allclose(y[0], [0.8, 0.2], rtol=0, atol=1e-15)
    # max ln 3: terms 1/3 and 1; the stored 1/3 is the fp16 value 1365 * 2^-12, the sum is the
    # unrounded 4/3
    y = oracle.softmax_rows_unfused(np.array([[0.0, math.log(3.0)]]), 1.0, "f16")
    np.testing.assert_allclose(y[0], [1365 * 2.0 ** -12 * 0.75, 0.75], rtol=0, atol=1e-15)


def _rne_integer(k: int, frac_bits: int) -> int:
    """Integer k rounded to a float with frac_bits fraction bits, ties to even, written out by
    hand: above 2^(frac_bits+1) the spacing is 2^(e - frac_bits); a tie goes to the neighbour
    whose last kept bit is zero."""
    e = k.bit_length() - 1
    q = 1 << max(0, e - frac_bits)
    lo, rem = (k // q) * q, k % q
    if 2 * rem < q:
        return lo
    if 2 * rem > q:
        return lo + q
    return lo if (lo // q) % 2 == 0 else lo + q


@pytest.mark.parametrize("kind,frac_bits,n", [("f16", 10, 4096), ("bf16", 7, 600)])
def test_unfused_cumsum_rounds_prefix_sums_before_the_scale(kind, frac_bits, n):
    # a row of ones: the stored prefix sums are the integers 1..n, exact up to 2^(frac_bits+1)
    # and rounded to even beyond it (f16: 2049 -> 2048, 2051 -> 2052); the scale kernel then
    # multiplies the stored value.  Scale 3: scaling before the rounding would give a different
    # grid point (f16: 3 * 2052 = 6156 against round(3 * 2051) = 6152).
    x = np.ones((2, n))
    y = oracle.cumsum_scale_rows_unfused(x, 3.0, kind)
    want = np.array([3.0 * _rne_integer(k, frac_bits) for k in range(1, n + 1)])
    np.testing.assert_array_equal(y[0], want)
    np.testing.assert_array_equal(y[1], want)
    # below 2^(frac_bits+1) every prefix sum is exact: the unfused chain equals the fused result
    m = 1 << (frac_bits + 1)
    np.testing.assert_array_equal(y[0, :m], oracle.cumsum_scale_rows(x, 3.0)[0, :m])


def test_rne_integer_helper_against_numpy_f16():
    ks = np.arange(1, 8193)
    np.testing.assert_array_equal([_rne_integer(int(k), 10) for k in ks], ks.astype(np.float16).astype(np.int64))


def test_unfused_swiglu_rounds_both_products():
    a = np.array([[1.0]])
    b1 = np.array([[1.0 + 2.0 ** -10]])  # not a bf16 value: rounds to 1
    b2 = np.array([[1.0 + 2.0 ** -10]])
    y = oracle.swiglu_unfused(a, b1, b2, "bf16")
    s1 = float(read_golden("logistic.txt")[1][1])
    assert abs(y[0, 0] - s1) < 1e-15


# ------------------------------------------------------------------------------------------------
# GEMM + BiasAdd + Activation ([P1] §二.1)
# ------------------------------------------------------------------------------------------------

def test_gemm_bias_act_identity_hits_table_values():
    # x = I: y = act(W + bias) element by element; W + bias lands on the tabulated points
    t = np.array([[1.0, -1.0, 3.0, 0.0], [-3.0, 2.5, -0.5, 7.0]])  # targets of W + bias
    bias = np.array([0.25, -0.5, 1.0, 0.0])
    w = t - bias[None, :]
    x = np.eye(2)
    phi = {float(a): float(b) for a, b in read_golden("normal_cdf.txt")}
    silu = {float(a): float(b) for a, b in read_golden("logistic.txt")}
    y = oracle.gemm_bias_act(x, w, bias, "gelu")
    assert abs(y[0, 0] - 1.0 * phi[1.0]) < 1e-15
    assert abs(y[0, 2] - 3.0 * phi[3.0]) < 1e-15
    assert abs(y[1, 0] - (-3.0) * (1 - phi[3.0])) < 1e-15
    y = oracle.gemm_bias_act(x, w, bias, "silu")
    assert abs(y[0, 0] - silu[1.0]) < 1e-15 and abs(y[0, 1] - silu[-1.0]) < 1e-15
    y = oracle.gemm_bias_act(x, w, bias, "relu")
    np.testing.assert_array_equal(y, np.maximum(t, 0.0))
    np.testing.assert_array_equal(oracle.gemm_bias_act(x, w, bias, "none"), t)


def test_gemm_bias_broadcasts_over_rows_and_rank_one():
    # M, N, K all different: a transposed operand or a bias indexed by row fails
    rng = np.random.default_rng(12)
    M, N, K = 5, 7, 3
    x = np.round(rng.standard_normal((M, K)) * 8) / 8
    w = np.round(rng.standard_normal((K, N)) * 8) / 8
    bias = np.arange(N, dtype=np.float64)
    y0 = oracle.gemm_bias_act(x, w, None, "none")
    y1 = oracle.gemm_bias_act(x, w, bias, "none")
    np.testing.assert_array_equal(y1 - y0, np.broadcast_to(bias, (M, N)))
    # K = 1: y = act(x_i * w_j + b_j)
    y = oracle.gemm_bias_act(x[:, :1], w[:1], bias, "relu")
    np.testing.assert_array_equal(y, np.maximum(x[:, :1] * w[:1] + bias, 0.0))


@pytest.mark.parametrize("act", ["none", "relu", "gelu", "silu"])
def test_gemm_bias_act_torch(act):
    rng = np.random.default_rng(13)
    x, w, b = rng.standard_normal((9, 33)), rng.standard_normal((33, 17)), rng.standard_normal(17)
    t = torch.from_numpy(x) @ torch.from_numpy(w) + torch.from_numpy(b)
    ref = {"none": t, "relu": F.relu(t), "gelu": F.gelu(t, approximate="none"), "silu": F.silu(t)}[act]
    np.testing.assert_allclose(oracle.gemm_bias_act(x, w, b, act), ref.numpy(), rtol=1e-13, atol=1e-13)


def test_gemm_bias_act_unfused_exact_when_intermediates_fit():
    # small integers: C and C + b are exact in bf16, so the unfused chain equals the fused result
    rng = np.random.default_rng(14)
    x = rng.integers(-3, 4, (6, 5)).astype(np.float64)
    w = rng.integers(-3, 4, (5, 8)).astype(np.float64)
    b = rng.integers(-4, 5, 8).astype(np.float64)
    for act in ("relu", "gelu", "silu"):
        np.testing.assert_array_equal(oracle.gemm_bias_act_unfused(x, w, b, act, "bf16"),
                                      oracle.gemm_bias_act(x, w, b, act))
    # and differs once C needs more than bf16's 8 significant bits
    w2 = w + 1.0 / 512
    assert not np.array_equal(oracle.gemm_bias_act_unfused(x, w2, b, "none", "bf16"),
                              oracle.gemm_bias_act(x, w2, b, "none"))
