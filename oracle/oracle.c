/*
 * oracle.c -- the CPU reference for the fused row kernels.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * Every routine is the plain mathematical definition of what the fused
 * kernels compute, written out in double precision with simple loops: the
 * row moments of LayerNorm and the exponential sum of softmax by pairwise
 * summation, products and prefix sums in ascending index order.  No blocking
 * and no fusion.  Rows are independent, so an OpenMP loop over rows changes
 * nothing in the arithmetic of any one row.
 *
 * Pages cited (titles abbreviated):
 *   [P1] "CUDA算子融合优化：提升GPU推理性能的核心机制"
 *   [P2] "4. 算子融合与Kernel合并：Element-wise算子融合、Reduce与Scan的融合策略…"
 *   [P3] "算子融合的收益量化：显存带宽瓶颈下的 Kernel 拼接实测"
 *   [P4] "融合计算范式对比：从分离 Kernel 到算子内融合的 GPU 应用优化实践"
 *
 * Inputs are the exact stored values of the device tensors (fp16 / bf16 /
 * fp32), widened to double by the caller.  Outputs are unrounded doubles.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/*
 * Sum of n doubles by recursive halving (pairwise summation).  Its rounding
 * error grows with log2(n) instead of n, so in double precision the row
 * statistics below are exact to far more digits than any fp32 / fp16 result
 * can resolve.  Blocks of up to eight terms are added left to right.
 */
static double pairwise_sum(const double *v, int64_t n)
{
    double s = 0.0;
    int64_t i, h;

    if (n <= 8) {
        for (i = 0; i < n; i++)
            s += v[i];
        return s;
    }
    h = n / 2;
    return pairwise_sum(v, h) + pairwise_sum(v + h, n - h);
}

/*
 * First two moments of a row of n values, by their definitions: the mean
 * mu = (1/n) sum v, the centred values c[i] = v[i] - mu (written to c), and
 * the population variance (1/n) sum c[i]^2 (divisor n, not n - 1).  Returns
 * the variance.  c may be v itself.
 */
static double row_moments(const double *v, double *c, int64_t n, double *mu)
{
    int64_t i;
    double m = pairwise_sum(v, n) / (double)n;

    for (i = 0; i < n; i++)
        c[i] = v[i] - m;
    for (i = 0; i < n; i++)
        c[i] = c[i] * c[i];
    *mu = m;
    return pairwise_sum(c, n) / (double)n;
}

/*
 * Residual add followed by LayerNorm (page "算子融合的收益量化", §1
 * 物理流量量化: the fused sub-graph is the sum A = X + R normalised by a
 * LayerNorm, and only the normalised Y leaves the kernel; page "4. 算子融合与
 * Kernel合并", §4.2: the normaliser is the population standard deviation with
 * eps added to the variance inside the root, and gamma / beta are indexed by
 * the position in the row).
 *
 * Per row: v = x + r; mu and var = the moments of v (row_moments);
 * y[i] = gamma[i] * (v[i] - mu) * (1 / sqrt(var + eps)) + beta[i].
 *
 * residual may be NULL, which gives the plain LayerNorm of x.
 * y may not alias x or residual.
 */
static void layernorm_row(const double *xr, const double *rr, const double *gamma,
                          const double *beta, double *v, double *work,
                          int64_t hidden, double eps, double *mu_out,
                          double *var_out)
{
    int64_t i;
    double mu, var, inv;

    for (i = 0; i < hidden; i++)
        v[i] = rr ? xr[i] + rr[i] : xr[i];
    var = row_moments(v, work, hidden, &mu);
    inv = 1.0 / sqrt(var + eps);
    if (mu_out)
        *mu_out = mu;
    if (var_out)
        *var_out = var;
    for (i = 0; i < hidden; i++)
        v[i] = gamma[i] * ((v[i] - mu) * inv) + beta[i];
}

void oracle_add_layernorm(const double *x, const double *residual,
                          const double *gamma, const double *beta, double *y,
                          int64_t rows, int64_t hidden, double eps)
{
    int64_t row;
#pragma omp parallel
    {
        double *work = malloc((size_t)(hidden > 0 ? hidden : 1) * sizeof(double));
#pragma omp for schedule(static)
        for (row = 0; row < rows; row++)
            layernorm_row(x + row * hidden,
                          residual ? residual + row * hidden : NULL, gamma,
                          beta, y + row * hidden, work, hidden, eps, NULL,
                          NULL);
        free(work);
    }
}

/*
 * Variants of the same residual-add + LayerNorm row operation.
 *
 * Page "CUDA算子融合优化", §二.1 lists "LayerNorm + ReLU" as one vertical
 * fusion: the activation is applied to the normalised value before it is
 * stored, y = max(LN(v), 0); relu != 0 selects it.  A NaN stays NaN (the test
 * is "below zero", which a NaN is not).
 * Page "4. 算子融合与Kernel合并", §4.4 (multi-output fusion): one pass over
 * the input yields several outputs, with mean and variance computed together
 * as its example.  Besides y, any of these may be requested (NULL = not
 * wanted):
 *   sum  [rows, hidden]  the pre-norm sum v = x + residual (the residual
 *                        stream a pre-norm block carries on);
 *   mean [rows]          mean of v;
 *   var  [rows]          population variance of v (without eps).
 * The statistics are those of oracle_add_layernorm (row_moments).
 */
void oracle_add_layernorm_ex(const double *x, const double *residual,
                             const double *gamma, const double *beta, double *y,
                             double *sum, double *mean, double *var,
                             int64_t rows, int64_t hidden, double eps, int relu)
{
    int64_t row;
#pragma omp parallel
    {
        double *work = malloc((size_t)(hidden > 0 ? hidden : 1) * sizeof(double));
#pragma omp for schedule(static)
        for (row = 0; row < rows; row++) {
            const double *xr = x + row * hidden;
            const double *rr = residual ? residual + row * hidden : NULL;
            double *yr = y + row * hidden;
            int64_t i;

            if (sum)
                for (i = 0; i < hidden; i++)
                    sum[row * hidden + i] = rr ? xr[i] + rr[i] : xr[i];
            layernorm_row(xr, rr, gamma, beta, yr, work, hidden, eps,
                          mean ? mean + row : NULL, var ? var + row : NULL);
            if (relu)
                for (i = 0; i < hidden; i++)
                    if (yr[i] < 0.0)
                        yr[i] = 0.0;
        }
        free(work);
    }
}

/*
 * Gaussian error linear unit, exact (erf) form: GELU(t) = t * Phi(t) with
 * Phi the standard normal CDF, Phi(t) = (1 + erf(t / sqrt 2)) / 2.
 * The pages name GELU without defining it; the erf form is the one the
 * workload specifies.
 *
 * Phi is evaluated as erfc(-t / sqrt 2) / 2, the same function: written as
 * 1 + erf(.) it cancels to exactly zero in double precision for t below
 * about -8.3, where Phi(t) is still ~1e-16, while C's erfc keeps full
 * relative accuracy in that tail.
 */
static double gelu_erf(double t)
{
    return t * (0.5 * erfc(-t / sqrt(2.0)));
}

/*
 * BiasAdd -> GELU -> ResidualAdd, the three-kernel chain of [P3]'s traffic
 * figure (intro diagram and §1): t = x + bias[col]; g = GELU(t); y = g + r.
 * The bias broadcasts over rows.
 */
void oracle_bias_gelu_residual(const double *x, const double *bias,
                               const double *residual, double *y,
                               int64_t rows, int64_t hidden)
{
    int64_t row;
#pragma omp parallel for schedule(static)
    for (row = 0; row < rows; row++) {
        int64_t i;
        for (i = 0; i < hidden; i++) {
            double t = x[row * hidden + i] + bias[i];
            double g = gelu_erf(t);
            y[row * hidden + i] = g + residual[row * hidden + i];
        }
    }
}

/*
 * Row prefix sum followed by a scale (the "Scan-Elementwise" pattern of
 * [P2] §4.4, example "Cumsum + Scale"; [P2] §4.3 on scans needing the
 * prefix sums of what precedes each element).
 *
 * y[row][j] = scale * (x[row][0] + ... + x[row][j]): the inclusive running
 * sum along the row, accumulated left to right, then multiplied by the
 * scalar.
 */
void oracle_cumsum_scale_rows(const double *x, double *y, int64_t rows,
                              int64_t cols, double scale)
{
    int64_t row;
#pragma omp parallel for schedule(static)
    for (row = 0; row < rows; row++) {
        double run = 0.0;
        int64_t j;
        for (j = 0; j < cols; j++) {
            run += x[row * cols + j];
            y[row * cols + j] = scale * run;
        }
    }
}

/*
 * Row softmax of scaled scores (page "CUDA算子融合优化", §二.1: "Softmax +
 * Scale" is one vertical fusion, so the scores are z = scale * x; page "4.
 * 算子融合与Kernel合并", §4.3: the row's maximum, the sum of the
 * exponentials, then the normalisation).
 *
 * Per row, by the definition y_j = e^{z_j} / sum_k e^{z_k} written in its
 * overflow-free form (numerator and denominator both multiplied by e^{-m}):
 * m = max_k z_k, e_k = e^{z_k - m}, s = sum_k e_k (pairwise), y_j = e_j / s.
 * m is an element of the row, so every exponent is at most 0 and s is in
 * [1, cols].
 */
void oracle_softmax_rows(const double *x, double *y, int64_t rows,
                         int64_t cols, double scale)
{
    int64_t row;
#pragma omp parallel for schedule(static)
    for (row = 0; row < rows; row++) {
        const double *xr = x + row * cols;
        double *yr = y + row * cols;
        double m = -INFINITY, s;
        int64_t j;

        for (j = 0; j < cols; j++)
            yr[j] = scale * xr[j];
        for (j = 0; j < cols; j++)
            m = (yr[j] > m || isnan(yr[j])) ? yr[j] : m;
        for (j = 0; j < cols; j++)
            yr[j] = exp(yr[j] - m);
        s = pairwise_sum(yr, cols);
        for (j = 0; j < cols; j++)
            yr[j] = yr[j] / s;
    }
}

/* SiLU(c) = c * sigmoid(c) = c / (1 + e^-c). */
static double silu(double c)
{
    return c / (1.0 + exp(-c));
}

/*
 * Plain matrix product c[M,N] = a[M,K] . b[K,N], all row-major, each entry
 * summed over k in ascending order.  The loop nest walks k outside j so that
 * b is read along its rows; the order of the terms of every c[i][j] is
 * unchanged by that.
 */
void oracle_matmul(const double *a, const double *b, double *c, int64_t M,
                   int64_t N, int64_t K)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; i++) {
        double *ci = c + i * N;
        int64_t j, k;
        for (j = 0; j < N; j++)
            ci[j] = 0.0;
        for (k = 0; k < K; k++) {
            double aik = a[i * K + k];
            const double *bk = b + k * N;
            for (j = 0; j < N; j++)
                ci[j] += aik * bk[j];
        }
    }
}

/*
 * SwiGLU of the MLP's first layer, [P4] 对比对象定义:
 * out = SiLU(matmul(a, b1)) * matmul(a, b2), element-wise product.
 * Computed as scheme A of the same page: both products first (c1, c2 are
 * caller-provided M x N scratch), then the activation and the product.
 */
void oracle_swiglu(const double *a, const double *b1, const double *b2,
                   double *out, double *c1, double *c2, int64_t M, int64_t N,
                   int64_t K)
{
    int64_t e;
    oracle_matmul(a, b1, c1, M, N, K);
    oracle_matmul(a, b2, c2, M, N, K);
    for (e = 0; e < M * N; e++)
        out[e] = silu(c1[e]) * c2[e];
}

/*
 * GEMM + BiasAdd + Activation, the first vertical fusion [P1] §二.1 lists
 * ("线性变换组合"), with its fused_gemm_bias_relu(x, W1, b1) example:
 * t = matmul(x, W) + bias[col], then the activation element-wise:
 *   act 0: none, 1: ReLU (t below zero becomes 0), 2: GELU (erf form),
 *   3: SiLU.
 * x [M,K], W [K,N], bias [N] (may be NULL: no bias), y [M,N], row-major.
 */
static double activation(double t, int act)
{
    if (act == 1)
        return t < 0.0 ? 0.0 : t;
    if (act == 2)
        return gelu_erf(t);
    if (act == 3)
        return silu(t);
    return t;
}

/* The activation alone, element-wise over n values (the last kernel of the
 * unfused chain). */
void oracle_activation(const double *t, double *y, int64_t n, int act)
{
    int64_t e;
    for (e = 0; e < n; e++)
        y[e] = activation(t[e], act);
}

void oracle_gemm_bias_act(const double *x, const double *w, const double *bias,
                          double *y, int64_t M, int64_t N, int64_t K, int act)
{
    int64_t e;
    oracle_matmul(x, w, y, M, N, K);
    for (e = 0; e < M * N; e++)
        y[e] = activation(y[e] + (bias ? bias[e % N] : 0.0), act);
}

/*
 * Round-to-nearest-even of a double to the binary16 / bfloat16 grid, the
 * value returned as a double.  Used where an unfused chain stores an
 * intermediate in the I/O type ([P3] §1 accounts each intermediate at the
 * I/O width).  IEEE 754 binary16: 10 fraction bits, exponent range
 * [-14, 15], subnormal quantum 2^-24.  bfloat16: 7 fraction bits, exponent
 * range [-126, 127], subnormal quantum 2^-133.  The round is done by scaling
 * to the quantum of the value's binade (exact for powers of two) and calling
 * nearbyint in the default round-to-nearest-even mode.
 */
static double round_to_grid(double v, int frac_bits, int emin, int emax)
{
    double a = fabs(v), q, r, maxfin;
    int e;

    if (isnan(v) || isinf(v) || v == 0.0)
        return v;
    /* largest finite value: (2 - 2^-frac) * 2^emax */
    maxfin = ldexp(2.0 - ldexp(1.0, -frac_bits), emax);
    frexp(a, &e); /* a = f * 2^e with f in [0.5, 1) => binade exponent e-1 */
    e -= 1;
    if (e < emin)
        e = emin; /* subnormal range shares the quantum of the lowest binade */
    q = ldexp(1.0, e - frac_bits);
    r = nearbyint(a / q) * q;
    /* values at or beyond max + half a quantum overflow to infinity */
    if (r > maxfin)
        r = INFINITY;
    return v < 0 ? -r : r;
}

/* kind 1 = binary16, kind 2 = bfloat16; any other kind copies unchanged. */
void oracle_round(const double *in, double *out, int64_t n, int kind)
{
    int64_t i;
    for (i = 0; i < n; i++) {
        if (kind == 1)
            out[i] = round_to_grid(in[i], 10, -14, 15);
        else if (kind == 2)
            out[i] = round_to_grid(in[i], 7, -126, 127);
        else
            out[i] = in[i];
    }
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int oracle_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the OpenMP threads of later parallel regions (n >= 1; no effect without OpenMP).  Used to
 * time the oracle single-threaded beside the all-core figure. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
