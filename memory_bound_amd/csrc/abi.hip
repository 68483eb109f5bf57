// abi.hip -- the C ABI of libfuse: argument validation, path selection and dispatch.
//
// Every entry point checks all of its arguments before it enqueues anything, so an error leaves
// the outputs untouched and the stream unchanged; launch failures are reported as FUSE_ERR_HIP
// with the hipError_t kept per thread.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "../../include/libfuse.h"
#include "launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

fuse_status_t hip_status(hipError_t e) {
    if (e == hipSuccess) return FUSE_OK;
    g_last_hip_error = (int)e;
    return FUSE_ERR_HIP;
}

int elem_bytes(fuse_dtype_t d) {
    switch (d) {
        case FUSE_F32: return 4;
        case FUSE_F16: return 2;
        case FUSE_BF16: return 2;
    }
    return 0;
}

bool valid_dtype(fuse_dtype_t d) { return d == FUSE_F32 || d == FUSE_F16 || d == FUSE_BF16; }

bool elem_aligned(const void* p, int e) { return ((uintptr_t)p % (uintptr_t)e) == 0; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// [a, a+na) and [b, b+nb) share at least one byte.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na && nb && x < y + nb && y < x + na;
}
// An output may be exactly an input of the same size, or disjoint from it.
bool bad_alias(const void* out, size_t nout, const void* in, size_t nin) {
    if (!in) return false;
    if (out == in && nout == nin) return false;
    return overlaps(out, nout, in, nin);
}

// rows * cols * e without overflow, capped well inside int64.
bool tensor_bytes(int64_t rows, int64_t cols, int e, size_t* out) {
    if (rows < 0 || cols < 0) return false;
    if (cols && rows > (INT64_C(1) << 46) / cols) return false;
    *out = (size_t)rows * (size_t)cols * (size_t)e;
    return true;
}

int env_int(const char* name) {
    const char* v = getenv(name);
    return v ? atoi(v) : 0;
}

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

bool workspace_ok(const void* ws, size_t have, size_t need) {
    return ws && have >= need && ((uintptr_t)ws & 255u) == 0;
}

template <class F> hipError_t by_dtype(fuse_dtype_t d, F&& f) {
    switch (d) {
        case FUSE_F32: return f.template operator()<fuse::DT::F32>();
        case FUSE_F16: return f.template operator()<fuse::DT::F16>();
        case FUSE_BF16: return f.template operator()<fuse::DT::BF16>();
    }
    return hipErrorInvalidValue;
}

// Common checks of the [rows, n] row operations.  Returns FUSE_OK and the tensor bytes.
fuse_status_t check_rows(int64_t rows, int64_t n, int64_t nmax, fuse_dtype_t dt, size_t* bytes) {
    if (!valid_dtype(dt)) return FUSE_ERR_BAD_DTYPE;
    if (rows < 0 || n < 1) return FUSE_ERR_BAD_SHAPE;
    if (nmax > 0 && n > nmax) return FUSE_ERR_UNSUPPORTED;
    if (rows > INT64_C(0x7fffffff)) return FUSE_ERR_BAD_SHAPE;
    if (!tensor_bytes(rows, n, elem_bytes(dt), bytes)) return FUSE_ERR_BAD_SHAPE;
    return FUSE_OK;
}

// 16-byte chunks per thread of the streaming kernels (2 measured fastest for 48 MiB); the
// FUSE_EW_CHUNKS environment variable overrides it for tuning sweeps.
int ew_chunks() {
    const int v = env_int("FUSE_EW_CHUNKS");
    return (v == 1 || v == 2 || v == 4 || v == 8) ? v : 2;
}

}  // namespace

extern "C" {

const char* fuse_status_string(fuse_status_t s) {
    switch (s) {
        case FUSE_OK: return "FUSE_OK";
        case FUSE_ERR_NULL_PTR: return "FUSE_ERR_NULL_PTR: a required pointer is NULL";
        case FUSE_ERR_BAD_SHAPE: return "FUSE_ERR_BAD_SHAPE: invalid or too large size";
        case FUSE_ERR_BAD_DTYPE: return "FUSE_ERR_BAD_DTYPE: storage type not supported by this operation";
        case FUSE_ERR_BAD_VALUE: return "FUSE_ERR_BAD_VALUE: eps or scale out of range";
        case FUSE_ERR_ALIAS: return "FUSE_ERR_ALIAS: output partially overlaps an input";
        case FUSE_ERR_UNSUPPORTED: return "FUSE_ERR_UNSUPPORTED: row longer than the kernel maximum";
        case FUSE_ERR_WORKSPACE: return "FUSE_ERR_WORKSPACE: workspace missing, too small or overlapping";
        case FUSE_ERR_MISALIGNED: return "FUSE_ERR_MISALIGNED: pointer not aligned to its element size";
        case FUSE_ERR_HIP: return "FUSE_ERR_HIP: the HIP runtime reported an error";
    }
    return "unknown fuse_status_t";
}

int fuse_last_hip_error(void) { return g_last_hip_error; }

const char* fuse_version(void) { return "libfuse 0.1 gfx950"; }

// ------------------------------------------------------------------------------------------------
// ResidualAdd + LayerNorm
// ------------------------------------------------------------------------------------------------

static fuse_status_t check_add_layernorm(const void* x, const void* residual, const void* gamma,
                                         const void* beta, void* y, int64_t rows, int64_t hidden,
                                         float eps, fuse_dtype_t dt, size_t* tb, bool* vec) {
    fuse_status_t st = check_rows(rows, hidden, FUSE_MAX_HIDDEN, dt, tb);
    if (st != FUSE_OK) return st;
    if (!isfinite(eps) || eps < 0.0f) return FUSE_ERR_BAD_VALUE;
    if (rows == 0) return FUSE_OK;
    if (!x || !gamma || !beta || !y) return FUSE_ERR_NULL_PTR;
    const int e = elem_bytes(dt);
    const void* ptrs[5] = {x, residual, gamma, beta, y};
    for (const void* p : ptrs)
        if (p && !elem_aligned(p, e)) return FUSE_ERR_MISALIGNED;
    const size_t pb = (size_t)hidden * e;
    if (bad_alias(y, *tb, x, *tb) || bad_alias(y, *tb, residual, *tb) || overlaps(y, *tb, gamma, pb) ||
        overlaps(y, *tb, beta, pb))
        return FUSE_ERR_ALIAS;
    bool a = (pb % 16) == 0;
    for (const void* p : ptrs)
        if (p && !aligned16(p)) a = false;
    *vec = a;
    return FUSE_OK;
}

fuse_status_t fuse_add_layernorm(const void* x, const void* residual, const void* gamma,
                                 const void* beta, void* y, int64_t rows, int64_t hidden, float eps,
                                 fuse_dtype_t dt, void* stream) {
    size_t tb = 0;
    bool vec = false;
    fuse_status_t st = check_add_layernorm(x, residual, gamma, beta, y, rows, hidden, eps, dt, &tb, &vec);
    if (st != FUSE_OK || rows == 0) return st;
    const fuse::RowPlan plan = fuse::plan_row(hidden, elem_bytes(dt), vec, env_int("FUSE_ROW_WPR"));
    return hip_status(by_dtype(dt, [&]<fuse::DT D>() {
        return fuse::launch_add_layernorm<D>(x, residual, gamma, beta, y, rows, (int)hidden, eps, plan,
                                             (hipStream_t)stream);
    }));
}

fuse_status_t fuse_add_layernorm_ex(const void* x, const void* residual, const void* gamma,
                                    const void* beta, void* y, void* sum_out, float* mean_out,
                                    float* var_out, int64_t rows, int64_t hidden, float eps,
                                    unsigned flags, fuse_dtype_t dt, void* stream) {
    size_t tb = 0;
    bool vec = false;
    fuse_status_t st = check_add_layernorm(x, residual, gamma, beta, y, rows, hidden, eps, dt, &tb, &vec);
    if (st != FUSE_OK) return st;
    if (flags & ~(unsigned)FUSE_LN_RELU) return FUSE_ERR_BAD_VALUE;
    if (rows == 0) return FUSE_OK;
    const int e = elem_bytes(dt);
    const size_t pb = (size_t)hidden * e, sb = (size_t)rows * sizeof(float);
    if (sum_out) {
        if (!elem_aligned(sum_out, e)) return FUSE_ERR_MISALIGNED;
        if (bad_alias(sum_out, tb, x, tb) || bad_alias(sum_out, tb, residual, tb) || overlaps(sum_out, tb, y, tb) ||
            overlaps(sum_out, tb, gamma, pb) || overlaps(sum_out, tb, beta, pb))
            return FUSE_ERR_ALIAS;
        if (!aligned16(sum_out)) vec = false;
    }
    const void* tensors[6] = {x, residual, y, sum_out, gamma, beta};
    const size_t sizes[6] = {tb, tb, tb, tb, pb, pb};
    float* const stats[2] = {mean_out, var_out};
    for (float* p : stats) {
        if (!p) continue;
        if (!elem_aligned(p, 4)) return FUSE_ERR_MISALIGNED;
        for (int i = 0; i < 6; i++)
            if (overlaps(p, sb, tensors[i], tensors[i] ? sizes[i] : 0)) return FUSE_ERR_ALIAS;
    }
    if (overlaps(mean_out, mean_out ? sb : 0, var_out, var_out ? sb : 0)) return FUSE_ERR_ALIAS;
    const int wpr = env_int("FUSE_ROW_WPR");
    fuse::RowPlan plan = fuse::plan_row(hidden, e, vec, wpr);
    // With the pre-norm sum stored as well, a row writes twice the bytes, and twice the waves per
    // row measured faster on MI355X ([2048, 4096] fp16 with ReLU, sum and statistics, cold
    // buffers, three rounds: 8 waves 13.35-13.38 us, 4 waves 13.84-13.88 us).
    if (wpr == 0 && sum_out && plan.vec && plan.wpr == 4) plan = fuse::plan_row(hidden, e, vec, 8);
    return hip_status(by_dtype(dt, [&]<fuse::DT D>() {
        return fuse::launch_add_layernorm_ex<D>(x, residual, gamma, beta, y, sum_out, mean_out, var_out,
                                                (flags & FUSE_LN_RELU) != 0, rows, (int)hidden, eps, plan,
                                                (hipStream_t)stream);
    }));
}

// ------------------------------------------------------------------------------------------------
// BiasAdd + GELU + Residual
// ------------------------------------------------------------------------------------------------

static fuse_status_t check_bias_gelu_residual(const void* x, const void* bias, const void* residual,
                                              void* y, int64_t rows, int64_t hidden,
                                              fuse_dtype_t dt, size_t* tb, bool* vec) {
    fuse_status_t st = check_rows(rows, hidden, 0, dt, tb);
    if (st != FUSE_OK) return st;
    if (rows * hidden >= (INT64_C(1) << 34)) return FUSE_ERR_BAD_SHAPE;
    if (rows == 0) return FUSE_OK;
    if (!x || !bias || !residual || !y) return FUSE_ERR_NULL_PTR;
    const int e = elem_bytes(dt);
    const void* ptrs[4] = {x, bias, residual, y};
    for (const void* p : ptrs)
        if (!elem_aligned(p, e)) return FUSE_ERR_MISALIGNED;
    const size_t pb = (size_t)hidden * e;
    if (bad_alias(y, *tb, x, *tb) || bad_alias(y, *tb, residual, *tb) || overlaps(y, *tb, bias, pb))
        return FUSE_ERR_ALIAS;
    bool a = (pb % 16) == 0;
    for (const void* p : ptrs)
        if (!aligned16(p)) a = false;
    *vec = a;
    return FUSE_OK;
}

fuse_status_t fuse_bias_gelu_residual(const void* x, const void* bias, const void* residual, void* y,
                                      int64_t rows, int64_t hidden, fuse_dtype_t dt, void* stream) {
    size_t tb = 0;
    bool vec = false;
    fuse_status_t st = check_bias_gelu_residual(x, bias, residual, y, rows, hidden, dt, &tb, &vec);
    if (st != FUSE_OK || rows == 0) return st;
    const int64_t n = rows * hidden;
    const int ch = ew_chunks();
    return hip_status(by_dtype(dt, [&]<fuse::DT D>() {
        return fuse::launch_ew<D>(fuse::EwOp::BiasGeluRes, vec, x, residual, bias, y, n, hidden, ch,
                                  (hipStream_t)stream);
    }));
}

// ------------------------------------------------------------------------------------------------
// Row softmax
// ------------------------------------------------------------------------------------------------

static fuse_status_t check_softmax(const void* x, void* y, int64_t rows, int64_t cols, float scale,
                                   fuse_dtype_t dt, size_t* tb, bool* vec) {
    fuse_status_t st = check_rows(rows, cols, FUSE_MAX_SOFTMAX_COLS, dt, tb);
    if (st != FUSE_OK) return st;
    if (!isfinite(scale)) return FUSE_ERR_BAD_VALUE;
    if (rows == 0) return FUSE_OK;
    if (!x || !y) return FUSE_ERR_NULL_PTR;
    const int e = elem_bytes(dt);
    if (!elem_aligned(x, e) || !elem_aligned(y, e)) return FUSE_ERR_MISALIGNED;
    if (bad_alias(y, *tb, x, *tb)) return FUSE_ERR_ALIAS;
    *vec = aligned16(x) && aligned16(y) && ((size_t)cols * e) % 16 == 0;
    return FUSE_OK;
}

fuse_status_t fuse_softmax_rows(const void* x, void* y, int64_t rows, int64_t cols, float scale,
                                fuse_dtype_t dt, void* stream) {
    size_t tb = 0;
    bool vec = false;
    fuse_status_t st = check_softmax(x, y, rows, cols, scale, dt, &tb, &vec);
    if (st != FUSE_OK || rows == 0) return st;
    const fuse::RowPlan plan = fuse::plan_row(cols, elem_bytes(dt), vec, env_int("FUSE_ROW_WPR"));
    return hip_status(by_dtype(dt, [&]<fuse::DT D>() {
        return fuse::launch_softmax_rows<D>(x, y, rows, (int)cols, scale, plan, (hipStream_t)stream);
    }));
}

// ------------------------------------------------------------------------------------------------
// Row cumsum + scale
// ------------------------------------------------------------------------------------------------

static fuse_status_t check_cumsum(const void* x, void* y, int64_t rows, int64_t cols, float scale,
                                  fuse_dtype_t dt, size_t* tb, bool* vec) {
    fuse_status_t st = check_rows(rows, cols, FUSE_MAX_HIDDEN, dt, tb);
    if (st != FUSE_OK) return st;
    if (!isfinite(scale)) return FUSE_ERR_BAD_VALUE;
    if (rows == 0) return FUSE_OK;
    if (!x || !y) return FUSE_ERR_NULL_PTR;
    const int e = elem_bytes(dt);
    if (!elem_aligned(x, e) || !elem_aligned(y, e)) return FUSE_ERR_MISALIGNED;
    if (bad_alias(y, *tb, x, *tb)) return FUSE_ERR_ALIAS;
    *vec = aligned16(x) && aligned16(y) && ((size_t)cols * e) % 16 == 0;
    return FUSE_OK;
}

fuse_status_t fuse_cumsum_scale_rows(const void* x, void* y, int64_t rows, int64_t cols, float scale,
                                     fuse_dtype_t dt, void* stream) {
    size_t tb = 0;
    bool vec = false;
    fuse_status_t st = check_cumsum(x, y, rows, cols, scale, dt, &tb, &vec);
    if (st != FUSE_OK || rows == 0) return st;
    const fuse::RowPlan plan = fuse::plan_row(cols, elem_bytes(dt), vec, env_int("FUSE_ROW_WPR"));
    return hip_status(by_dtype(dt, [&]<fuse::DT D>() {
        return fuse::launch_cumsum_scale<D>(x, y, rows, (int)cols, scale, plan, (hipStream_t)stream);
    }));
}

// ------------------------------------------------------------------------------------------------
// SwiGLU dual GEMM
// ------------------------------------------------------------------------------------------------

static fuse_status_t check_swiglu(const void* a, const void* b1, const void* b2, void* out,
                                  int64_t M, int64_t N, int64_t K, fuse_dtype_t dt) {
    if (!valid_dtype(dt)) return FUSE_ERR_BAD_DTYPE;
    if (dt != FUSE_BF16) return FUSE_ERR_BAD_DTYPE;
    if (M < 0 || N < 1 || K < 1) return FUSE_ERR_BAD_SHAPE;
    const int64_t lim = INT64_C(0x7fffffff);
    if (M > lim || N > lim || K > lim) return FUSE_ERR_BAD_SHAPE;
    // 32-bit offsets inside one 256-row tile of a or out and one 64-row step of b
    if (K > (INT64_C(1) << 21) || N > (INT64_C(1) << 21)) return FUSE_ERR_UNSUPPORTED;
    size_t ab, bb, ob;
    if (!tensor_bytes(M, K, 2, &ab) || !tensor_bytes(K, N, 2, &bb) || !tensor_bytes(M, N, 2, &ob))
        return FUSE_ERR_BAD_SHAPE;
    if (M == 0) return FUSE_OK;
    if (!a || !b1 || !b2 || !out) return FUSE_ERR_NULL_PTR;
    if (!elem_aligned(a, 2) || !elem_aligned(b1, 2) || !elem_aligned(b2, 2) || !elem_aligned(out, 2))
        return FUSE_ERR_MISALIGNED;
    if (overlaps(out, ob, a, ab) || overlaps(out, ob, b1, bb) || overlaps(out, ob, b2, bb))
        return FUSE_ERR_ALIAS;
    return FUSE_OK;
}

fuse_status_t fuse_swiglu_dualgemm(const void* a, const void* b1, const void* b2, void* out,
                                   int64_t M, int64_t N, int64_t K, fuse_dtype_t dt, void* stream) {
    fuse_status_t st = check_swiglu(a, b1, b2, out, M, N, K, dt);
    if (st != FUSE_OK || M == 0) return st;
    return hip_status(fuse::launch_swiglu(a, b1, b2, out, (int)M, (int)N, (int)K, (hipStream_t)stream));
}

// ------------------------------------------------------------------------------------------------
// GEMM + bias + activation
// ------------------------------------------------------------------------------------------------

static fuse_status_t check_gemm(const void* x, const void* w, const void* bias, void* y, int64_t M, int64_t N,
                                int64_t K, fuse_act_t act, fuse_dtype_t dt) {
    if (!valid_dtype(dt) || dt != FUSE_BF16) return FUSE_ERR_BAD_DTYPE;
    if (act != FUSE_ACT_NONE && act != FUSE_ACT_RELU && act != FUSE_ACT_GELU && act != FUSE_ACT_SILU)
        return FUSE_ERR_BAD_VALUE;
    if (M < 0 || N < 1 || K < 1) return FUSE_ERR_BAD_SHAPE;
    const int64_t lim = INT64_C(0x7fffffff);
    if (M > lim || N > lim || K > lim) return FUSE_ERR_BAD_SHAPE;
    if (K > (INT64_C(1) << 21) || N > (INT64_C(1) << 21)) return FUSE_ERR_UNSUPPORTED;
    size_t xb, wb, yb;
    if (!tensor_bytes(M, K, 2, &xb) || !tensor_bytes(K, N, 2, &wb) || !tensor_bytes(M, N, 2, &yb))
        return FUSE_ERR_BAD_SHAPE;
    if (M == 0) return FUSE_OK;
    if (!x || !w || !y) return FUSE_ERR_NULL_PTR;
    if (!elem_aligned(x, 2) || !elem_aligned(w, 2) || !elem_aligned(y, 2) || (bias && !elem_aligned(bias, 2)))
        return FUSE_ERR_MISALIGNED;
    if (overlaps(y, yb, x, xb) || overlaps(y, yb, w, wb) || overlaps(y, yb, bias, bias ? (size_t)N * 2 : 0))
        return FUSE_ERR_ALIAS;
    return FUSE_OK;
}

fuse_status_t fuse_gemm_bias_act(const void* x, const void* w, const void* bias, void* y, int64_t M, int64_t N,
                                 int64_t K, fuse_act_t act, fuse_dtype_t dt, void* stream) {
    fuse_status_t st = check_gemm(x, w, bias, y, M, N, K, act, dt);
    if (st != FUSE_OK || M == 0) return st;
    return hip_status(fuse::launch_gemm_bias_act(x, w, bias, y, (int)M, (int)N, (int)K, (int)act,
                                                 (hipStream_t)stream));
}

// ------------------------------------------------------------------------------------------------
// Shape-dependent plans (split K when the tiles cannot fill the CUs)
// ------------------------------------------------------------------------------------------------

int fuse_auto_splits(fuse_op_t op, int64_t M, int64_t N, int64_t K) {
    if (M < 1 || N < 1 || K < 1 || M > INT64_C(0x7fffffff) || N > (INT64_C(1) << 21) || K > (INT64_C(1) << 21))
        return 0;
    if (op == FUSE_OP_SWIGLU)
        return fuse::swiglu_auto_splits((int)M, (int)N, (int)K, nullptr, nullptr, nullptr, nullptr, nullptr);
    if (op == FUSE_OP_GEMM_BIAS_ACT)
        return fuse::gemm_auto_splits((int)M, (int)N, (int)K, nullptr, nullptr, nullptr, nullptr);
    return 0;
}

size_t fuse_auto_workspace_bytes(fuse_op_t op, int64_t M, int64_t N, int64_t K, fuse_dtype_t dt) {
    if (dt != FUSE_BF16 || M < 1 || N < 1 || K < 1 || M > INT64_C(0x7fffffff) || N > (INT64_C(1) << 21) ||
        K > (INT64_C(1) << 21))
        return 0;
    size_t b = 0;
    if (op == FUSE_OP_SWIGLU)
        fuse::swiglu_auto_splits((int)M, (int)N, (int)K, nullptr, nullptr, nullptr, nullptr, &b);
    else if (op == FUSE_OP_GEMM_BIAS_ACT)
        fuse::gemm_auto_splits((int)M, (int)N, (int)K, nullptr, nullptr, nullptr, &b);
    return b;
}

fuse_status_t fuse_swiglu_auto(const void* a, const void* b1, const void* b2, void* out, int64_t M, int64_t N,
                               int64_t K, fuse_dtype_t dt, void* ws, size_t ws_bytes, void* stream) {
    fuse_status_t st = check_swiglu(a, b1, b2, out, M, N, K, dt);
    if (st != FUSE_OK || M == 0) return st;
    size_t need = 0;
    fuse::swiglu_auto_splits((int)M, (int)N, (int)K, a, b1, b2, out, &need);
    if (need) {
        if (!workspace_ok(ws, ws_bytes, need)) return FUSE_ERR_WORKSPACE;
        const size_t ab = (size_t)M * K * 2, bb = (size_t)K * N * 2, ob = (size_t)M * N * 2;
        if (overlaps(ws, need, a, ab) || overlaps(ws, need, b1, bb) || overlaps(ws, need, b2, bb) ||
            overlaps(ws, need, out, ob))
            return FUSE_ERR_WORKSPACE;
    }
    return hip_status(fuse::launch_swiglu_auto(a, b1, b2, out, (int)M, (int)N, (int)K, ws, (hipStream_t)stream));
}

static_assert(FUSE_NOALLOC_SCRATCH_BYTES == fuse::SWIGLU_NOALLOC_SCRATCH_BYTES, "header and library agree");

fuse_status_t fuse_swiglu_auto_noalloc(const void* a, const void* b1, const void* b2, void* out, int64_t M,
                                       int64_t N, int64_t K, fuse_dtype_t dt, void* stream) {
    fuse_status_t st = check_swiglu(a, b1, b2, out, M, N, K, dt);
    if (st != FUSE_OK || M == 0) return st;
    if (fuse::swiglu_noalloc_need((int)M, (int)N, (int)K, a, b1, b2, out) > FUSE_NOALLOC_SCRATCH_BYTES)
        return FUSE_ERR_WORKSPACE;
    return hip_status(fuse::launch_swiglu_auto_noalloc(a, b1, b2, out, (int)M, (int)N, (int)K, (hipStream_t)stream));
}

fuse_status_t fuse_gemm_bias_act_auto(const void* x, const void* w, const void* bias, void* y, int64_t M, int64_t N,
                                      int64_t K, fuse_act_t act, fuse_dtype_t dt, void* ws, size_t ws_bytes,
                                      void* stream) {
    fuse_status_t st = check_gemm(x, w, bias, y, M, N, K, act, dt);
    if (st != FUSE_OK || M == 0) return st;
    size_t need = 0;
    fuse::gemm_auto_splits((int)M, (int)N, (int)K, x, w, y, &need);
    if (need) {
        if (!workspace_ok(ws, ws_bytes, need)) return FUSE_ERR_WORKSPACE;
        const size_t xb = (size_t)M * K * 2, wb = (size_t)K * N * 2, yb = (size_t)M * N * 2;
        if (overlaps(ws, need, x, xb) || overlaps(ws, need, w, wb) || overlaps(ws, need, y, yb) ||
            overlaps(ws, need, bias, bias ? (size_t)N * 2 : 0))
            return FUSE_ERR_WORKSPACE;
    }
    return hip_status(fuse::launch_gemm_bias_act_auto(x, w, bias, y, (int)M, (int)N, (int)K, (int)act, ws,
                                                      (hipStream_t)stream));
}

// ------------------------------------------------------------------------------------------------
// Unfused baselines
// ------------------------------------------------------------------------------------------------

size_t fuse_unfused_workspace_bytes(fuse_op_t op, int64_t d0, int64_t d1, int64_t d2,
                                    fuse_dtype_t dt) {
    if (!valid_dtype(dt)) return 0;
    size_t tb = 0;
    switch (op) {
        case FUSE_OP_ADD_LAYERNORM:
            if (!tensor_bytes(d0, d1, elem_bytes(dt), &tb)) return 0;
            return round256(tb);
        case FUSE_OP_BIAS_GELU_RESIDUAL:
            if (!tensor_bytes(d0, d1, elem_bytes(dt), &tb)) return 0;
            return 2 * round256(tb);
        case FUSE_OP_SOFTMAX_ROWS:
            if (!tensor_bytes(d0, d1, elem_bytes(dt), &tb)) return 0;
            return round256(tb) + 2 * round256((size_t)d0 * 4);
        case FUSE_OP_SWIGLU:
            if (dt != FUSE_BF16 || !tensor_bytes(d0, d1, 2, &tb)) return 0;
            return 2 * round256(tb);
        case FUSE_OP_CUMSUM_SCALE:
            if (!tensor_bytes(d0, d1, elem_bytes(dt), &tb)) return 0;
            return round256(tb);
        case FUSE_OP_GEMM_BIAS_ACT:
            if (dt != FUSE_BF16 || !tensor_bytes(d0, d1, 2, &tb)) return 0;
            return 2 * round256(tb);
    }
    return 0;
}


fuse_status_t fuse_unfused_add_layernorm(const void* x, const void* residual, const void* gamma,
                                         const void* beta, void* y, int64_t rows, int64_t hidden,
                                         float eps, fuse_dtype_t dt, void* ws, size_t ws_bytes,
                                         void* stream) {
    size_t tb = 0;
    bool vec = false;
    fuse_status_t st = check_add_layernorm(x, residual, gamma, beta, y, rows, hidden, eps, dt, &tb, &vec);
    if (st != FUSE_OK || rows == 0) return st;
    if (!residual) return FUSE_ERR_NULL_PTR;
    const size_t need = fuse_unfused_workspace_bytes(FUSE_OP_ADD_LAYERNORM, rows, hidden, 0, dt);
    if (!workspace_ok(ws, ws_bytes, need)) return FUSE_ERR_WORKSPACE;
    const size_t pb = (size_t)hidden * elem_bytes(dt);
    if (overlaps(ws, need, x, tb) || overlaps(ws, need, residual, tb) || overlaps(ws, need, y, tb) ||
        overlaps(ws, need, gamma, pb) || overlaps(ws, need, beta, pb))
        return FUSE_ERR_WORKSPACE;
    const fuse::RowPlan plan = fuse::plan_row(hidden, elem_bytes(dt), vec, env_int("FUSE_ROW_WPR"));
    const int ch = ew_chunks();
    return hip_status(by_dtype(dt, [&]<fuse::DT D>() {
        hipError_t e = fuse::launch_ew<D>(fuse::EwOp::Add, vec, x, residual, nullptr, ws, rows * hidden,
                                          hidden, ch, (hipStream_t)stream);
        if (e != hipSuccess) return e;
        return fuse::launch_add_layernorm<D>(ws, nullptr, gamma, beta, y, rows, (int)hidden, eps, plan,
                                             (hipStream_t)stream);
    }));
}

fuse_status_t fuse_unfused_bias_gelu_residual(const void* x, const void* bias, const void* residual,
                                              void* y, int64_t rows, int64_t hidden, fuse_dtype_t dt,
                                              void* ws, size_t ws_bytes, void* stream) {
    size_t tb = 0;
    bool vec = false;
    fuse_status_t st = check_bias_gelu_residual(x, bias, residual, y, rows, hidden, dt, &tb, &vec);
    if (st != FUSE_OK || rows == 0) return st;
    const size_t need = fuse_unfused_workspace_bytes(FUSE_OP_BIAS_GELU_RESIDUAL, rows, hidden, 0, dt);
    if (!workspace_ok(ws, ws_bytes, need)) return FUSE_ERR_WORKSPACE;
    const size_t pb = (size_t)hidden * elem_bytes(dt);
    if (overlaps(ws, need, x, tb) || overlaps(ws, need, residual, tb) || overlaps(ws, need, y, tb) ||
        overlaps(ws, need, bias, pb))
        return FUSE_ERR_WORKSPACE;
    void* t = ws;
    void* g = (char*)ws + round256(tb);
    const int64_t n = rows * hidden;
    const int ch = ew_chunks();
    const hipStream_t s = (hipStream_t)stream;
    return hip_status(by_dtype(dt, [&]<fuse::DT D>() {
        hipError_t e = fuse::launch_ew<D>(fuse::EwOp::BiasAdd, vec, x, nullptr, bias, t, n, hidden, ch, s);
        if (e != hipSuccess) return e;
        e = fuse::launch_ew<D>(fuse::EwOp::Gelu, vec, t, nullptr, nullptr, g, n, hidden, ch, s);
        if (e != hipSuccess) return e;
        return fuse::launch_ew<D>(fuse::EwOp::Add, vec, g, residual, nullptr, y, n, hidden, ch, s);
    }));
}

fuse_status_t fuse_unfused_softmax_rows(const void* x, void* y, int64_t rows, int64_t cols, float scale,
                                        fuse_dtype_t dt, void* ws, size_t ws_bytes, void* stream) {
    size_t tb = 0;
    bool vec = false;
    fuse_status_t st = check_softmax(x, y, rows, cols, scale, dt, &tb, &vec);
    if (st != FUSE_OK || rows == 0) return st;
    const size_t need = fuse_unfused_workspace_bytes(FUSE_OP_SOFTMAX_ROWS, rows, cols, 0, dt);
    if (!workspace_ok(ws, ws_bytes, need)) return FUSE_ERR_WORKSPACE;
    if (overlaps(ws, need, x, tb) || overlaps(ws, need, y, tb)) return FUSE_ERR_WORKSPACE;
    void* e = ws;
    float* m = (float*)((char*)ws + round256(tb));
    float* s = (float*)((char*)m + round256((size_t)rows * 4));
    return hip_status(by_dtype(dt, [&]<fuse::DT D>() {
        return fuse::launch_softmax_unfused<D>(x, y, rows, (int)cols, scale, vec, e, m, s,
                                               (hipStream_t)stream);
    }));
}

fuse_status_t fuse_unfused_cumsum_scale_rows(const void* x, void* y, int64_t rows, int64_t cols, float scale,
                                             fuse_dtype_t dt, void* ws, size_t ws_bytes, void* stream) {
    size_t tb = 0;
    bool vec = false;
    fuse_status_t st = check_cumsum(x, y, rows, cols, scale, dt, &tb, &vec);
    if (st != FUSE_OK || rows == 0) return st;
    const size_t need = fuse_unfused_workspace_bytes(FUSE_OP_CUMSUM_SCALE, rows, cols, 0, dt);
    if (!workspace_ok(ws, ws_bytes, need)) return FUSE_ERR_WORKSPACE;
    if (overlaps(ws, need, x, tb) || overlaps(ws, need, y, tb)) return FUSE_ERR_WORKSPACE;
    const bool wvec = vec;  // the workspace is 256-byte aligned
    const fuse::RowPlan plan = fuse::plan_row(cols, elem_bytes(dt), wvec, env_int("FUSE_ROW_WPR"));
    return hip_status(by_dtype(dt, [&]<fuse::DT D>() {
        // scan kernel stores the prefix sums S in the I/O type, the element-wise kernel y = scale * S
        hipError_t e = fuse::launch_cumsum_scale<D>(x, ws, rows, (int)cols, 1.0f, plan, (hipStream_t)stream);
        if (e != hipSuccess) return e;
        return fuse::launch_ew<D>(fuse::EwOp::Scale, vec, ws, nullptr, nullptr, y, rows * cols, cols, ew_chunks(),
                                  (hipStream_t)stream, scale);
    }));
}

fuse_status_t fuse_unfused_swiglu(const void* a, const void* b1, const void* b2, void* out, int64_t M,
                                  int64_t N, int64_t K, fuse_dtype_t dt, void* ws, size_t ws_bytes,
                                  void* stream) {
    fuse_status_t st = check_swiglu(a, b1, b2, out, M, N, K, dt);
    if (st != FUSE_OK || M == 0) return st;
    const size_t need = fuse_unfused_workspace_bytes(FUSE_OP_SWIGLU, M, N, K, dt);
    if (!workspace_ok(ws, ws_bytes, need)) return FUSE_ERR_WORKSPACE;
    const size_t ab = (size_t)M * K * 2, bb = (size_t)K * N * 2, ob = (size_t)M * N * 2;
    if (overlaps(ws, need, a, ab) || overlaps(ws, need, b1, bb) || overlaps(ws, need, b2, bb) ||
        overlaps(ws, need, out, ob))
        return FUSE_ERR_WORKSPACE;
    void* c1 = ws;
    void* c2 = (char*)ws + round256(ob);
    return hip_status(fuse::launch_swiglu_unfused(a, b1, b2, out, (int)M, (int)N, (int)K, c1, c2,
                                                  (hipStream_t)stream));
}

fuse_status_t fuse_unfused_gemm_bias_act(const void* x, const void* w, const void* bias, void* y, int64_t M,
                                         int64_t N, int64_t K, fuse_act_t act, fuse_dtype_t dt, void* ws,
                                         size_t ws_bytes, void* stream) {
    fuse_status_t st = check_gemm(x, w, bias, y, M, N, K, act, dt);
    if (st != FUSE_OK || M == 0) return st;
    const size_t need = fuse_unfused_workspace_bytes(FUSE_OP_GEMM_BIAS_ACT, M, N, K, dt);
    if (!workspace_ok(ws, ws_bytes, need)) return FUSE_ERR_WORKSPACE;
    const size_t xb = (size_t)M * K * 2, wb = (size_t)K * N * 2, yb = (size_t)M * N * 2;
    if (overlaps(ws, need, x, xb) || overlaps(ws, need, w, wb) || overlaps(ws, need, y, yb) ||
        overlaps(ws, need, bias, bias ? (size_t)N * 2 : 0))
        return FUSE_ERR_WORKSPACE;
    void* c = ws;
    void* t = (char*)ws + round256(yb);
    return hip_status(fuse::launch_gemm_bias_act_unfused(x, w, bias, y, (int)M, (int)N, (int)K, (int)act, c, t,
                                                         (hipStream_t)stream));
}

// ------------------------------------------------------------------------------------------------
// Calibration copy
// ------------------------------------------------------------------------------------------------

fuse_status_t fuse_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (bytes == 0) return FUSE_OK;
    if (!src || !dst) return FUSE_ERR_NULL_PTR;
    if (bytes > ((size_t)1 << 40)) return FUSE_ERR_BAD_SHAPE;
    if (overlaps(src, bytes, dst, bytes)) return FUSE_ERR_ALIAS;
    return hip_status(fuse::launch_copy(src, dst, bytes, (hipStream_t)stream));
}

fuse_status_t fuse_mfma_ceiling(int64_t workgroups, int64_t iters, void* out, void* stream) {
    if (workgroups < 1 || workgroups > FUSE_MAX_CEILING_WORKGROUPS) return FUSE_ERR_BAD_SHAPE;
    if (iters < 1 || iters > FUSE_MAX_CEILING_ITERS) return FUSE_ERR_BAD_SHAPE;
    if (!out) return FUSE_ERR_NULL_PTR;
    if (((uintptr_t)out & 3u) != 0) return FUSE_ERR_MISALIGNED;
    return hip_status(fuse::launch_mfma_ceiling((int)workgroups, (int)iters, (float*)out, (hipStream_t)stream));
}

fuse_status_t fuse_empty_kernels(int64_t count, void* stream) {
    if (count < 0 || count > FUSE_MAX_EMPTY_KERNELS) return FUSE_ERR_BAD_SHAPE;
    return hip_status(fuse::launch_empty(count, (hipStream_t)stream));
}

}  // extern "C"
