/*
 * libfuse.h -- C ABI of libfuse: single-pass fused row kernels for AMD MI355X (gfx950).
 *
 * Pages cited (titles abbreviated):
 *   [P1] "CUDA算子融合优化：提升GPU推理性能的核心机制"
 *   [P2] "4. 算子融合与Kernel合并：Element-wise算子融合、Reduce与Scan的融合策略…"
 *   [P3] "算子融合的收益量化：显存带宽瓶颈下的 Kernel 拼接实测"
 *   [P4] "融合计算范式对比：从分离 Kernel 到算子内融合的 GPU 应用优化实践"
 *
 * Conventions shared by every entry point:
 *
 *  - Memory.  Every tensor pointer is a device pointer (memory of the device that is current
 *    on the calling thread).  The caller owns all buffers; the library never allocates or
 *    frees device memory.  Fused operations need no workspace.
 *  - Layout.  Dense, row-major, no padding: an activation [B, S, H] is passed as rows = B*S
 *    rows of `hidden` elements; per-column parameters (gamma, beta, bias) are [hidden] vectors
 *    in the activation type.  SwiGLU takes a [M,K], b1 and b2 [K,N], out [M,N].
 *  - Types.  FUSE_F32, FUSE_F16 (IEEE binary16) or FUSE_BF16 storage; arithmetic is fp32 in
 *    every kernel; every fp32 -> fp16/bf16 conversion rounds to nearest even.
 *  - Streams.  `stream` is a hipStream_t (NULL = the null stream).  Every call only enqueues
 *    work on it and returns without synchronising ([P1] §三.3 asynchronous execution).
 *  - Errors.  Every argument is checked before anything is launched; on an error nothing is
 *    enqueued and the outputs are untouched ([P1] §三.3 atomic execution of a fused kernel).
 *    A failed launch returns FUSE_ERR_HIP; fuse_last_hip_error() then gives the hipError_t.
 *    No entry point aborts or throws.
 *  - Alignment.  Any element-aligned pointer is accepted.  When every pointer is 16-byte
 *    aligned and a row is a whole number of 16-byte words the kernels use 128-bit accesses,
 *    otherwise a per-element path with the same results.
 *  - Aliasing.  An output may be exactly the same buffer as a same-shaped input (in-place use:
 *    each element is read before it is written by the same lane).  Any other overlap between
 *    an output and an input returns FUSE_ERR_ALIAS.
 *  - Sizes.  rows == 0 (or M == 0) is a valid no-op.  Negative sizes are FUSE_ERR_BAD_SHAPE.
 *  - Thread safety.  The library keeps no state besides a per-thread last-error code and a
 *    per-device cache of the compute-unit count (read once with hipDeviceGetAttribute).
 *  - Tuning overrides.  Launch plans are chosen per shape and device; these environment
 *    variables, read at every call, override them for measurement and tests and never change
 *    what is computed.  FUSE_ROW_STEPS, FUSE_EW_CHUNKS, FUSE_SWIGLU_STAGES, FUSE_SWIGLU_TAIL and
 *    FUSE_SWIGLU_PERSIST leave every result bit-identical, and so does FUSE_SWIGLU_GENERAL for fuse_swiglu_dualgemm
 *    and fuse_gemm_bias_act; FUSE_ROW_WPR, FUSE_SPLITK and FUSE_SWIGLU_GENERAL on the *_auto
 *    entry points (it turns the split-K plan off) change the order of the sums, within the same
 *    tolerance:
 *    FUSE_ROW_WPR (waves per row: 1, 2, 4, 8), FUSE_ROW_STEPS (row blocks per workgroup: 1, 2,
 *    4), FUSE_EW_CHUNKS (16-byte chunks per thread of the streaming kernels: 1, 2, 4, 8),
 *    FUSE_SWIGLU_STAGES (LDS ring depth of the dual-product kernels: 3, 4, 5; depths other
 *    than the default 4 run one workgroup per tile),
 *    FUSE_SWIGLU_TAIL (last-round slices: 0 off, 2 halves only), FUSE_SWIGLU_PERSIST (0: one
 *    workgroup per tile instead of one per CU walking its tiles), FUSE_SWIGLU_GENERAL (any
 *    value: the general dual-product kernel for every shape), FUSE_SPLITK (K splits of the
 *    per-shape plan; 1 = never split).
 */
#ifndef LIBFUSE_H
#define LIBFUSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations below are passed by value across the ABI, where a caller may pass any int.
 * Compiled as C++ they get int as their fixed underlying type, so that every int a caller passes
 * is a value of the type (validation then rejects the ones that name nothing); in C an
 * enumeration is an int already. */
#ifdef __cplusplus
#define FUSE_ENUM_BASE : int
#else
#define FUSE_ENUM_BASE
#endif

typedef enum fuse_status_e FUSE_ENUM_BASE {
    FUSE_OK = 0,
    FUSE_ERR_NULL_PTR = 1,    /* a required pointer is NULL */
    FUSE_ERR_BAD_SHAPE = 2,   /* a size is negative, zero where it must be positive, or too big */
    FUSE_ERR_BAD_DTYPE = 3,   /* the storage type is not one this operation supports */
    FUSE_ERR_BAD_VALUE = 4,   /* eps or scale is not finite, or eps is negative */
    FUSE_ERR_ALIAS = 5,       /* an output overlaps an input other than by exact in-place use */
    FUSE_ERR_UNSUPPORTED = 6, /* a row is longer than the in-register maximum */
    FUSE_ERR_WORKSPACE = 7,   /* an unfused baseline was given too small a workspace */
    FUSE_ERR_MISALIGNED = 8,  /* a pointer is not aligned to its element size */
    FUSE_ERR_HIP = 9          /* the HIP runtime reported an error at launch */
} fuse_status_t;

typedef enum fuse_dtype_e FUSE_ENUM_BASE { FUSE_F32 = 0, FUSE_F16 = 1, FUSE_BF16 = 2 } fuse_dtype_t;

/* Longest row the register-resident row kernels accept (elements). */
#define FUSE_MAX_HIDDEN 16384
#define FUSE_MAX_SOFTMAX_COLS 16384

/*
 * Fused ResidualAdd + LayerNorm, one pass over HBM.
 *   v = x + residual;  mean = sum(v)/H;  var = sum((v - mean)^2)/H;
 *   y = gamma * (v - mean) / sqrt(var + eps) + beta.
 * [P3] §1 (物理流量量化): X and R are read once into registers, the sum and the LayerNorm
 * reduction happen in place, and only Y is written (48 MB instead of 80 MB at
 * [1,2048,4096] fp16).  [P2] §4.2 fixes the statistics: population variance (divide by H)
 * and eps added to the variance inside the square root.
 *
 *   x, residual : [rows, hidden] inputs.  residual may be NULL (plain LayerNorm of x).
 *   gamma, beta : [hidden] scale and shift.
 *   y           : [rows, hidden] output; may equal x or residual.
 *   eps         : finite, >= 0.
 *   dtype       : FUSE_F32, FUSE_F16 or FUSE_BF16 (all tensors share it).
 * hidden must be in [1, FUSE_MAX_HIDDEN].
 */
fuse_status_t fuse_add_layernorm(const void *x, const void *residual, const void *gamma,
                                 const void *beta, void *y, int64_t rows, int64_t hidden,
                                 float eps, fuse_dtype_t dtype, void *stream);

/*
 * Variants of the fused ResidualAdd + LayerNorm, same single pass over HBM:
 *   y = gamma * (v - mean) / sqrt(var + eps) + beta, then y = max(y, 0) with FUSE_LN_RELU,
 * plus optional extra outputs of the same pass.
 * [P1] §二.1 lists "LayerNorm + ReLU" as one vertical fusion (the activation is applied in
 * registers before the single store).  [P2] §4.4 multi-output fusion: one pass over the input
 * yields several outputs, its example being mean and var computed together.
 *
 *   x, residual, gamma, beta, y, eps : as fuse_add_layernorm.
 *   sum_out  : [rows, hidden] in the I/O type, or NULL: the pre-norm sum v = x + residual (the
 *              residual stream of a pre-norm block).  May equal x or residual (in place); must
 *              not overlap y, gamma or beta.
 *   mean_out : [rows] fp32, or NULL: mean of v.
 *   var_out  : [rows] fp32, or NULL: population variance of v (eps not added).
 *              The statistics buffers must not overlap each other or any tensor argument.
 *   flags    : 0 or FUSE_LN_RELU; any other bit is FUSE_ERR_BAD_VALUE.  A NaN stays NaN
 *              through the ReLU.
 * Under one launch plan, y (before the ReLU) and the statistics equal fuse_add_layernorm's bit for
 * bit.  A call that stores sum_out may run more waves per row than one that does not, and a
 * different split of the row sums can change the last bit of y and the statistics.
 */
#define FUSE_LN_RELU 1u
fuse_status_t fuse_add_layernorm_ex(const void *x, const void *residual, const void *gamma,
                                    const void *beta, void *y, void *sum_out, float *mean_out,
                                    float *var_out, int64_t rows, int64_t hidden, float eps,
                                    unsigned flags, fuse_dtype_t dtype, void *stream);

/*
 * Fused BiasAdd + GELU + ResidualAdd, one pass over HBM.
 *   t = x + bias[col];  g = t * Phi(t) = t/2 * (1 + erf(t / sqrt 2));  y = g + residual.
 * [P3] intro diagram and §1: the three kernels BiasAdd, GELU and Residual become one kernel
 * that reads its inputs once and writes its output once.  The GELU is the exact (erf) form.
 *
 *   x, residual : [rows, hidden];  bias : [hidden];  y : [rows, hidden], may equal x or residual.
 *   dtype       : FUSE_F32, FUSE_F16 or FUSE_BF16.
 * hidden >= 1; rows*hidden must be below 2^34 elements.
 */
fuse_status_t fuse_bias_gelu_residual(const void *x, const void *bias, const void *residual,
                                      void *y, int64_t rows, int64_t hidden,
                                      fuse_dtype_t dtype, void *stream);

/*
 * Fused row softmax of scaled scores, one pass over HBM.
 *   z = scale * x;  m = max_j z_j;  y_j = exp(z_j - m) / sum_k exp(z_k - m).
 * [P2] §4.3: max-reduce, exp-and-sum reduce, and the element-wise divide fused into one
 * kernel.  [P1] §二.1 lists "Softmax + Scale" as one vertical fusion: the scale is applied
 * inside the same kernel.
 *
 *   x : [rows, cols];  y : [rows, cols], may equal x.
 *   scale : finite, any sign.
 *   dtype : FUSE_F32, FUSE_F16 or FUSE_BF16.
 * cols must be in [1, FUSE_MAX_SOFTMAX_COLS].
 */
fuse_status_t fuse_softmax_rows(const void *x, void *y, int64_t rows, int64_t cols, float scale,
                                fuse_dtype_t dtype, void *stream);

/*
 * Fused row cumsum + scale, one pass over HBM (the Scan-Elementwise pattern of [P2] §4.4,
 * example "Cumsum + Scale"; [P2] §4.3 on scans, which need the prefix sums of all that precedes
 * each element):
 *   y[r][j] = scale * (x[r][0] + ... + x[r][j])   (inclusive running sum along the row).
 * The row stays in registers: the running sum is built per lane, across the wave and across
 * the waves of the row, and the scale is applied before the single store.
 *
 *   x : [rows, cols];  y : [rows, cols], may equal x.
 *   scale : finite, any sign.
 *   dtype : FUSE_F32, FUSE_F16 or FUSE_BF16 (sums in fp32).
 * cols must be in [1, FUSE_MAX_HIDDEN].
 */
fuse_status_t fuse_cumsum_scale_rows(const void *x, void *y, int64_t rows, int64_t cols, float scale,
                                     fuse_dtype_t dtype, void *stream);

/*
 * Fused SwiGLU dual GEMM (scheme B of [P4] 对比对象定义):
 *   out = SiLU(a . b1) * (a . b2),  SiLU(c) = c / (1 + e^-c).
 * Each workgroup loads its tile of a once and multiplies it with the matching tiles of b1 and
 * b2 ([P4] 核心差异分析 §1); both fp32 accumulators stay in registers and the activation and
 * product are applied before the single store of out.
 *
 *   a : [M, K];  b1, b2 : [K, N];  out : [M, N], must not overlap a, b1 or b2.
 *   dtype : FUSE_BF16 (bf16 inputs and output, fp32 accumulation).
 * M >= 0, N >= 1, K >= 1, each below 2^31; K or N above 2^21 is FUSE_ERR_UNSUPPORTED.
 */
fuse_status_t fuse_swiglu_dualgemm(const void *a, const void *b1, const void *b2, void *out,
                                   int64_t M, int64_t N, int64_t K, fuse_dtype_t dtype,
                                   void *stream);

/*
 * Fused GEMM + BiasAdd + Activation, the first vertical fusion of [P1] §二.1 ("线性变换组合":
 * GEMM + BiasAdd + Activation; its example fused_gemm_bias_relu(x, W1, b1) replaces the three
 * kernels gemm, bias_add, relu):
 *   y = act(x . w + bias[col]).
 * Runs on the SwiGLU kernel's matrix-core main loop: each 256 x 256 tile of y is two adjacent
 * 128-column halves sharing the x tile; the bias and the activation are applied to the fp32
 * accumulators before the single store.
 *
 *   x : [M, K];  w : [K, N];  bias : [N] or NULL (no bias);  y : [M, N], must not overlap the
 *   others.  dtype FUSE_BF16 (bf16 in and out, fp32 accumulation).
 *   act : FUSE_ACT_NONE, FUSE_ACT_RELU (a NaN stays NaN), FUSE_ACT_GELU (erf form, as the GELU
 *   chain) or FUSE_ACT_SILU; another value is FUSE_ERR_BAD_VALUE.
 * M >= 0, N >= 1, K >= 1, each below 2^31; K or N above 2^21 is FUSE_ERR_UNSUPPORTED.
 */
typedef enum fuse_act_e FUSE_ENUM_BASE { FUSE_ACT_NONE = 0, FUSE_ACT_RELU = 1, FUSE_ACT_GELU = 2, FUSE_ACT_SILU = 3 } fuse_act_t;
fuse_status_t fuse_gemm_bias_act(const void *x, const void *w, const void *bias, void *y, int64_t M,
                                 int64_t N, int64_t K, fuse_act_t act, fuse_dtype_t dtype,
                                 void *stream);

/*
 * Unfused baselines (measurement companions).  Each runs the same computation as separate
 * kernels that store every intermediate in HBM in the I/O type, as the pages' "before
 * fusion" pictures do ([P3] §1: Add kernel writes A, LayerNorm kernel reads it; [P3] intro
 * diagram: BiasAdd, GELU, Residual; [P2] §4.3: row max, exp and sum, divide; [P4] scheme A:
 * one kernel for both products, one for SiLU and the product; [P2] §4.4: the scan kernel
 * storing the prefix sums, then the scale; [P1] §二.1: gemm, bias_add and activation kernels).  They exist so that the
 * traffic and time fusion saves can be measured, and they are the semantic reference the
 * pages recommend keeping ([P4] 迁移与使用注意事项 §3).
 *
 * The workspace is caller-owned device memory of at least fuse_unfused_workspace_bytes()
 * bytes (256-byte aligned), not overlapping any argument.  `op` selects the operation:
 */
typedef enum fuse_op_e FUSE_ENUM_BASE {
    FUSE_OP_ADD_LAYERNORM = 0,
    FUSE_OP_BIAS_GELU_RESIDUAL = 1,
    FUSE_OP_SOFTMAX_ROWS = 2,
    FUSE_OP_SWIGLU = 3,
    FUSE_OP_CUMSUM_SCALE = 4,
    FUSE_OP_GEMM_BIAS_ACT = 5
} fuse_op_t;

/* Workspace bytes for an unfused baseline: (rows, hidden, -) for the row operations,
 * (M, N, K) for SwiGLU and GEMM + bias + activation.  Returns 0 for invalid arguments. */
size_t fuse_unfused_workspace_bytes(fuse_op_t op, int64_t d0, int64_t d1, int64_t d2,
                                    fuse_dtype_t dtype);

fuse_status_t fuse_unfused_add_layernorm(const void *x, const void *residual, const void *gamma,
                                         const void *beta, void *y, int64_t rows,
                                         int64_t hidden, float eps, fuse_dtype_t dtype,
                                         void *workspace, size_t workspace_bytes, void *stream);

fuse_status_t fuse_unfused_bias_gelu_residual(const void *x, const void *bias,
                                              const void *residual, void *y, int64_t rows,
                                              int64_t hidden, fuse_dtype_t dtype,
                                              void *workspace, size_t workspace_bytes,
                                              void *stream);

fuse_status_t fuse_unfused_softmax_rows(const void *x, void *y, int64_t rows, int64_t cols,
                                        float scale, fuse_dtype_t dtype, void *workspace,
                                        size_t workspace_bytes, void *stream);

fuse_status_t fuse_unfused_swiglu(const void *a, const void *b1, const void *b2, void *out,
                                  int64_t M, int64_t N, int64_t K, fuse_dtype_t dtype,
                                  void *workspace, size_t workspace_bytes, void *stream);

fuse_status_t fuse_unfused_cumsum_scale_rows(const void *x, void *y, int64_t rows, int64_t cols,
                                             float scale, fuse_dtype_t dtype, void *workspace,
                                             size_t workspace_bytes, void *stream);

fuse_status_t fuse_unfused_gemm_bias_act(const void *x, const void *w, const void *bias, void *y,
                                         int64_t M, int64_t N, int64_t K, fuse_act_t act,
                                         fuse_dtype_t dtype, void *workspace, size_t workspace_bytes,
                                         void *stream);

/*
 * Shape-dependent selection between the fused single kernel and a split form ([P4]
 * 不同场景下的选型建议 and 迁移与使用注意事项 §4: whether fusing pays depends on whether the fused
 * kernel's blocks fill the GPU, so the choice is made per shape from the device's attributes).
 * The fused kernel's time has a floor: one workgroup walks all of K for its output tile.  When the
 * tiles cover less than half of the device's CUs (the CU count is read from the device), K may be
 * split over several workgroups per tile, each storing fp32 partial products in the workspace,
 * and a second kernel sums them in a fixed order and applies the same epilogue.  The split count
 * minimises an estimated time: the rounds of tiles x splits workgroups over the CUs times the K
 * steps of one split, plus, when split, a fixed cost for the second kernel and the partials'
 * traffic.  Each split keeps at least 4 K steps of 32 and the partials stay within 64 MiB.
 * Full-tile, 16-byte aligned shapes only; anything else runs the single fused kernel.
 *
 * fuse_auto_splits: the number of K splits the plan uses for (op, M, N, K) on the current device
 *   (1 = the single fused kernel; 0 for an invalid shape).  op is FUSE_OP_SWIGLU or
 *   FUSE_OP_GEMM_BIAS_ACT.
 * fuse_auto_workspace_bytes: the workspace that plan needs (0 when it is the single kernel).
 * fuse_swiglu_auto / fuse_gemm_bias_act_auto: as fuse_swiglu_dualgemm / fuse_gemm_bias_act,
 *   following the plan; workspace as for the unfused baselines (256-byte aligned, not
 *   overlapping any argument; may be NULL when the plan needs none).
 */
int fuse_auto_splits(fuse_op_t op, int64_t M, int64_t N, int64_t K);
size_t fuse_auto_workspace_bytes(fuse_op_t op, int64_t M, int64_t N, int64_t K, fuse_dtype_t dtype);
fuse_status_t fuse_swiglu_auto(const void *a, const void *b1, const void *b2, void *out, int64_t M,
                               int64_t N, int64_t K, fuse_dtype_t dtype, void *workspace,
                               size_t workspace_bytes, void *stream);
fuse_status_t fuse_gemm_bias_act_auto(const void *x, const void *w, const void *bias, void *y,
                                      int64_t M, int64_t N, int64_t K, fuse_act_t act,
                                      fuse_dtype_t dtype, void *workspace, size_t workspace_bytes,
                                      void *stream);

/*
 * Allocation-free form of fuse_swiglu_auto, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments without the workspace, same plan, same kernels and the same result bit for bit.
 * When the plan splits K, the fp32 partial products go to a fixed array inside the library of
 * FUSE_NOALLOC_SCRATCH_BYTES (64 MiB) per device, which each device the library runs on holds
 * from the first call there until the process ends; every plan the library chooses fits (it
 * keeps split partials within this size).  A plan that needs more (a split count forced with
 * FUSE_SPLITK) returns FUSE_ERR_WORKSPACE with nothing launched.  The call
 * allocates nothing (the array's device address is looked up once per device, on the first
 * call there).  Every call on one device shares that device's array: calls that overlap on a
 * device (on two streams, or from two threads) race on it and must be serialised by the
 * caller.  Nothing in the array needs clearing between calls.  Validation and other errors as
 * fuse_swiglu_dualgemm.
 */
#define FUSE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
fuse_status_t fuse_swiglu_auto_noalloc(const void *a, const void *b1, const void *b2, void *out,
                                       int64_t M, int64_t N, int64_t K, fuse_dtype_t dtype,
                                       void *stream);

/*
 * Plain device-to-device copy of `bytes` bytes, the calibration kernel of the roofline: its
 * achieved bandwidth is the practical ceiling a streaming kernel can reach, and its hardware
 * byte counters give the scale between counter readings and bytes moved.  src and dst must
 * not overlap; bytes at most 2^40.
 */
fuse_status_t fuse_copy(const void *src, void *dst, size_t bytes, void *stream);

/*
 * Matrix-core calibration kernel ([P4] 核心差异分析 §1 and 对比总结表 place the fused dual GEMM
 * near the compute peak; this measures the peak the matrix cores actually sustain): each of
 * `workgroups` workgroups of 256 threads (4 waves, up to 2 workgroups resident per CU) runs
 * `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 per wave, operands in registers and
 * no memory traffic in the loop -- the instruction the dual-product kernels issue.  Work per
 * call: workgroups * 4 * iters * 8 * 32768 flops.  Thread t of workgroup b writes the sum of its
 * accumulators, 2048 * iters exactly for iters <= 8192 (every operand is 1), to
 * out[256 b + t] (fp32, 4-byte aligned, workgroups * 256 values).
 * 1 <= workgroups <= FUSE_MAX_CEILING_WORKGROUPS, 1 <= iters <= FUSE_MAX_CEILING_ITERS.
 */
#define FUSE_MAX_CEILING_WORKGROUPS 65536
#define FUSE_MAX_CEILING_ITERS (1 << 24)
fuse_status_t fuse_mfma_ceiling(int64_t workgroups, int64_t iters, void *out, void *stream);

/*
 * Launch-cost probe ([P2] §4.5 and [P3] §2 argue that per-launch cost, not only traffic, is what
 * fusion and graph capture remove): enqueues `count` launches of a kernel that does nothing (one
 * 64-thread workgroup each) on `stream`, from a plain loop inside the library, so the host cost
 * per launch, the back-to-back dispatch interval and the per-kernel cost inside a captured graph
 * can be timed without any binding overhead in between.  0 <= count <= FUSE_MAX_EMPTY_KERNELS.
 */
#define FUSE_MAX_EMPTY_KERNELS 1048576
fuse_status_t fuse_empty_kernels(int64_t count, void *stream);

/* Human-readable name of a status code (static storage). */
const char *fuse_status_string(fuse_status_t status);

/* hipError_t of the last FUSE_ERR_HIP returned on this thread (0 if none). */
int fuse_last_hip_error(void);

/* Library version string (static storage). */
const char *fuse_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBFUSE_H */
