// launch.hpp -- internal interface between the C ABI (abi.hip) and the kernel translation units.
// Every launcher only enqueues on `stream`; the ABI layer has already validated the arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fuse_common.hpp"
#include "row_plan.hpp"

namespace fuse {

enum class EwOp : int { BiasGeluRes = 0, Add = 1, BiasAdd = 2, Gelu = 3, SiluMul = 4, Scale = 5, Relu = 6, Silu = 7 };

template <DT D>
hipError_t launch_add_layernorm(const void* x, const void* res, const void* gamma, const void* beta,
                                void* y, int64_t rows, int hidden, float eps, RowPlan plan,
                                hipStream_t stream);
template <DT D>
hipError_t launch_add_layernorm_ex(const void* x, const void* res, const void* gamma, const void* beta,
                                   void* y, void* sum, float* mean, float* var, bool relu, int64_t rows,
                                   int hidden, float eps, RowPlan plan, hipStream_t stream);
template <DT D>
hipError_t launch_softmax_rows(const void* x, void* y, int64_t rows, int cols, float scale,
                               RowPlan plan, hipStream_t stream);
// alpha is used by EwOp::Scale only.
template <DT D>
hipError_t launch_ew(EwOp op, bool vec, const void* a, const void* b, const void* c, void* out,
                     int64_t n, int64_t hidden, int chunks_per_thread, hipStream_t stream,
                     float alpha = 0.0f);
template <DT D>
hipError_t launch_cumsum_scale(const void* x, void* y, int64_t rows, int cols, float scale,
                               RowPlan plan, hipStream_t stream);
template <DT D>
hipError_t launch_softmax_unfused(const void* x, void* y, int64_t rows, int cols, float scale,
                                  bool vec, void* e, float* m, float* s, hipStream_t stream);

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);
hipError_t launch_empty(int64_t count, hipStream_t stream);
hipError_t launch_mfma_ceiling(int workgroups, int iters, float* out, hipStream_t stream);

// SwiGLU dual GEMM, bf16.  unfused = true runs the scheme-A pair instead: the same product
// kernel storing c1 and c2 (bf16, in `c1`, `c2`), then the element-wise SiLU(c1) * c2.
hipError_t launch_swiglu(const void* a, const void* b1, const void* b2, void* out, int M, int N,
                         int K, hipStream_t stream);
hipError_t launch_swiglu_unfused(const void* a, const void* b1, const void* b2, void* out, int M,
                                 int N, int K, void* c1, void* c2, hipStream_t stream);

// GEMM + bias + activation, bf16: y = act(x . w + bias) with act 0 none, 1 ReLU, 2 GELU (erf),
// 3 SiLU; bias may be null.  The unfused chain stores C (and T = C + bias) in `c` and `t`.
hipError_t launch_gemm_bias_act(const void* x, const void* w, const void* bias, void* y, int M, int N, int K,
                                int act, hipStream_t stream);
// Shape-dependent plans: K split over several workgroups per tile when the tiles alone cannot
// fill the CUs (splits > 1 needs *ws_bytes of fp32 workspace).  The *_auto launchers follow the
// plan: the single fused kernel, or the split kernel and its reduction.
int swiglu_auto_splits(int M, int N, int K, const void* a, const void* b1, const void* b2, const void* out,
                       size_t* ws_bytes);
int gemm_auto_splits(int M, int N, int K, const void* x, const void* w, const void* y, size_t* ws_bytes);
hipError_t launch_swiglu_auto(const void* a, const void* b1, const void* b2, void* out, int M, int N, int K,
                              void* ws, hipStream_t stream);
hipError_t launch_gemm_bias_act_auto(const void* x, const void* w, const void* bias, void* y, int M, int N, int K,
                                     int act, void* ws, hipStream_t stream);
// Allocation-free form of launch_swiglu_auto: split-K partials in a fixed per-device array of
// SWIGLU_NOALLOC_SCRATCH_BYTES; swiglu_noalloc_need gives the bytes a shape's plan needs (0: no split).
constexpr size_t SWIGLU_NOALLOC_SCRATCH_BYTES = size_t(64) << 20;
size_t swiglu_noalloc_need(int M, int N, int K, const void* a, const void* b1, const void* b2, const void* out);
hipError_t launch_swiglu_auto_noalloc(const void* a, const void* b1, const void* b2, void* out, int M, int N, int K,
                                      hipStream_t stream);
hipError_t launch_gemm_bias_act_unfused(const void* x, const void* w, const void* bias, void* y, int M, int N,
                                        int K, int act, void* c, void* t, hipStream_t stream);

}  // namespace fuse
