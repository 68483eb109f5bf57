// row_launch.hpp -- launchers of the row and streaming kernels, instantiated once per storage
// type by rows_f32.hip / rows_f16.hip / rows_bf16.hip.
#pragma once

#include "launch.hpp"
#include "row_kernels.hpp"
#include "row_plan.hpp"
#include "stream_kernels.hpp"

namespace fuse {

namespace detail {

template <int WPR> inline int64_t row_blocks(int64_t rows) {
    constexpr int R = RowShape<WPR>::ROWS_PER_BLOCK;
    return (rows + R - 1) / R;
}

// Calls f.template operator()<VECP, NV, WPR>() for the compiled plan equal to p; returns false
// for a plan outside the compiled set.
//   128-bit path: WPR in {1,2,4,8} x NV in {1,2,4,8}, and NV = 16 for WPR in {1,2,4}
//   per-element path: (WPR,NV) in {(1,1),(1,4),(1,16),(4,16),(8,32)}
template <class F> bool with_plan(const RowPlan& p, F&& f) {
#define FUSE_PLAN(VECP, NV, WPR) \
    if (p.vec == VECP && p.nv == NV && p.wpr == WPR) { f.template operator()<VECP, NV, WPR>(); return true; }
#define FUSE_PLAN_NV(WPR) \
    FUSE_PLAN(true, 1, WPR) FUSE_PLAN(true, 2, WPR) FUSE_PLAN(true, 4, WPR) FUSE_PLAN(true, 8, WPR)
    FUSE_PLAN_NV(1)
    FUSE_PLAN_NV(2)
    FUSE_PLAN_NV(4)
    FUSE_PLAN_NV(8)
    FUSE_PLAN(true, 16, 1)
    FUSE_PLAN(true, 16, 2)
    FUSE_PLAN(true, 16, 4)
    FUSE_PLAN(false, 1, 1)
    FUSE_PLAN(false, 4, 1)
    FUSE_PLAN(false, 16, 1)
    FUSE_PLAN(false, 16, 4)
    FUSE_PLAN(false, 32, 8)
#undef FUSE_PLAN_NV
#undef FUSE_PLAN
    return false;
}

}  // namespace detail

// Calls run.template operator()<KS>() with KS = steps (1, 2 or 4, from row_steps or scan_steps)
// on the 128-bit path with up to 4 chunks per lane when the row fills every chunk of the slice
// (full), KS = 1 otherwise.
template <bool VECP, int NV, class R> void with_steps(int steps, bool full, R&& run) {
    if constexpr (VECP && NV <= 4) {
        switch (full ? steps : 1) {
            case 2: run.template operator()<2>(); return;
            case 4: run.template operator()<4>(); return;
            default: run.template operator()<1>(); return;
        }
    } else {
        run.template operator()<1>();
    }
}

template <DT D>
hipError_t launch_add_layernorm(const void* x, const void* res, const void* gamma, const void* beta,
                                void* y, int64_t rows, int hidden, float eps, RowPlan plan,
                                hipStream_t stream) {
    using T = typename Elem<D>::T;
    hipError_t err = hipErrorInvalidValue;
    auto go = [&]<bool VECP, int NV, int WPR>() {
        const int64_t blocks = detail::row_blocks<WPR>(rows);
        const bool full = VECP && (int64_t)hidden == (int64_t)NV * WPR * 64 * Elem<D>::VEC;
        with_steps<VECP, NV>(row_steps(blocks), full, [&]<int KS>() {
            const dim3 grid((unsigned)((blocks + KS - 1) / KS)), block(RowShape<WPR>::THREADS);
            if (res)
                hipLaunchKernelGGL((add_layernorm_kernel<D, VECP, NV, WPR, true, KS>), grid, block, 0, stream,
                                   (const T*)x, (const T*)res, (const T*)gamma, (const T*)beta, (T*)y,
                                   rows, hidden, eps);
            else
                hipLaunchKernelGGL((add_layernorm_kernel<D, VECP, NV, WPR, false, KS>), grid, block, 0, stream,
                                   (const T*)x, (const T*)nullptr, (const T*)gamma, (const T*)beta, (T*)y,
                                   rows, hidden, eps);
            err = hipGetLastError();
        });
    };
    if (!detail::with_plan(plan, go)) return hipErrorInvalidValue;
    return err;
}

template <DT D>
hipError_t launch_add_layernorm_ex(const void* x, const void* res, const void* gamma, const void* beta,
                                   void* y, void* sum, float* mean, float* var, bool relu, int64_t rows,
                                   int hidden, float eps, RowPlan plan, hipStream_t stream) {
    using T = typename Elem<D>::T;
    hipError_t err = hipErrorInvalidValue;
    const LnExtra<T> ex{(T*)sum, mean, var, relu ? 1 : 0};
    auto go = [&]<bool VECP, int NV, int WPR>() {
        const int64_t blocks = detail::row_blocks<WPR>(rows);
        const bool full = VECP && (int64_t)hidden == (int64_t)NV * WPR * 64 * Elem<D>::VEC;
        with_steps<VECP, NV>(row_steps(blocks), full, [&]<int KS>() {
            const dim3 grid((unsigned)((blocks + KS - 1) / KS)), block(RowShape<WPR>::THREADS);
            if (res)
                hipLaunchKernelGGL((add_layernorm_ex_kernel<D, VECP, NV, WPR, true, KS>), grid, block, 0, stream,
                                   (const T*)x, (const T*)res, (const T*)gamma, (const T*)beta, (T*)y,
                                   rows, hidden, eps, ex);
            else
                hipLaunchKernelGGL((add_layernorm_ex_kernel<D, VECP, NV, WPR, false, KS>), grid, block, 0, stream,
                                   (const T*)x, (const T*)nullptr, (const T*)gamma, (const T*)beta, (T*)y,
                                   rows, hidden, eps, ex);
            err = hipGetLastError();
        });
    };
    if (!detail::with_plan(plan, go)) return hipErrorInvalidValue;
    return err;
}

template <DT D>
hipError_t launch_softmax_rows(const void* x, void* y, int64_t rows, int cols, float scale,
                               RowPlan plan, hipStream_t stream) {
    using T = typename Elem<D>::T;
    hipError_t err = hipErrorInvalidValue;
    auto go = [&]<bool VECP, int NV, int WPR>() {
        const dim3 grid((unsigned)detail::row_blocks<WPR>(rows)), block(RowShape<WPR>::THREADS);
        // rows that fill every chunk of the slice need no masking of empty chunks
        const bool full = VECP && (int64_t)cols == (int64_t)NV * WPR * 64 * Elem<D>::VEC;
        if (full)
            hipLaunchKernelGGL((softmax_rows_kernel<D, VECP, NV, WPR, true>), grid, block, 0, stream,
                               (const T*)x, (T*)y, rows, cols, scale);
        else
            hipLaunchKernelGGL((softmax_rows_kernel<D, VECP, NV, WPR, false>), grid, block, 0, stream,
                               (const T*)x, (T*)y, rows, cols, scale);
        err = hipGetLastError();
    };
    if (!detail::with_plan(plan, go)) return hipErrorInvalidValue;
    return err;
}

template <DT D>
hipError_t launch_cumsum_scale(const void* x, void* y, int64_t rows, int cols, float scale,
                               RowPlan plan, hipStream_t stream) {
    using T = typename Elem<D>::T;
    hipError_t err = hipErrorInvalidValue;
    auto go = [&]<bool VECP, int NV, int WPR>() {
        const int64_t blocks = detail::row_blocks<WPR>(rows);
        const bool full = VECP && (int64_t)cols == (int64_t)NV * WPR * 64 * Elem<D>::VEC;
        with_steps<VECP, NV>(scan_steps(blocks), full, [&]<int KS>() {
            const dim3 grid((unsigned)((blocks + KS - 1) / KS)), block(RowShape<WPR>::THREADS);
            hipLaunchKernelGGL((cumsum_scale_kernel<D, VECP, NV, WPR, KS>), grid, block, 0, stream,
                               (const T*)x, (T*)y, rows, cols, scale);
            err = hipGetLastError();
        });
    };
    if (!detail::with_plan(plan, go)) return hipErrorInvalidValue;
    return err;
}

template <DT D>
hipError_t launch_ew(EwOp op, bool vec, const void* a, const void* b, const void* c, void* out,
                     int64_t n, int64_t hidden, int chunks_per_thread, hipStream_t stream, float alpha) {
    using T = typename Elem<D>::T;
    const int V = vec ? Elem<D>::VEC : 1;
    const uint64_t total = (uint64_t)(n / V);
    const uint32_t cpr = (uint32_t)(hidden / V);
    hipError_t err = hipErrorInvalidValue;
    auto go = [&]<class Op, bool VECP, int CH>() {
        const uint64_t per_block = 256ull * CH;
        const dim3 grid((unsigned)((total + per_block - 1) / per_block)), block(256);
        hipLaunchKernelGGL((ew_kernel<D, VECP, CH, Op>), grid, block, 0, stream, (const T*)a,
                           (const T*)b, (const T*)c, (T*)out, total, cpr, alpha);
        err = hipGetLastError();
    };
    auto by_ch = [&]<class Op, bool VECP>() {
        switch (chunks_per_thread) {
            case 1: go.template operator()<Op, VECP, 1>(); break;
            case 2: go.template operator()<Op, VECP, 2>(); break;
            case 4: go.template operator()<Op, VECP, 4>(); break;
            case 8: go.template operator()<Op, VECP, 8>(); break;
            default: break;
        }
    };
    auto by_vec = [&]<class Op>() {
        if (vec) by_ch.template operator()<Op, true>();
        else by_ch.template operator()<Op, false>();
    };
    switch (op) {
        case EwOp::BiasGeluRes: by_vec.template operator()<OpBiasGeluRes>(); break;
        case EwOp::Add: by_vec.template operator()<OpAdd>(); break;
        case EwOp::BiasAdd: by_vec.template operator()<OpBiasAdd>(); break;
        case EwOp::Gelu: by_vec.template operator()<OpGelu>(); break;
        case EwOp::SiluMul: by_vec.template operator()<OpSiluMul>(); break;
        case EwOp::Scale: by_vec.template operator()<OpScale>(); break;
        case EwOp::Relu: by_vec.template operator()<OpRelu>(); break;
        case EwOp::Silu: by_vec.template operator()<OpSilu>(); break;
    }
    return err;
}

template <DT D>
hipError_t launch_softmax_unfused(const void* x, void* y, int64_t rows, int cols, float scale,
                                  bool vec, void* e, float* m, float* s, hipStream_t stream) {
    using T = typename Elem<D>::T;
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    auto go = [&]<bool VECP>() -> hipError_t {
        hipLaunchKernelGGL((softmax_rowmax_kernel<D, VECP>), grid, block, 0, stream, (const T*)x, m,
                           rows, cols, scale);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL((softmax_expsum_kernel<D, VECP>), grid, block, 0, stream, (const T*)x,
                           (const float*)m, (T*)e, s, rows, cols, scale);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL((softmax_divide_kernel<D, VECP>), grid, block, 0, stream, (const T*)e,
                           (const float*)s, (T*)y, rows, cols);
        return hipGetLastError();
    };
    return vec ? go.template operator()<true>() : go.template operator()<false>();
}

}  // namespace fuse

#define FUSE_INSTANTIATE_ROWS(D)                                                                   \
    template hipError_t launch_add_layernorm<D>(const void*, const void*, const void*,       \
                                                      const void*, void*, int64_t, int, float,     \
                                                      RowPlan, hipStream_t);                       \
    template hipError_t launch_add_layernorm_ex<D>(const void*, const void*, const void*,    \
                                                   const void*, void*, void*, float*, float*, bool, \
                                                   int64_t, int, float, RowPlan, hipStream_t);     \
    template hipError_t launch_softmax_rows<D>(const void*, void*, int64_t, int, float,      \
                                                     RowPlan, hipStream_t);                        \
    template hipError_t launch_ew<D>(EwOp, bool, const void*, const void*, const void*,      \
                                           void*, int64_t, int64_t, int, hipStream_t, float);      \
    template hipError_t launch_cumsum_scale<D>(const void*, void*, int64_t, int, float,      \
                                                     RowPlan, hipStream_t);                        \
    template hipError_t launch_softmax_unfused<D>(const void*, void*, int64_t, int, float,   \
                                                        bool, void*, float*, float*, hipStream_t);
