// stream_kernels.hpp -- element-wise streaming kernels and the looped row kernels of the
// unfused softmax chain.
//
// Element-wise mapping: the tensor is a flat array of chunks (16 bytes on the 128-bit path, one
// element otherwise); thread t of workgroup b handles chunks b*256*CH + j*256 + t, j < CH, so
// each wave instruction covers 64 consecutive chunks.  All CH loads are issued before the
// arithmetic.  A per-column vector (bias) is indexed by chunk modulo chunks-per-row.
#pragma once

#include "fuse_common.hpp"

namespace fuse {

// out = f(a, b, c[col]); the flags say which of b (same shape as a) and c (per column) exist.
struct OpBiasGeluRes {  // fused chain: GELU(x + bias) + residual
    static constexpr bool USE_B = true, USE_C = true;
    __device__ __forceinline__ float operator()(float a, float b, float c) const {
        return gelu_erf(a + c) + b;
    }
};
struct OpAdd {  // residual add: x + r
    static constexpr bool USE_B = true, USE_C = false;
    __device__ __forceinline__ float operator()(float a, float b, float) const { return a + b; }
};
struct OpBiasAdd {  // x + bias[col]
    static constexpr bool USE_B = false, USE_C = true;
    __device__ __forceinline__ float operator()(float a, float, float c) const { return a + c; }
};
struct OpGelu {  // GELU(t)
    static constexpr bool USE_B = false, USE_C = false;
    __device__ __forceinline__ float operator()(float a, float, float) const { return gelu_erf(a); }
};
struct OpSiluMul {  // SiLU(c1) * c2 (second kernel of the unfused SwiGLU)
    static constexpr bool USE_B = true, USE_C = false;
    __device__ __forceinline__ float operator()(float a, float b, float) const { return silu(a) * b; }
};

template <DT D, bool VECP, int CH, class Op, class Idx>
__device__ __forceinline__ void ew_body(const typename Elem<D>::T* a, const typename Elem<D>::T* b,
                                        const typename Elem<D>::T* c, typename Elem<D>::T* out,
                                        Idx total, Idx cpr) {
    constexpr int V = VECP ? Elem<D>::VEC : 1;
    const Op op;
    const Idx base = (Idx)blockIdx.x * (Idx)(256 * CH) + (Idx)threadIdx.x;
    float va[CH][V], vb[CH][V], vc[CH][V];
#pragma unroll
    for (int j = 0; j < CH; j++) {
        const Idx ch = base + (Idx)(j * 256);
        if (ch < total) {
            if constexpr (VECP) {
                unpack<D>(load16(a + ch * V), va[j]);
                if constexpr (Op::USE_B) unpack<D>(load16(b + ch * V), vb[j]);
                if constexpr (Op::USE_C) unpack<D>(load16(c + (ch % cpr) * V), vc[j]);
            } else {
                va[j][0] = load_scalar<D>(a + ch);
                if constexpr (Op::USE_B) vb[j][0] = load_scalar<D>(b + ch);
                if constexpr (Op::USE_C) vc[j][0] = load_scalar<D>(c + ch % cpr);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < CH; j++) {
        const Idx ch = base + (Idx)(j * 256);
        if (ch < total) {
            float o[V];
#pragma unroll
            for (int k = 0; k < V; k++)
                o[k] = op(va[j][k], Op::USE_B ? vb[j][k] : 0.0f, Op::USE_C ? vc[j][k] : 0.0f);
            if constexpr (VECP) store16(out + ch * V, pack<D>(o));
            else store_scalar<D>(out + ch, o[0]);
        }
    }
}

// 32-bit chunk arithmetic when the tensor has fewer than 2^32 chunks (the modulo for the
// per-column index is then a 32-bit one), 64-bit otherwise; the branch is uniform.
template <DT D, bool VECP, int CH, class Op>
__global__ void __launch_bounds__(256)
ew_kernel(const typename Elem<D>::T* a, const typename Elem<D>::T* b, const typename Elem<D>::T* c,
          typename Elem<D>::T* out, uint64_t total_chunks, uint64_t chunks_per_row) {
    if (total_chunks < (1ull << 32) - (uint64_t)(256 * CH))
        ew_body<D, VECP, CH, Op, uint32_t>(a, b, c, out, (uint32_t)total_chunks, (uint32_t)chunks_per_row);
    else
        ew_body<D, VECP, CH, Op, uint64_t>(a, b, c, out, total_chunks, chunks_per_row);
}

// ------------------------------------------------------------------------------------------------
// Unfused softmax: three kernels with the intermediates in HBM.  One wave per row; the row is
// walked in 64-chunk steps (no register residency needed, each kernel touches the row once).
// ------------------------------------------------------------------------------------------------
template <DT D, bool VECP>
__global__ void __launch_bounds__(256)
softmax_rowmax_kernel(const typename Elem<D>::T* x, float* m, int64_t rows, int cols, float scale) {
    constexpr int V = VECP ? Elem<D>::VEC : 1;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // whole wave leaves together; no barrier in this kernel
    const auto* xr = x + row * cols;
    const int nchunk = cols / V;
    float mx = -__builtin_inff();
    for (int c = lane; c < nchunk; c += 64) {
        float v[V];
        if constexpr (VECP) unpack<D>(load16(xr + (int64_t)c * V), v);
        else v[0] = load_scalar<D>(xr + c);
#pragma unroll
        for (int k = 0; k < V; k++) mx = fmaxf(mx, v[k] * scale);
    }
    mx = wave_allreduce(mx, MaxOp{});
    if (lane == 0) m[row] = mx;
}

template <DT D, bool VECP>
__global__ void __launch_bounds__(256)
softmax_expsum_kernel(const typename Elem<D>::T* x, const float* m, typename Elem<D>::T* e,
                      float* s, int64_t rows, int cols, float scale) {
    constexpr int V = VECP ? Elem<D>::VEC : 1;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const auto* xr = x + row * cols;
    auto* er = e + row * cols;
    const int nchunk = cols / V;
    const float mx = m[row];
    float sum = 0.0f;
    for (int c = lane; c < nchunk; c += 64) {
        float v[V];
        if constexpr (VECP) unpack<D>(load16(xr + (int64_t)c * V), v);
        else v[0] = load_scalar<D>(xr + c);
#pragma unroll
        for (int k = 0; k < V; k++) {
            v[k] = exp2_fast((v[k] * scale - mx) * LOG2E);
            sum += v[k];
        }
        if constexpr (VECP) store16(er + (int64_t)c * V, pack<D>(v));
        else store_scalar<D>(er + c, v[0]);
    }
    sum = wave_allreduce(sum, SumOp{});
    if (lane == 0) s[row] = sum;
}

template <DT D, bool VECP>
__global__ void __launch_bounds__(256)
softmax_divide_kernel(const typename Elem<D>::T* e, const float* s, typename Elem<D>::T* y,
                      int64_t rows, int cols) {
    constexpr int V = VECP ? Elem<D>::VEC : 1;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const auto* er = e + row * cols;
    auto* yr = y + row * cols;
    const int nchunk = cols / V;
    const float inv = 1.0f / s[row];
    for (int c = lane; c < nchunk; c += 64) {
        float v[V];
        if constexpr (VECP) unpack<D>(load16(er + (int64_t)c * V), v);
        else v[0] = load_scalar<D>(er + c);
#pragma unroll
        for (int k = 0; k < V; k++) v[k] *= inv;
        if constexpr (VECP) store16(yr + (int64_t)c * V, pack<D>(v));
        else store_scalar<D>(yr + c, v[0]);
    }
}

}  // namespace fuse
