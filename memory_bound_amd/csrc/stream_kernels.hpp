// stream_kernels.hpp -- element-wise streaming kernels and the looped row kernels of the
// unfused softmax chain.
//
// Element-wise mapping: the tensor is a flat array of chunks (16 bytes on the 128-bit path, one
// element otherwise); thread t of workgroup b handles chunks b*256*CH + j*256 + t, j < CH, so
// each wave instruction covers 64 consecutive chunks.  All CH loads (of every operand) are in
// flight before the arithmetic.  A per-column vector (bias) is indexed by chunk modulo
// chunks-per-row.
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
struct OpRelu {  // activation kernel of the unfused GEMM + bias + ReLU (a NaN stays NaN)
    static constexpr bool USE_B = false, USE_C = false;
    __device__ __forceinline__ float operator()(float a, float, float) const { return a < 0.0f ? 0.0f : a; }
};
struct OpSilu {  // activation kernel of the unfused GEMM + bias + SiLU
    static constexpr bool USE_B = false, USE_C = false;
    __device__ __forceinline__ float operator()(float a, float, float) const { return silu(a); }
};
struct OpScale {  // alpha * s (second kernel of the unfused cumsum + scale)
    static constexpr bool USE_B = false, USE_C = false;
    float alpha;
    __device__ __forceinline__ float operator()(float a, float, float) const { return alpha * a; }
};

// Workgroup b owns chunks [b*256*CH, (b+1)*256*CH) of the flat tensor; its buffer resources
// start at that chunk and end at the tensor's end, so the tail needs no branches and the 32-bit
// offsets stay small.  The per-column index is (first chunk mod chunks-per-row) + local chunk,
// reduced once more modulo chunks-per-row.
template <DT D, bool VECP, int CH, class Op>
__global__ void __launch_bounds__(256)
ew_kernel(const typename Elem<D>::T* a, const typename Elem<D>::T* b, const typename Elem<D>::T* c,
          typename Elem<D>::T* out, uint64_t total_chunks, uint32_t chunks_per_row, float alpha) {
    using T = typename Elem<D>::T;
    constexpr int V = VECP ? Elem<D>::VEC : 1;
    constexpr uint32_t CB = VECP ? 16u : (uint32_t)sizeof(T);  // bytes per chunk
    Op op;
    if constexpr (requires { op.alpha; }) op.alpha = alpha;
    const uint64_t first = (uint64_t)blockIdx.x * (256u * CH);
    const uint64_t left = total_chunks - first;
    const uint32_t bytes = (uint32_t)(left < 256u * CH ? left : 256u * CH) * CB;
    const rsrc_t ra = make_rsrc(a + first * V, bytes);
    const rsrc_t rb = make_rsrc(Op::USE_B ? b + first * V : a, Op::USE_B ? bytes : 0u);
    const rsrc_t ro = make_rsrc(out + first * V, bytes);
    const rsrc_t rc = make_rsrc(Op::USE_C ? c : a, Op::USE_C ? chunks_per_row * CB : 0u);
    const uint32_t col0 = Op::USE_C ? (uint32_t)(first % chunks_per_row) : 0u;

    float va[CH][V], vb[CH][V], vc[CH][V];
#pragma unroll
    for (int j = 0; j < CH; j++) {
        const uint32_t local = (uint32_t)(j * 256) + threadIdx.x;
        const uint32_t col = Op::USE_C ? (col0 + local) % chunks_per_row : 0u;
        if constexpr (VECP) {
            unpack<D>(bload16<AUX_STREAM>(ra, local * 16u), va[j]);
            if constexpr (Op::USE_B) unpack<D>(bload16<AUX_STREAM>(rb, local * 16u), vb[j]);
            if constexpr (Op::USE_C) unpack<D>(bload16(rc, col * 16u), vc[j]);
        } else {
            va[j][0] = bload_elem<D, AUX_STREAM>(ra, local);
            if constexpr (Op::USE_B) vb[j][0] = bload_elem<D, AUX_STREAM>(rb, local);
            if constexpr (Op::USE_C) vc[j][0] = bload_elem<D>(rc, col);
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // all loads in flight before the arithmetic
#pragma unroll
    for (int j = 0; j < CH; j++) {
        const uint32_t local = (uint32_t)(j * 256) + threadIdx.x;
        float o[V];
#pragma unroll
        for (int k = 0; k < V; k++)
            o[k] = op(va[j][k], Op::USE_B ? vb[j][k] : 0.0f, Op::USE_C ? vc[j][k] : 0.0f);
        if constexpr (VECP) bstore16<AUX_STREAM>(ro, local * 16u, pack<D>(o));
        else bstore_elem<D, AUX_STREAM>(ro, local, o[0]);
    }
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
    const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows) return;  // whole wave leaves together; no barrier in this kernel
    const rsrc_t rx = make_rsrc(x + row * cols, (uint32_t)cols * (uint32_t)sizeof(typename Elem<D>::T));
    const int nchunk = cols / V;
    float mx = -__builtin_inff();
    for (int c = lane; c < nchunk; c += 64) {
        float v[V];
        if constexpr (VECP) unpack<D>(bload16(rx, (uint32_t)c * 16u), v);
        else v[0] = bload_elem<D>(rx, (uint32_t)c);
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
    const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows) return;
    const uint32_t row_bytes = (uint32_t)cols * (uint32_t)sizeof(typename Elem<D>::T);
    const rsrc_t rx = make_rsrc(x + row * cols, row_bytes);
    const rsrc_t re = make_rsrc(e + row * cols, row_bytes);
    const int nchunk = cols / V;
    const float mx = m[row];
    float sum = 0.0f;
    for (int c = lane; c < nchunk; c += 64) {
        float v[V];
        if constexpr (VECP) unpack<D>(bload16(rx, (uint32_t)c * 16u), v);
        else v[0] = bload_elem<D>(rx, (uint32_t)c);
#pragma unroll
        for (int k = 0; k < V; k++) {
            v[k] = exp2_fast((v[k] * scale - mx) * LOG2E);
            sum += v[k];
        }
        if constexpr (VECP) bstore16(re, (uint32_t)c * 16u, pack<D>(v));
        else bstore_elem<D>(re, (uint32_t)c, v[0]);
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
    const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows) return;
    const uint32_t row_bytes = (uint32_t)cols * (uint32_t)sizeof(typename Elem<D>::T);
    const rsrc_t re = make_rsrc(e + row * cols, row_bytes);
    const rsrc_t ry = make_rsrc(y + row * cols, row_bytes);
    const int nchunk = cols / V;
    const float inv = 1.0f / s[row];
    for (int c = lane; c < nchunk; c += 64) {
        float v[V];
        if constexpr (VECP) unpack<D>(bload16(re, (uint32_t)c * 16u), v);
        else v[0] = bload_elem<D>(re, (uint32_t)c);
#pragma unroll
        for (int k = 0; k < V; k++) v[k] *= inv;
        if constexpr (VECP) bstore16(ry, (uint32_t)c * 16u, pack<D>(v));
        else bstore_elem<D>(ry, (uint32_t)c, v[0]);
    }
}

}  // namespace fuse
