// row_kernels.hpp -- register-resident fused row kernels: ResidualAdd+LayerNorm and the scaled
// row softmax.
//
// Mapping.  A row is owned by WPR wavefronts (WPR in {1,2,4,8}); a 256-thread workgroup holds
// 4/WPR rows (one 512-thread workgroup per row when WPR = 8).  The row is cut into chunks of V
// elements (V = 16 bytes / element size on the 128-bit path, V = 1 on the per-element path);
// chunk c = (j * WPR + w) * 64 + lane goes to lane `lane` of wave w, j = 0..NV-1, so every
// load instruction of a wave covers 64 consecutive chunks (1 KiB on the 128-bit path).  All
// loads of the row are issued before any arithmetic, the row then lives in VGPRs as fp32, and
// HBM sees exactly one read of each input and one write of the output.
//
// Reductions.  Each lane folds its own values, then wave_allreduce (DPP + swizzle) combines
// the 64 lanes, then, for WPR > 1, the per-wave results go through LDS and every wave adds
// them in wave order.  The order is fixed, so results are bit-reproducible run to run.
#pragma once

#include "fuse_common.hpp"

namespace fuse {

template <int WPR> struct RowShape {
    static constexpr int ROWS_PER_BLOCK = WPR >= 4 ? 1 : 4 / WPR;
    static constexpr int THREADS = 64 * WPR * ROWS_PER_BLOCK;
};

// Combine a per-lane partial over the WPR waves of a row; every lane of the row gets the result.
template <int WPR, class Op>
__device__ __forceinline__ float row_allreduce(float v, Op op, float* lds_slot) {
    v = wave_allreduce(v, op);
    if constexpr (WPR == 1) {
        return v;
    } else {
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) lds_slot[wave] = v;
        __syncthreads();
        const int first = wave - wave % WPR;
        float t = lds_slot[first];
#pragma unroll
        for (int i = 1; i < WPR; i++) t = op(t, lds_slot[first + i]);
        return t;
    }
}

// Per-lane slice of one row: NV chunks of V elements.
template <DT D, bool VECP, int NV, int WPR> struct RowSlice {
    using T = typename Elem<D>::T;
    static constexpr int V = VECP ? Elem<D>::VEC : 1;

    int first_chunk;  // chunk index of j = 0 for this lane
    int nchunk;       // chunks in the row

    __device__ __forceinline__ RowSlice(int hidden) {
        const int lane = threadIdx.x & 63;
        const int wpos = (threadIdx.x >> 6) % WPR;
        first_chunk = wpos * 64 + lane;
        nchunk = hidden / V;  // per-element path: V = 1
    }
    __device__ __forceinline__ int chunk(int j) const { return first_chunk + j * WPR * 64; }
    __device__ __forceinline__ bool ok(int j) const { return chunk(j) < nchunk; }

    // Read chunk j of `row` (or zeros when out of the row) as fp32.
    __device__ __forceinline__ void load(const T* row, int j, bool active, float* out) const {
        const int c = chunk(j);
        if (active && c < nchunk) {
            if constexpr (VECP) {
                unpack<D>(load16(row + (int64_t)c * V), out);
            } else {
                out[0] = load_scalar<D>(row + c);
            }
        } else {
#pragma unroll
            for (int k = 0; k < V; k++) out[k] = 0.0f;
        }
    }
    __device__ __forceinline__ void store(T* row, int j, bool active, const float* v) const {
        const int c = chunk(j);
        if (active && c < nchunk) {
            if constexpr (VECP) {
                store16(row + (int64_t)c * V, pack<D>(v));
            } else {
                store_scalar<D>(row + c, v[0]);
            }
        }
    }
};

// ------------------------------------------------------------------------------------------------
// ResidualAdd + LayerNorm.  v = x + r; mean = sum v / H; var = sum (v - mean)^2 / H (second
// sweep over the registers, not over HBM); y = (v - mean) * rstd * gamma + beta with
// rstd = 1 / sqrt(var + eps).  HAS_RES = false gives the plain LayerNorm (the second kernel of
// the unfused chain).
// ------------------------------------------------------------------------------------------------
template <DT D, bool VECP, int NV, int WPR, bool HAS_RES>
__global__ void __launch_bounds__(RowShape<WPR>::THREADS)
add_layernorm_kernel(const typename Elem<D>::T* x, const typename Elem<D>::T* res,
                     const typename Elem<D>::T* gamma, const typename Elem<D>::T* beta,
                     typename Elem<D>::T* y, int64_t rows, int hidden, float eps) {
    using S = RowSlice<D, VECP, NV, WPR>;
    constexpr int V = S::V;
    // Keep gamma/beta loads in flight with x and r when the slice is small; otherwise load
    // them after the statistics so that the register footprint stays bounded.
    constexpr bool PREFETCH_AFFINE = NV * V <= 32;
    __shared__ float lds_sum[8], lds_sq[8];

    const S s(hidden);
    const int64_t row = (int64_t)blockIdx.x * RowShape<WPR>::ROWS_PER_BLOCK + (threadIdx.x >> 6) / WPR;
    const bool active = row < rows;
    const auto* xr = x + row * hidden;
    const auto* rr = HAS_RES ? res + row * hidden : nullptr;
    auto* yr = y + row * hidden;

    float v[NV][V], rv[NV][V], g[NV][V], b[NV][V];
#pragma unroll
    for (int j = 0; j < NV; j++) {
        s.load(xr, j, active, v[j]);
        if constexpr (HAS_RES) s.load(rr, j, active, rv[j]);
        if constexpr (PREFETCH_AFFINE) {
            s.load(gamma, j, active, g[j]);
            s.load(beta, j, active, b[j]);
        }
    }

    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; j++) {
#pragma unroll
        for (int k = 0; k < V; k++) {
            if constexpr (HAS_RES) v[j][k] += rv[j][k];
            sum += v[j][k];  // zeros outside the row
        }
    }
    sum = row_allreduce<WPR>(sum, SumOp{}, lds_sum);
    const float mean = sum / (float)hidden;

    float sq = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; j++) {
        if (s.ok(j)) {
#pragma unroll
            for (int k = 0; k < V; k++) {
                const float d = v[j][k] - mean;
                sq = fmaf(d, d, sq);
            }
        }
    }
    sq = row_allreduce<WPR>(sq, SumOp{}, lds_sq);
    const float rstd = 1.0f / sqrtf(sq / (float)hidden + eps);

    if constexpr (!PREFETCH_AFFINE) {
#pragma unroll
        for (int j = 0; j < NV; j++) {
            s.load(gamma, j, active, g[j]);
            s.load(beta, j, active, b[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < NV; j++) {
        float o[V];
#pragma unroll
        for (int k = 0; k < V; k++) o[k] = fmaf((v[j][k] - mean) * rstd, g[j][k], b[j][k]);
        s.store(yr, j, active, o);
    }
}

// ------------------------------------------------------------------------------------------------
// Row softmax of scaled scores.  z = scale * x; m = max z; e = 2^((z - m) log2 e); y = e / sum e
// (as e times the correctly rounded reciprocal of the sum).
// ------------------------------------------------------------------------------------------------
template <DT D, bool VECP, int NV, int WPR>
__global__ void __launch_bounds__(RowShape<WPR>::THREADS)
softmax_rows_kernel(const typename Elem<D>::T* x, typename Elem<D>::T* y, int64_t rows, int cols,
                    float scale) {
    using S = RowSlice<D, VECP, NV, WPR>;
    constexpr int V = S::V;
    __shared__ float lds_max[8], lds_sum[8];

    const S s(cols);
    const int64_t row = (int64_t)blockIdx.x * RowShape<WPR>::ROWS_PER_BLOCK + (threadIdx.x >> 6) / WPR;
    const bool active = row < rows;
    const auto* xr = x + row * cols;
    auto* yr = y + row * cols;

    float z[NV][V];
#pragma unroll
    for (int j = 0; j < NV; j++) s.load(xr, j, active, z[j]);

    float m = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < NV; j++) {
#pragma unroll
        for (int k = 0; k < V; k++) {
            z[j][k] *= scale;
            if (s.ok(j)) m = fmaxf(m, z[j][k]);
        }
    }
    m = row_allreduce<WPR>(m, MaxOp{}, lds_max);

    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; j++) {
        if (s.ok(j)) {
#pragma unroll
            for (int k = 0; k < V; k++) {
                z[j][k] = exp2_fast((z[j][k] - m) * LOG2E);
                sum += z[j][k];
            }
        }
    }
    sum = row_allreduce<WPR>(sum, SumOp{}, lds_sum);
    const float inv = 1.0f / sum;

#pragma unroll
    for (int j = 0; j < NV; j++) {
        float o[V];
#pragma unroll
        for (int k = 0; k < V; k++) o[k] = z[j][k] * inv;
        s.store(yr, j, active, o);
    }
}

}  // namespace fuse
