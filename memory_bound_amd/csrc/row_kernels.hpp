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

#include <type_traits>

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

// Per-lane slice of one row: NV chunks of V elements.  Rows are read and written through buffer
// resources whose range is the row (empty for a row past the end), so chunks beyond the row
// load as zeros and are not stored, without branches.
template <DT D, bool VECP, int NV, int WPR> struct RowSlice {
    using T = typename Elem<D>::T;
    static constexpr int V = VECP ? Elem<D>::VEC : 1;

    int first_chunk;  // chunk index of j = 0 for this lane
    int nchunk;       // chunks in the row

    __device__ __forceinline__ RowSlice(int hidden) {
        const int lane = threadIdx.x & 63;
        const int wpos = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) % WPR;
        first_chunk = wpos * 64 + lane;
        nchunk = hidden / V;  // per-element path: V = 1
    }
    __device__ __forceinline__ int chunk(int j) const { return first_chunk + j * WPR * 64; }
    __device__ __forceinline__ bool ok(int j) const { return chunk(j) < nchunk; }

    // Raw bits of chunk j (a 128-bit word, or one element's bits on the per-element path).
    using Raw = typename std::conditional<VECP, uint4, uint32_t>::type;
    template <int AUX = AUX_DEFAULT> __device__ __forceinline__ Raw load_raw(rsrc_t r, int j) const {
        if constexpr (VECP) return bload16<AUX>(r, (uint32_t)chunk(j) * 16u);
        else if constexpr (sizeof(T) == 4) return bload_b32<AUX>(r, (uint32_t)chunk(j) * 4u);
        else return bload_b16<AUX>(r, (uint32_t)chunk(j) * 2u);
    }
    __device__ __forceinline__ void unpack_raw(const Raw& w, float* out) const {
        if constexpr (VECP) unpack<D>(w, out);
        else if constexpr (D == DT::F32) out[0] = __builtin_bit_cast(float, w);
        else if constexpr (D == DT::F16) out[0] = f16_to_f32(w);
        else out[0] = bf16_to_f32(w);
    }
    // One 32-bit word of a raw chunk (used to make later code depend on the load).
    __device__ __forceinline__ static uint32_t word0(const Raw& w) {
        if constexpr (VECP) return w.x;
        else return w;
    }

    // Chunk j as fp32 (zeros outside the resource's range).
    template <int AUX = AUX_DEFAULT> __device__ __forceinline__ void load(rsrc_t r, int j, float* out) const {
        if constexpr (VECP) unpack<D>(bload16<AUX>(r, (uint32_t)chunk(j) * 16u), out);
        else out[0] = bload_elem<D, AUX>(r, (uint32_t)chunk(j));
    }
    template <int AUX = AUX_DEFAULT> __device__ __forceinline__ void store_raw(rsrc_t r, int j, const uint4& w) const {
        bstore16<AUX>(r, (uint32_t)chunk(j) * 16u, w);
    }
    template <int AUX = AUX_DEFAULT> __device__ __forceinline__ void store(rsrc_t r, int j, const float* v) const {
        if constexpr (VECP) bstore16<AUX>(r, (uint32_t)chunk(j) * 16u, pack<D>(v));
        else bstore_elem<D, AUX>(r, (uint32_t)chunk(j), v[0]);
    }
};

// ------------------------------------------------------------------------------------------------
// ResidualAdd + LayerNorm.  v = x + r; mean = sum v / H; var = sum (v - mean)^2 / H (second
// sweep over the registers, not over HBM); y = (v - mean) * rstd * gamma + beta with
// rstd = 1 / sqrt(var + eps).  HAS_RES = false gives the plain LayerNorm (the second kernel of
// the unfused chain).
//
// EX adds the variants: y clamped below at 0 (LayerNorm + ReLU), and any of the pre-norm sum v
// (stored in the I/O type) and the per-row mean and population variance (fp32) as extra
// outputs.  A missing output gets an empty buffer resource, so its stores are dropped without a
// branch.
// ------------------------------------------------------------------------------------------------
template <class T> struct LnExtra {
    T* sum;       // [rows, hidden] pre-norm sum, or null
    float* mean;  // [rows], or null
    float* var;   // [rows], or null
    int relu;     // nonzero: y = max(y, 0) (a NaN stays NaN)
};

// Raw x and r chunks of one row, as loaded.
template <class S, int NV> struct LnRowIn {
    typename S::Raw wx[NV], wr[NV];
};

// Workgroup steps.  With KS = 1 a workgroup owns one block of rows (ROWS_PER_BLOCK rows).  With
// KS > 1 (launched only when the row fills every chunk of the slice) it walks KS blocks,
// blockIdx.x + k * gridDim.x for k < KS, keeping DEPTH of them in flight: the loads of block
// k + DEPTH go out as soon as block k is normalised and stored, and gamma/beta are loaded once
// for all KS blocks.  Fewer, longer-lived workgroups then spread each
// CU's reads over the kernel and interleave them with its writes instead of issuing every read at
// the start; the arithmetic per row is the same, so the results are bit-identical for every KS.
template <DT D, bool VECP, int NV, int WPR, bool HAS_RES, bool EX, int KS, int DEPTH>
__device__ __forceinline__ void add_layernorm_rows(const typename Elem<D>::T* x, const typename Elem<D>::T* res,
                                                   const typename Elem<D>::T* gamma,
                                                   const typename Elem<D>::T* beta, typename Elem<D>::T* y,
                                                   int64_t rows, int hidden, float eps,
                                                   const LnExtra<typename Elem<D>::T>& ex) {
    using S = RowSlice<D, VECP, NV, WPR>;
    using T = typename S::T;
    constexpr int V = S::V;
    static_assert(KS >= 1 && DEPTH >= 1 && DEPTH <= KS, "steps and depth");
    // Keep gamma/beta loads in flight with x and r when the slice is small; otherwise load
    // them after the statistics so that the register footprint stays bounded.
    constexpr bool PREFETCH_AFFINE = NV * V <= 64;
    static_assert(KS == 1 || PREFETCH_AFFINE, "multi-step workgroups hold gamma/beta in registers");
    __shared__ float lds_sum[8], lds_sq[8];

    const S s(hidden);
    const int row_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) / WPR;
    const uint32_t par_bytes = (uint32_t)hidden * (uint32_t)sizeof(T);
    const rsrc_t rg = make_rsrc(gamma, par_bytes);
    const rsrc_t rb = make_rsrc(beta, par_bytes);
    auto row_of = [&](int k) {
        return ((int64_t)blockIdx.x + (int64_t)k * gridDim.x) * RowShape<WPR>::ROWS_PER_BLOCK + row_in_block;
    };
    // x and r of step k; a row past the end gets empty resources (loads return zeros)
    auto issue = [&](int k, LnRowIn<S, NV>& in) {
        const int64_t row = row_of(k);
        const uint32_t row_bytes = row < rows ? par_bytes : 0u;
        const rsrc_t rx = make_rsrc(x + row * hidden, row_bytes);
        const rsrc_t rr = make_rsrc(HAS_RES ? res + row * hidden : x, HAS_RES ? row_bytes : 0u);
#pragma unroll
        for (int j = 0; j < NV; j++) {
            in.wx[j] = s.template load_raw<AUX_STREAM>(rx, j);
            if constexpr (HAS_RES) in.wr[j] = s.template load_raw<AUX_STREAM>(rr, j);
        }
    };

    // The first DEPTH steps' loads and gamma/beta are issued here; gamma and beta stay raw until
    // the normalisation.  One step (KS = 1): x and r first, then gamma/beta.  Left alone the
    // compiler sinks the gamma/beta loads below the reductions, which adds a cache round trip to
    // the row's critical path; a zero-valued data dependency of the row sum on one word of each
    // of them (masked with hidden >> 31, zero for any valid row length but unknown at compile
    // time) keeps them in flight together with x and r.  Several steps: gamma/beta first, as the
    // oldest loads they return before any row's data, and no dependency is needed.
    LnRowIn<S, NV> in[DEPTH];
    typename S::Raw wg[NV], wb[NV];
    auto issue_affine = [&]() {
        if constexpr (PREFETCH_AFFINE) {
#pragma unroll
            for (int j = 0; j < NV; j++) {
                wg[j] = s.load_raw(rg, j);
                wb[j] = s.load_raw(rb, j);
            }
        }
    };
    if constexpr (KS > 1) {
        issue_affine();
        issue(0, in[0]);
    } else {
        issue(0, in[0]);
        issue_affine();
    }
#pragma unroll
    for (int d = 1; d < DEPTH; d++) issue(d, in[d]);
    __builtin_amdgcn_sched_barrier(0);  // issue all of the above before anything below

    // 1 / hidden, correctly rounded; computed while the loads are in flight
    const float inv_h = 1.0f / (float)hidden;
    const float hf = (float)hidden;
    const float one = opaque_one();

#pragma unroll
    for (int k = 0; k < KS; k++) {
        const LnRowIn<S, NV>& cur = in[k % DEPTH];
        // Four steps (two workgroups per CU): a wave whose block has arrived runs its reductions,
        // stores and next loads ahead of the other wave on its SIMD, still waiting for data.
        // [2048,4096]: fp16 10.32-10.44 -> 10.13-10.31 us, bf16 10.3-10.4 -> 10.0-10.2 us
        // (alternating runs); with 2 steps ([16384,4096]) it measured 0.5 % slower, so only KS = 4.
        if constexpr (KS == 4) __builtin_amdgcn_s_setprio(1);
        const int64_t row = row_of(k);
        const uint32_t row_bytes = row < rows ? par_bytes : 0u;
        const rsrc_t ry = make_rsrc(y + row * hidden, row_bytes);
        const rsrc_t rsum = make_rsrc(EX && ex.sum ? ex.sum + row * hidden : y, EX && ex.sum ? row_bytes : 0u);

        float v[NV][V], g[NV][V], b[NV][V];
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < NV; j++) {
            s.unpack_raw(cur.wx[j], v[j]);
            if constexpr (HAS_RES) {
                float rv[V];
                s.unpack_raw(cur.wr[j], rv);
#pragma unroll
                for (int q = 0; q < V; q++) v[j][q] = fmaf(v[j][q], one, rv[q]);  // x + r
            }
#pragma unroll
            for (int q = 0; q < V; q++) sum += v[j][q];  // zeros outside the row
            if constexpr (EX) s.template store<AUX_STREAM>(rsum, j, v[j]);
        }
        if constexpr (PREFETCH_AFFINE && KS == 1) {
            uint32_t dep = 0;
#pragma unroll
            for (int j = 0; j < NV; j++) dep |= S::word0(wg[j]) | S::word0(wb[j]);
            sum += __builtin_bit_cast(float, dep & (uint32_t)(hidden >> 31));  // adds +0.0f
        }
        sum = row_allreduce<WPR>(sum, SumOp{}, lds_sum);
        // mean = sum / hidden correctly rounded: the product with the correctly rounded
        // reciprocal, then one correction by the exact remainder (Markstein's division step).  A
        // constant row thus has its value as mean exactly, whenever its sum is exact.
        const float q0 = sum * inv_h;
        const float mean = fmaf(fmaf(-q0, hf, sum), inv_h, q0);

        // deviations d = v - mean, kept for the output; chunks past the end of the row (only
        // when the row leaves some of the slice's chunks empty) are left out of the second sum
        // with a select
        float sq = 0.0f;
#pragma unroll
        for (int j = 0; j < NV; j++)
#pragma unroll
            for (int q = 0; q < V; q++) v[j][q] -= mean;
        // (several steps are launched only for rows that fill every chunk: no mask, no branch)
        if (KS > 1 || s.nchunk == NV * WPR * 64) {
#pragma unroll
            for (int j = 0; j < NV; j++)
#pragma unroll
                for (int q = 0; q < V; q++) sq = fmaf(v[j][q], v[j][q], sq);
        } else {
#pragma unroll
            for (int j = 0; j < NV; j++) {
                const bool in_row = s.ok(j);
#pragma unroll
                for (int q = 0; q < V; q++) {
                    const float d = in_row ? v[j][q] : 0.0f;
                    sq = fmaf(d, d, sq);
                }
            }
        }
        sq = row_allreduce<WPR>(sq, SumOp{}, lds_sq);
        const float var = sq * inv_h;
        const float rstd = __builtin_amdgcn_rsqf(var + eps);  // v_rsq_f32, within about 1 ulp
        if constexpr (EX) {
            // one lane of the row's first wave writes the statistics
            const bool leader =
                (threadIdx.x & 63) == 0 && (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) % WPR) == 0;
            const rsrc_t rm = make_rsrc(ex.mean ? ex.mean + row : (float*)y, ex.mean && row < rows ? 4u : 0u);
            const rsrc_t rv = make_rsrc(ex.var ? ex.var + row : (float*)y, ex.var && row < rows ? 4u : 0u);
            bstore_b32(rm, leader ? 0u : OOB, __builtin_bit_cast(uint32_t, mean));
            bstore_b32(rv, leader ? 0u : OOB, __builtin_bit_cast(uint32_t, var));
        }

        if constexpr (D == DT::F16 && VECP) {
            // f16 out: y = round_f16(d * rstd * gamma + beta) from the packed gamma/beta words,
            // one rounding per element, two instructions per pair
#pragma unroll
            for (int j = 0; j < NV; j++) {
                if constexpr (!PREFETCH_AFFINE) {
                    wg[j] = s.load_raw(rg, j);
                    wb[j] = s.load_raw(rb, j);
                }
                const uint32_t gw[4] = {wg[j].x, wg[j].y, wg[j].z, wg[j].w};
                const uint32_t bw[4] = {wb[j].x, wb[j].y, wb[j].z, wb[j].w};
                uint32_t u[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    u[i] = fma_mix_f16x2(v[j][2 * i] * rstd, v[j][2 * i + 1] * rstd, gw[i], bw[i]);
                    if constexpr (EX) {
                        // ReLU on the rounded values: a half with its sign set that is not a NaN
                        // (a negative number or -0) becomes +0
                        if (ex.relu) {
                            const uint32_t lo = u[i] & 0xffffu, hi = u[i] >> 16;
                            const bool zlo = (lo & 0x8000u) && (lo & 0x7fffu) <= 0x7c00u;
                            const bool zhi = (hi & 0x8000u) && (hi & 0x7fffu) <= 0x7c00u;
                            u[i] = (zlo ? 0u : lo) | ((zhi ? 0u : hi) << 16);
                        }
                    }
                }
                s.template store_raw<AUX_STREAM>(ry, j, make_uint4(u[0], u[1], u[2], u[3]));
            }
        } else {
#pragma unroll
            for (int j = 0; j < NV; j++) {
                if constexpr (PREFETCH_AFFINE) {
                    s.unpack_raw(wg[j], g[j]);
                    s.unpack_raw(wb[j], b[j]);
                } else {
                    s.load(rg, j, g[j]);
                    s.load(rb, j, b[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < NV; j++) {
                float o[V];
#pragma unroll
                for (int q = 0; q < V; q++) o[q] = fmaf(v[j][q] * rstd, g[j][q], b[j][q]);
                if constexpr (EX) {
#pragma unroll
                    for (int q = 0; q < V; q++) o[q] = (ex.relu && o[q] < 0.0f) ? 0.0f : o[q];
                }
                s.template store<AUX_STREAM>(ry, j, o);
            }
        }
        // Reuse of the exchange slots needs no extra barrier: every wave reads lds_sum of step k
        // before it reaches the lds_sq barrier of step k, and reads lds_sq of step k before it
        // reaches the lds_sum barrier of step k + 1.
        if (k + DEPTH < KS) issue(k + DEPTH, in[k % DEPTH]);
        if constexpr (KS == 4) __builtin_amdgcn_s_setprio(0);
    }
}

// KS row blocks per workgroup (1, 2 or 4), DEPTH = min(KS, 2) of them in flight.
template <DT D, bool VECP, int NV, int WPR, bool HAS_RES, int KS>
__global__ void __launch_bounds__(RowShape<WPR>::THREADS)
add_layernorm_kernel(const typename Elem<D>::T* x, const typename Elem<D>::T* res,
                     const typename Elem<D>::T* gamma, const typename Elem<D>::T* beta,
                     typename Elem<D>::T* y, int64_t rows, int hidden, float eps) {
    add_layernorm_rows<D, VECP, NV, WPR, HAS_RES, false, KS, (KS > 1 ? 2 : 1)>(
        x, res, gamma, beta, y, rows, hidden, eps, LnExtra<typename Elem<D>::T>{nullptr, nullptr, nullptr, 0});
}

template <DT D, bool VECP, int NV, int WPR, bool HAS_RES, int KS>
__global__ void __launch_bounds__(RowShape<WPR>::THREADS)
add_layernorm_ex_kernel(const typename Elem<D>::T* x, const typename Elem<D>::T* res,
                        const typename Elem<D>::T* gamma, const typename Elem<D>::T* beta,
                        typename Elem<D>::T* y, int64_t rows, int hidden, float eps,
                        LnExtra<typename Elem<D>::T> ex) {
    add_layernorm_rows<D, VECP, NV, WPR, HAS_RES, true, KS, (KS > 1 ? 2 : 1)>(x, res, gamma, beta, y, rows,
                                                                             hidden, eps, ex);
}

// ------------------------------------------------------------------------------------------------
// Row softmax of scaled scores.  z = scale * x; m = max z; e = 2^((z - m) log2 e); y = e / sum e
// (as e times the correctly rounded reciprocal of the sum).
// ------------------------------------------------------------------------------------------------
template <DT D, bool VECP, int NV, int WPR, bool FULL>
__global__ void __launch_bounds__(RowShape<WPR>::THREADS)
softmax_rows_kernel(const typename Elem<D>::T* x, typename Elem<D>::T* y, int64_t rows, int cols,
                    float scale) {
    using S = RowSlice<D, VECP, NV, WPR>;
    constexpr int V = S::V;
    __shared__ float lds_max[8], lds_sum[8];

    const S s(cols);
    const int64_t row = (int64_t)blockIdx.x * RowShape<WPR>::ROWS_PER_BLOCK +
                        __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) / WPR;
    const uint32_t row_bytes = row < rows ? (uint32_t)cols * (uint32_t)sizeof(typename S::T) : 0u;
    const rsrc_t rx = make_rsrc(x + row * cols, row_bytes);
    const rsrc_t ry = make_rsrc(y + row * cols, row_bytes);

    float z[NV][V];
#pragma unroll
    for (int j = 0; j < NV; j++) s.template load<AUX_STREAM>(rx, j, z[j]);

    // e_j = exp(s x_j - max_k s x_k) = 2^(c x_j - m) with c = s log2(e) and m = |c| max_k (sign(c) x_k),
    // which is c times the largest scaled value whatever the sign of s: one FMA per element.
    // Chunks past the row hold zeros and take no part in the max or the sum (FULL: there are none).
    const float c = scale * LOG2E;
    float mx = -__builtin_inff();
    if (c >= 0.0f) {
#pragma unroll
        for (int j = 0; j < NV; j++) {
            const bool in_row = FULL || s.ok(j);
#pragma unroll
            for (int k = 0; k < V; k++) mx = fmaxf(mx, in_row ? z[j][k] : -__builtin_inff());
        }
    } else {
#pragma unroll
        for (int j = 0; j < NV; j++) {
            const bool in_row = FULL || s.ok(j);
#pragma unroll
            for (int k = 0; k < V; k++) mx = fmaxf(mx, in_row ? -z[j][k] : -__builtin_inff());
        }
    }
    mx = row_allreduce<WPR>(mx, MaxOp{}, lds_max);
    const float m = fabsf(c) * mx;

    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; j++) {
        const bool in_row = FULL || s.ok(j);
#pragma unroll
        for (int k = 0; k < V; k++) {
            z[j][k] = __builtin_amdgcn_exp2f(fmaf(z[j][k], c, -m));
            sum += in_row ? z[j][k] : 0.0f;
        }
    }
    sum = row_allreduce<WPR>(sum, SumOp{}, lds_sum);
    const float inv = 1.0f / sum;

#pragma unroll
    for (int j = 0; j < NV; j++) {
        float o[V];
#pragma unroll
        for (int k = 0; k < V; k++) o[k] = z[j][k] * inv;
        s.template store<AUX_STREAM>(ry, j, o);
    }
}

// ------------------------------------------------------------------------------------------------
// Row cumsum + scale.  y_j = scale * (x_0 + ... + x_j).  The row's chunks are spread over the lanes
// as in the other row kernels (chunk c = (j * WPR + w) * 64 + lane), so the running sum is built
// in three levels: each lane scans its V-element chunks in registers; a DPP scan over the 64
// lanes turns the chunk totals into per-lane offsets within each (j, wave) block of 64 chunks; the
// block totals go through LDS and every wave adds the totals of the blocks before its own (blocks
// are ordered j first, then wave).
// ------------------------------------------------------------------------------------------------

// v moved by a DPP control, 0 where the lane has no source (or its row is masked off).
template <int CTRL, int ROW_MASK> __device__ __forceinline__ float dpp_zero(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                                                 0xF, true));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8 lanes within each
// 16-lane row (row_shr), then the gfx9 row broadcasts carry the row totals on: lane 15 of each
// row into the next row (rows 1 and 3), lane 31 into rows 2 and 3.
__device__ __forceinline__ float wave_inclusive_scan(float v) {
    v += dpp_zero<0x111, 0xF>(v);
    v += dpp_zero<0x112, 0xF>(v);
    v += dpp_zero<0x114, 0xF>(v);
    v += dpp_zero<0x118, 0xF>(v);
    v += dpp_zero<0x142, 0xA>(v);
    v += dpp_zero<0x143, 0xC>(v);
    return v;
}

// KS row blocks per workgroup (1, 2 or 4; more than 1 only when the row fills every chunk of the
// slice), blockIdx.x + k * gridDim.x for k < KS, with the raw loads of the next block in flight
// while a block is scanned and stored -- the workgroup steps of the LayerNorm kernel.  The block
// totals in LDS alternate between two buffers by step parity: a wave writes step k + 2's totals
// only after the barrier of step k + 1, which every wave reaches after reading step k's.  The
// arithmetic per row does not depend on KS, so the results are bit-identical for every KS.
template <DT D, bool VECP, int NV, int WPR, int KS>
__global__ void __launch_bounds__(RowShape<WPR>::THREADS)
cumsum_scale_kernel(const typename Elem<D>::T* x, typename Elem<D>::T* y, int64_t rows, int cols,
                    float scale) {
    using S = RowSlice<D, VECP, NV, WPR>;
    constexpr int V = S::V;
    constexpr int RPB = RowShape<WPR>::ROWS_PER_BLOCK;
    constexpr int DEPTH = KS > 1 ? 2 : 1;
    static_assert(KS == 1 || KS == 2 || KS == 4, "workgroup steps");
    __shared__ float lds_tot[KS > 1 ? 2 : 1][RPB][NV][WPR];

    const S s(cols);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rib = wave / WPR, wpos = wave % WPR;
    const uint32_t full_bytes = (uint32_t)cols * (uint32_t)sizeof(typename S::T);
    auto row_of = [&](int k) { return ((int64_t)blockIdx.x + (int64_t)k * gridDim.x) * RPB + rib; };
    // raw chunks of step k; a row past the end gets an empty resource (loads return zeros)
    typename S::Raw in[DEPTH][NV];
    auto issue = [&](int k, typename S::Raw (&w)[NV]) {
        const int64_t row = row_of(k);
        const rsrc_t rx = make_rsrc(x + row * cols, row < rows ? full_bytes : 0u);
#pragma unroll
        for (int j = 0; j < NV; j++) w[j] = s.template load_raw<AUX_STREAM>(rx, j);
    };
#pragma unroll
    for (int d = 0; d < DEPTH; d++) issue(d, in[d]);
    __builtin_amdgcn_sched_barrier(0);  // issue all of the above before anything below

#pragma unroll
    for (int k = 0; k < KS; k++) {
        const int64_t row = row_of(k);
        const rsrc_t ry = make_rsrc(y + row * cols, row < rows ? full_bytes : 0u);
        float v[NV][V];
#pragma unroll
        for (int j = 0; j < NV; j++) s.unpack_raw(in[k % DEPTH][j], v[j]);  // zeros past the row

        // chunk-local inclusive scans, then the exclusive scan of the chunk totals over the wave
        float excl[NV], btot[NV];
#pragma unroll
        for (int j = 0; j < NV; j++) {
#pragma unroll
            for (int e = 1; e < V; e++) v[j][e] += v[j][e - 1];
            const float inc = wave_inclusive_scan(v[j][V - 1]);
            excl[j] = dpp_zero<0x138, 0xF>(inc);  // wave_shr:1 -- lane 0 gets 0
            btot[j] = lane_read(inc, 63);
        }

        // offsets of the blocks before this wave's (j, wpos) blocks: the running sum `off` of the
        // block totals in (j, wave) order, taken for each j as it is stored, so that only one
        // chunk group's totals are live at a time
        float (&tot)[NV][WPR] = lds_tot[KS > 1 ? (k & 1) : 0][rib];
        if constexpr (WPR > 1) {
            if ((threadIdx.x & 63) == 0) {
#pragma unroll
                for (int j = 0; j < NV; j++) tot[j][wpos] = btot[j];
            }
            __syncthreads();
        }
        float off = 0.0f;

#pragma unroll
        for (int j = 0; j < NV; j++) {
            float pre = 0.0f;
            if constexpr (WPR == 1) {
                pre = off;
                off += btot[j];
            } else {
#pragma unroll
                for (int w = 0; w < WPR; w++) {
                    if (w == wpos) pre = off;
                    off += tot[j][w];
                }
            }
            const float base = pre + excl[j];
            float o[V];
#pragma unroll
            for (int e = 0; e < V; e++) o[e] = scale * (base + v[j][e]);
            s.template store<AUX_STREAM>(ry, j, o);
        }
        if (k + DEPTH < KS) issue(k + DEPTH, in[k % DEPTH]);
    }
}

}  // namespace fuse
