// swiglu.hip -- fused SwiGLU dual GEMM on the gfx950 matrix cores:
//   out[M,N] = SiLU(a[M,K] . b1[K,N]) * (a[M,K] . b2[K,N]), bf16 in and out, fp32 accumulation.
//
// Tiling.  A 256-thread workgroup (4 waves, 2 x 2) owns a 128 x 128 tile of out and keeps two
// fp32 accumulator sets, one per product: each wave holds 2 x 2 blocks of 32 x 32 for C1 and the
// same for C2 (v_mfma_f32_32x32x16_bf16, 16 fp32 per lane per block, 128 accumulators per lane).
// Per K step of 64 the workgroup stages one tile of a (128 x 64) and the matching tiles of b1 and
// b2 (64 x 128 each) in LDS; every A fragment read from LDS feeds one MFMA against b1 and one
// against b2, so the a tile is loaded from memory once for both products.
//
// Layouts.  The matrix cores want both operands with 8 consecutive k values per lane.  a is
// row-major [M,K] (k contiguous) and is copied to LDS as is.  b1 and b2 are row-major [K,N]
// (n contiguous); each thread loads an 8 (k) x 8 (n) block with eight 128-bit loads, transposes
// it in registers and writes eight 128-bit rows of the k-contiguous LDS tile Bt[n][k].  LDS rows
// are 64 bf16 (eight 16-byte chunks); chunk q of row r lives at chunk q ^ ((r ^ r>>3) & 7), which
// keeps the fragment reads (8 consecutive rows per 8 lanes) and the transposed writes (rows 8
// apart) free of bank conflicts.
//
// Pipeline.  LDS holds two stages (96 KiB).  While the MFMAs consume stage s, the registers
// loaded during the previous step are written to the other LDS stage and the global loads of
// step s + 2 are issued, so each K step needs one barrier and memory latency hides behind the
// matrix work.  One workgroup per CU (4 waves, one per SIMD) gets up to 512 registers per lane,
// enough for both accumulator sets without spilling.
//
// Scheduling.  Workgroups are dispatched round-robin over the 8 XCDs; the tile index is remapped
// so that each XCD owns a contiguous range of tiles, walked with M fastest, so that workgroups
// resident on one XCD share their b1/b2 column tiles in that XCD's L2.
#include "launch.hpp"
#include "stream_kernels.hpp"

namespace fuse {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64, THREADS = 256;
constexpr int NUM_XCD = 8;

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
// Element offset of 16-byte chunk q (0..7) of LDS row r.
__device__ __forceinline__ int lds_off(int r, int q) { return r * BK + ((q ^ swz(r)) << 3); }

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// 8 bf16 at element offset e0 of resource r; elements at index >= avail are zero (per-element
// path for operands whose rows are not 16-byte aligned).
__device__ __forceinline__ uint4 load8_guarded(rsrc_t r, uint32_t e0, int avail) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t lo = bload_b16(r, 2 * i < avail ? (e0 + 2 * i) * 2u : OOB);
        const uint32_t hi = bload_b16(r, 2 * i + 1 < avail ? (e0 + 2 * i + 1) * 2u : OOB);
        w[i] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// r[i] holds n = 0..7 of row k = i; returns o with o[j] holding k = 0..7 of column n = j.
__device__ __forceinline__ void transpose8x8(const uint4* r, uint4* o) {
#pragma unroll
    for (int j = 0; j < 8; j++) {
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; p++) {
            const uint32_t lo = word(r[2 * p], j >> 1), hi = word(r[2 * p + 1], j >> 1);
            w[p] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        o[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

struct Tile {
    int m0, n0;
};

// Bijective remap of the dispatch index so that XCD x (= bid % 8) gets a contiguous tile range.
__device__ __forceinline__ Tile tile_of(int bid, int tiles_m, int tiles_n) {
    const int nt = tiles_m * tiles_n;
    const int xcd = bid % NUM_XCD, slot = bid / NUM_XCD;
    const int q = nt / NUM_XCD, rem = nt % NUM_XCD;
    const int t = xcd * q + min(xcd, rem) + slot;
    return {(t % tiles_m) * BM, (t / tiles_m) * BN};
}

// Global -> registers for one K step.  The a resource spans the tile's valid rows and the b
// resource the step's valid k rows, so rows past M or K read as zeros; columns past K (a) or N (b)
// are sent to an offset outside the resource.  All loads are unconditional.
template <bool ALIGNED>
__device__ __forceinline__ void load_stage(const uint16_t* a, const uint16_t* b1, const uint16_t* b2,
                                           int M, int N, int K, int m0, int n0, int k0,
                                           uint4 (&ra)[4], uint4 (&rb)[8]) {
    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    {
        const int mrows = min(M - m0, BM);
        const rsrc_t r = make_rsrc(a + (int64_t)m0 * K, (uint32_t)mrows * (uint32_t)K * 2u);
        const int k = k0 + 8 * (t & 7);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t e0 = (uint32_t)((t >> 3) + 32 * i) * (uint32_t)K + (uint32_t)k;
            if (ALIGNED) ra[i] = bload16(r, k < K ? e0 * 2u : OOB);
            else ra[i] = load8_guarded(r, e0, K - k);
        }
    }
    {
        // waves 0-1 load b1, waves 2-3 load b2: the 8 x 8 block (kb, nb), kb = bt>>4, nb = bt&15
        const int krows = min(K - k0, BK);
        const rsrc_t r = make_rsrc((wave < 2 ? b1 : b2) + (int64_t)k0 * N, (uint32_t)krows * (uint32_t)N * 2u);
        const int bt = t & 127;
        const int n = n0 + 8 * (bt & 15), kb = 8 * (bt >> 4);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t e0 = (uint32_t)(kb + i) * (uint32_t)N + (uint32_t)n;
            if (ALIGNED) rb[i] = bload16(r, n < N ? e0 * 2u : OOB);
            else rb[i] = load8_guarded(r, e0, N - n);
        }
    }
}

__device__ __forceinline__ void store_stage(uint16_t* lds_a, uint16_t* lds_b1, uint16_t* lds_b2,
                                            const uint4 (&ra)[4], const uint4 (&rb)[8]) {
    const int t = threadIdx.x;
    {
        const int q = t & 7;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int r = (t >> 3) + 32 * i;
            *reinterpret_cast<uint4*>(lds_a + lds_off(r, q)) = ra[i];
        }
    }
    {
        const int bt = t & 127;
        uint16_t* lb = __builtin_amdgcn_readfirstlane(t >> 6) < 2 ? lds_b1 : lds_b2;
        const int nb = bt & 15, kb = bt >> 4;
        uint4 o[8];
        transpose8x8(rb, o);
#pragma unroll
        for (int j = 0; j < 8; j++) *reinterpret_cast<uint4*>(lb + lds_off(8 * nb + j, kb)) = o[j];
    }
}

template <bool ALIGNED, bool STORE_PRODUCTS>
__global__ void __launch_bounds__(THREADS, 1)
swiglu_kernel(const uint16_t* a, const uint16_t* b1, const uint16_t* b2, uint16_t* out,
              uint16_t* c1_out, uint16_t* c2_out, int M, int N, int K, int tiles_m, int tiles_n) {
    constexpr int STAGE = (BM + 2 * BN) * BK;  // bf16 elements per LDS stage
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

    const Tile tile = tile_of(blockIdx.x, tiles_m, tiles_n);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    floatx16 acc1[2][2], acc2[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc1[i][j][r] = acc2[i][j][r] = 0.0f;

    const int kt_n = (K + BK - 1) / BK;
    uint4 ra[4], rb[8];
    load_stage<ALIGNED>(a, b1, b2, M, N, K, tile.m0, tile.n0, 0, ra, rb);
    store_stage(lds, lds + BM * BK, lds + (BM + BN) * BK, ra, rb);
    if (kt_n > 1) load_stage<ALIGNED>(a, b1, b2, M, N, K, tile.m0, tile.n0, BK, ra, rb);
    __syncthreads();

    for (int kt = 0; kt < kt_n; kt++) {
        const uint16_t* la = lds + (kt & 1) * STAGE;
        const uint16_t* lb1 = la + BM * BK;
        const uint16_t* lb2 = lb1 + BN * BK;
#pragma unroll
        for (int kk = 0; kk < BK / 16; kk++) {
            const int q = 2 * kk + (lane >> 5);
            bf16x8 fa[2], fb1[2], fb2[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                fa[i] = *reinterpret_cast<const bf16x8*>(la + lds_off(64 * wm + 32 * i + (lane & 31), q));
                fb1[i] = *reinterpret_cast<const bf16x8*>(lb1 + lds_off(64 * wn + 32 * i + (lane & 31), q));
                fb2[i] = *reinterpret_cast<const bf16x8*>(lb2 + lds_off(64 * wn + 32 * i + (lane & 31), q));
            }
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    acc1[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb1[j], acc1[i][j], 0, 0, 0);
                    acc2[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb2[j], acc2[i][j], 0, 0, 0);
                }
        }
        if (kt + 1 < kt_n) {
            // stage kt+1 goes to the other buffer: nobody reads it until after the barrier below,
            // and its previous contents (stage kt-1) were consumed before the last barrier
            uint16_t* na = lds + ((kt + 1) & 1) * STAGE;
            store_stage(na, na + BM * BK, na + (BM + BN) * BK, ra, rb);
            if (kt + 2 < kt_n)
                load_stage<ALIGNED>(a, b1, b2, M, N, K, tile.m0, tile.n0, (kt + 2) * BK, ra, rb);
        }
        __syncthreads();
    }

    // Epilogue.  Block (i, j) element r of lane l sits at row 8 (r/4) + 4 (l/32) + r%4, column l%32.
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int col = tile.n0 + 64 * wn + 32 * j + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int row = tile.m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < M && col < N) {
                    const int64_t o = (int64_t)row * N + col;
                    const float c1 = acc1[i][j][r], c2 = acc2[i][j][r];
                    if constexpr (STORE_PRODUCTS) {
                        c1_out[o] = __builtin_bit_cast(uint16_t, (__bf16)c1);
                        c2_out[o] = __builtin_bit_cast(uint16_t, (__bf16)c2);
                    } else {
                        out[o] = __builtin_bit_cast(uint16_t, (__bf16)(silu(c1) * c2));
                    }
                }
            }
        }
}

template <bool STORE_PRODUCTS>
hipError_t launch(const void* a, const void* b1, const void* b2, void* out, void* c1, void* c2, int M,
                  int N, int K, hipStream_t stream) {
    const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    const bool aligned = (K % 8 == 0) && (N % 8 == 0) && (((uintptr_t)a | (uintptr_t)b1 | (uintptr_t)b2) & 15u) == 0;
    const dim3 grid((unsigned)(tm * tn)), block(THREADS);
    if (aligned)
        hipLaunchKernelGGL((swiglu_kernel<true, STORE_PRODUCTS>), grid, block, 0, stream, (const uint16_t*)a,
                           (const uint16_t*)b1, (const uint16_t*)b2, (uint16_t*)out, (uint16_t*)c1,
                           (uint16_t*)c2, M, N, K, tm, tn);
    else
        hipLaunchKernelGGL((swiglu_kernel<false, STORE_PRODUCTS>), grid, block, 0, stream, (const uint16_t*)a,
                           (const uint16_t*)b1, (const uint16_t*)b2, (uint16_t*)out, (uint16_t*)c1,
                           (uint16_t*)c2, M, N, K, tm, tn);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_swiglu(const void* a, const void* b1, const void* b2, void* out, int M, int N, int K,
                         hipStream_t stream) {
    if ((int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN) > 0x7fffffff) return hipErrorInvalidValue;
    return launch<false>(a, b1, b2, out, nullptr, nullptr, M, N, K, stream);
}

hipError_t launch_swiglu_unfused(const void* a, const void* b1, const void* b2, void* out, int M, int N,
                                 int K, void* c1, void* c2, hipStream_t stream) {
    if ((int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN) > 0x7fffffff) return hipErrorInvalidValue;
    hipError_t e = launch<true>(a, b1, b2, nullptr, c1, c2, M, N, K, stream);
    if (e != hipSuccess) return e;
    // second kernel of scheme A: out = SiLU(c1) * c2, element-wise over M*N
    const bool vec = (N % 8 == 0) && (((uintptr_t)out | (uintptr_t)c1 | (uintptr_t)c2) & 15u) == 0;
    return launch_ew<DT::BF16>(EwOp::SiluMul, vec, c1, c2, nullptr, out, (int64_t)M * N, N, 4, stream);
}

}  // namespace fuse
