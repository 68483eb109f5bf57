// swiglu.hip -- dual-product MFMA kernels on the gfx950 matrix cores, bf16 in and out, fp32
// accumulation:
//   SwiGLU            out = SiLU(a . b1) * (a . b2)          (a [M,K], b1 and b2 [K,N])
//   GEMM + bias + act y = act(x . W + bias)                  (each 256-column tile as two halves)
// and the split-K form and the unfused baselines built on the same kernels.
//
// Tiling.  A 256-thread workgroup (4 waves, 2 x 2) owns a 256 x 128 tile and keeps two fp32
// accumulator sets, one per product: each wave holds 4 x 2 blocks of 32 x 32 for C1 and the same
// for C2 (v_mfma_f32_32x32x16_bf16, 16 fp32 per lane per block, 256 accumulators per lane, held
// in AGPRs).  Per 16-deep k slice a wave reads 8 fragments from LDS (4 of a, 2 of b1, 2 of b2)
// for 16 MFMAs: every a fragment feeds one MFMA against b1 and one against b2, so the a tile is
// loaded from memory once for both products.
//
// Two kernels.  Full tiles (the workloads) take the direct kernel further down: operands go
// straight from memory into a ring of LDS stages and b is transposed at fragment-read time.
// Any other shape takes the general kernel below, which stages through registers:
//
// General kernel layouts.  The matrix cores want both operands with 8 consecutive k values per
// lane.  a is row-major [M,K] (k contiguous) and is copied to LDS as is.  b1 and b2 are
// row-major [K,N] (n contiguous); each thread loads an 8 (k) x 8 (n) block with eight 128-bit
// loads, transposes it in registers and writes eight 128-bit rows of the k-contiguous LDS tile
// Bt[n][k].  LDS rows are 64 bf16 (eight 16-byte chunks); chunk q of row r lives at chunk
// q ^ ((r ^ r>>3) & 7), which keeps the fragment reads (16 consecutive rows per 16 lanes, 64
// banks) and the transposed writes (rows 8 apart) free of bank conflicts.
//
// General kernel pipeline.  LDS holds two stages of 64 KiB.  While the MFMAs consume one stage,
// the registers loaded during the previous step are written to the other stage and the global
// loads of the step after are issued; fragments are double-buffered in registers so the LDS
// reads of the next k slice are in flight during the current slice's MFMAs.  One barrier per K
// step of 64; one workgroup per CU (one wave per SIMD, up to 512 registers per lane).
//
// Scheduling.  Workgroups are dispatched round-robin over the 8 XCDs; the tile index is remapped
// so that each XCD owns a contiguous range of tiles, walked with M fastest, so that workgroups
// resident on one XCD share their b1/b2 column tiles in that XCD's L2.
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "launch.hpp"
#include "stream_kernels.hpp"

namespace fuse {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 128, BK = 64, THREADS = 256;
constexpr int WM = 4, WN = 2;  // 32 x 32 blocks per wave along M and N (wave tile 128 x 64)
constexpr int NUM_XCD = 8;

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
// Element offset of 16-byte chunk q (0..7) of LDS row r.
__device__ __forceinline__ int lds_off(int r, int q) { return r * BK + ((q ^ swz(r)) << 3); }

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

// Bijective remap of the dispatch index so that XCD x (= bid % 8) gets a contiguous tile range,
// and tiles in that range ordered in groups of up to 8 row tiles by every column tile (row tile
// fastest): the 32 tiles an XCD's CUs run at once then share 8 a row panels and about 4 b column
// panels in its L2, whatever the row count.  With 8 row tiles or fewer this is plain column
// order.
__device__ __forceinline__ Tile tile_of(int bid, int tiles_m, int tiles_n, int bn_step) {
    const int nt = tiles_m * tiles_n;
    const int xcd = bid % NUM_XCD, slot = bid / NUM_XCD;
    const int q = nt / NUM_XCD, rem = nt % NUM_XCD;
    const int t = xcd * q + min(xcd, rem) + slot;
    constexpr int GM = 8;
    const int gm = min(GM, tiles_m);
    const int g = t / (gm * tiles_n), r = t - g * gm * tiles_n;
    const int rows = min(gm, tiles_m - g * gm);  // the last group may hold fewer row tiles
    return {(g * gm + r % rows) * BM, (r / rows) * bn_step};
}

// Global -> registers for one K step.  The a resource spans the tile's valid rows and the b
// resource the step's valid k rows, so rows past M or K read as zeros; columns past K (a) or N (b)
// are sent to an offset outside the resource.  All loads are unconditional.
template <bool ALIGNED>
__device__ __forceinline__ void load_stage(const uint16_t* a, const uint16_t* b1, const uint16_t* b2,
                                           int M, int N, int K, int nlim2, int m0, int n0, int k0,
                                           uint4 (&ra)[8], uint4 (&rb)[8]) {
    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    {
        const int mrows = min(M - m0, BM);
        const rsrc_t r = make_rsrc(a + (int64_t)m0 * K, (uint32_t)mrows * (uint32_t)K * 2u);
        const int k = k0 + 8 * (t & 7);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t e0 = (uint32_t)((t >> 3) + 32 * i) * (uint32_t)K + (uint32_t)k;
            if (ALIGNED) ra[i] = bload16(r, k < K ? e0 * 2u : OOB);
            else ra[i] = load8_guarded(r, e0, K - k);
        }
    }
    {
        // waves 0-1 load b1, waves 2-3 load b2: the 8 x 8 block (kb, nb), kb = bt>>4, nb = bt&15
        const int krows = min(K - k0, BK);
        // columns of b2 may end before N (when b2 is b1 shifted by 128 columns)
        const rsrc_t r = make_rsrc((wave < 2 ? b1 : b2) + (int64_t)k0 * N, (uint32_t)krows * (uint32_t)N * 2u);
        const int nlim = wave < 2 ? N : nlim2;
        const int bt = t & 127;
        const int n = n0 + 8 * (bt & 15), kb = 8 * (bt >> 4);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t e0 = (uint32_t)(kb + i) * (uint32_t)N + (uint32_t)n;
            if (ALIGNED) rb[i] = bload16(r, n < nlim ? e0 * 2u : OOB);
            else rb[i] = load8_guarded(r, e0, nlim - n);
        }
    }
}

__device__ __forceinline__ void store_stage(uint16_t* lds_a, uint16_t* lds_b1, uint16_t* lds_b2,
                                            const uint4 (&ra)[8], const uint4 (&rb)[8]) {
    const int t = threadIdx.x;
    {
        const int q = t & 7;
#pragma unroll
        for (int i = 0; i < 8; i++) {
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

struct Frags {
    bf16x8 a[WM], b1[WN], b2[WN];
};

// Fragments of k slice kk (16 deep) of one LDS stage for this wave.
__device__ __forceinline__ void read_frags(const uint16_t* la, const uint16_t* lb1, const uint16_t* lb2,
                                           int wm, int wn, int lane, int kk, Frags& f) {
    const int q = 2 * kk + (lane >> 5);
#pragma unroll
    for (int i = 0; i < WM; i++)
        f.a[i] = *reinterpret_cast<const bf16x8*>(la + lds_off(128 * wm + 32 * i + (lane & 31), q));
#pragma unroll
    for (int j = 0; j < WN; j++) {
        f.b1[j] = *reinterpret_cast<const bf16x8*>(lb1 + lds_off(64 * wn + 32 * j + (lane & 31), q));
        f.b2[j] = *reinterpret_cast<const bf16x8*>(lb2 + lds_off(64 * wn + 32 * j + (lane & 31), q));
    }
}

__device__ __forceinline__ void mfma_slice(const Frags& f, floatx16 (&acc1)[WM][WN], floatx16 (&acc2)[WM][WN]) {
#pragma unroll
    for (int i = 0; i < WM; i++)
#pragma unroll
        for (int j = 0; j < WN; j++) {
            acc1[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b1[j], acc1[i][j], 0, 0, 0);
            acc2[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b2[j], acc2[i][j], 0, 0, 0);
        }
}

// What one launch of the dual-product kernels computes.  Both products share the a tile; b1 and
// b2 are two [K, *] operands with row stride N: the two SwiGLU weight matrices, or one GEMM
// weight read as two adjacent 128-column halves of each 256-column tile (b2 = b1 + 128).
constexpr int MODE_SWIGLU = 0;    // out = SiLU(c1) * c2
constexpr int MODE_PRODUCTS = 1;  // c1, c2 stored as they are (first kernel of the unfused SwiGLU)
constexpr int MODE_BIAS = 2;      // MODE_BIAS + act: out = act(c + bias[col]) for both halves
constexpr int MODE_PART_DUAL = 8;  // split K: fp32 partial c1, c2 of this workgroup's K range
constexpr int MODE_PART_GEMM = 9;  // split K: fp32 partial of a GEMM tile (both halves, one plane)
constexpr int ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2, ACT_SILU = 3;

struct DualArgs {
    const uint16_t* a;
    const uint16_t* b1;
    const uint16_t* b2;
    uint16_t* out;         // [M, N]
    uint16_t* c1;          // products mode
    uint16_t* c2;
    const uint16_t* bias;  // bias mode: [N], or null for none
    int M, N, K;           // N is also the row stride of b1, b2 and every output
    int nlim2;             // columns of b2 that exist: N, or N - 128 when b2 = b1 + 128
    int tiles_m, tiles_n, bn_step;
    int ksteps;            // 32-deep K steps per workgroup (all of K unless split)
    float* part;           // split K: [splits][planes][M][N] fp32 partial products
    int tail;              // full-tile kernel: the last `tail` tiles run as `parts` row slices each
    int parts;             // 2 (128-row halves) or 4 (64-row quarters)
    int units;             // full-tile kernel: work units (whole tiles, then last-round slices; or
                           // tiles x splits), walked by workgroup b as b, b + grid, b + 2 grid, ...
};

template <int ACT> __device__ __forceinline__ float activation(float t) {
    if constexpr (ACT == ACT_RELU) return t < 0.0f ? 0.0f : t;  // a NaN stays NaN
    else if constexpr (ACT == ACT_GELU) return gelu_erf(t);
    else if constexpr (ACT == ACT_SILU) return silu(t);
    else return t;
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// A 4 x 4 block held by a quad of lanes -- lane s of the quad has column c + s, rows r .. r+3 in
// v0..v3 -- rearranged so that lane t of the quad holds row r + t, columns c .. c+3, as four bf16
// (RNE): one exchange with the neighbouring lane and one with the lane two over (DPP quad_perm),
// byte selects in between (v_perm_b32).
__device__ __forceinline__ u32x2 quad_rows_bf16(float v0, float v1, float v2, float v3, int lane) {
    const bf162_t h0 = {(__bf16)v0, (__bf16)v1}, h1 = {(__bf16)v2, (__bf16)v3};
    const uint32_t p0 = __builtin_bit_cast(uint32_t, h0), p1 = __builtin_bit_cast(uint32_t, h1);
    const uint32_t n0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p0, DPP_QUAD_XOR1, 0xF, 0xF, false);
    const uint32_t n1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p1, DPP_QUAD_XOR1, 0xF, 0xF, false);
    // even lane s: (own lo, neighbour lo) = rows r, r+2 of columns s, s+1; odd lane s: (neighbour
    // hi, own hi) = rows r+1, r+3 of columns s-1, s
    const uint32_t sel = (lane & 1) ? 0x03020706u : 0x05040100u;
    const uint32_t q0 = __builtin_amdgcn_perm(n0, p0, sel), q1 = __builtin_amdgcn_perm(n1, p1, sel);
    // lanes 0, 1 keep their row r / r+1 pair and take columns c+2, c+3 from lanes 2, 3, which in
    // turn take columns c, c+1 of rows r+2 / r+3
    const bool low = (lane & 2) == 0;
    const uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)(low ? q1 : q0), DPP_QUAD_XOR2, 0xF, 0xF, false);
    return low ? u32x2{q0, y} : u32x2{y, q1};
}

template <int AUX>
__device__ __forceinline__ void bstore8(rsrc_t r, uint32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, AUX);
}

// Stores the tile at (m0, n0) (64 WMT rows).  Block (i, j) element r of lane l sits at row
// 8 (r/4) + 4 (l/32) + r%4, column l%32 of the block; the wave's blocks start at row 32 WMT wm,
// column 64 wn of each product's 128-column tile.  Rows past M and columns past N fall outside
// the store resources.  QUAD (whole tiles, N a multiple of the tile width): each group of four
// rows goes out through quad_rows_bf16 as one 8-byte store per lane instead of four 2-byte ones.
// Measured at 2048x8960x1536: GEMM + bias + ReLU 70.6 -> 69.3 us per synchronised dispatch;
// SwiGLU 112.4 -> 110.2 us per synchronised dispatch and about 2.5 us faster over the back-to-back
// launches of the benchmark (faster in 7 of 8 interleaved pairs), where the clock sits at the
// power limit.
template <int MODE, int WMT = WM, bool QUAD = false>
__device__ __forceinline__ void store_tile(const DualArgs& p, const floatx16 (&acc1)[WMT][WN],
                                           const floatx16 (&acc2)[WMT][WN], int m0, int n0, int wm, int wn,
                                           int lane, int split) {
    constexpr int TM = 64 * WMT;  // tile rows: two waves of 32 * WMT rows
    const int mrows = min(p.M - m0, TM);
    const uint32_t out_bytes = (uint32_t)mrows * (uint32_t)p.N * 2u;
    // QUAD: lane l stores row 8 b + 4 (l/32) + l%4 of block (i, j), columns 4 ((l%32)/4) .. +3
    const int qrow = 4 * (lane >> 5) + (lane & 3), qcol = 4 * ((lane & 31) >> 2);
    if constexpr (QUAD && (MODE == MODE_PRODUCTS || MODE == MODE_SWIGLU)) {
        constexpr bool PROD = MODE == MODE_PRODUCTS;
        const rsrc_t ro = make_rsrc((PROD ? p.c1 : p.out) + (int64_t)m0 * p.N, out_bytes);
        const rsrc_t ro2 = make_rsrc(PROD ? p.c2 + (int64_t)m0 * p.N : p.out, PROD ? out_bytes : 0u);
#pragma unroll
        for (int i = 0; i < WMT; i++)
#pragma unroll
            for (int j = 0; j < WN; j++)
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    const int row = 32 * WMT * wm + 32 * i + 8 * b + qrow;
                    const int col = n0 + 64 * wn + 32 * j + qcol;
                    const uint32_t off = ((uint32_t)row * (uint32_t)p.N + (uint32_t)col) * 2u;
                    float v[4], w[4];
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const float c1 = acc1[i][j][4 * b + q], c2 = acc2[i][j][4 * b + q];
                        v[q] = PROD ? c1 : silu(c1) * c2;
                        w[q] = c2;
                    }
                    bstore8<AUX_STREAM>(ro, off, quad_rows_bf16(v[0], v[1], v[2], v[3], lane));
                    if constexpr (PROD) bstore8<AUX_STREAM>(ro2, off, quad_rows_bf16(w[0], w[1], w[2], w[3], lane));
                }
    } else if constexpr (QUAD && MODE >= MODE_BIAS && MODE < MODE_PART_DUAL) {
        constexpr int ACT = MODE - MODE_BIAS;
        const rsrc_t ro = make_rsrc(p.out + (int64_t)m0 * p.N, out_bytes);
        const rsrc_t rbias = make_rsrc(p.bias ? p.bias : p.out, p.bias ? (uint32_t)p.N * 2u : 0u);  // none: zeros
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int j = 0; j < WN; j++) {
                const int ccol = n0 + 128 * h + 64 * wn + 32 * j;  // first column of the block
                const float bv = bf16_to_f32(bload_b16(rbias, (uint32_t)(ccol + (lane & 31)) * 2u));
#pragma unroll
                for (int i = 0; i < WMT; i++)
#pragma unroll
                    for (int b = 0; b < 4; b++) {
                        const int row = 32 * WMT * wm + 32 * i + 8 * b + qrow;
                        const uint32_t off = ((uint32_t)row * (uint32_t)p.N + (uint32_t)(ccol + qcol)) * 2u;
                        float v[4];
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            const float c = h == 0 ? acc1[i][j][4 * b + q] : acc2[i][j][4 * b + q];
                            v[q] = activation<ACT>(c + bv);
                        }
                        bstore8<AUX_STREAM>(ro, off, quad_rows_bf16(v[0], v[1], v[2], v[3], lane));
                    }
            }
    } else if constexpr (MODE == MODE_PART_DUAL || MODE == MODE_PART_GEMM) {
        // fp32 partials of this K range (full tiles only): plane h of a dual product is c_h; a GEMM
        // keeps one plane, its halves at their own columns
        constexpr int PLANES = MODE == MODE_PART_DUAL ? 2 : 1;
        const int64_t plane = (int64_t)p.M * p.N;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            float* base = p.part + ((int64_t)split * PLANES + (PLANES == 2 ? h : 0)) * plane + (int64_t)m0 * p.N;
            const rsrc_t rp = make_rsrc(base, (uint32_t)TM * (uint32_t)p.N * 4u);
#pragma unroll
            for (int j = 0; j < WN; j++) {
                const int col = n0 + (PLANES == 2 ? 0 : 128 * h) + 64 * wn + 32 * j + (lane & 31);
#pragma unroll
                for (int i = 0; i < WMT; i++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int row = 32 * WMT * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        const float c = h == 0 ? acc1[i][j][r] : acc2[i][j][r];
                        // default cache policy: the reduction kernel reads these right back
                        bstore_b32(rp, ((uint32_t)row * (uint32_t)p.N + (uint32_t)col) * 4u,
                                   __builtin_bit_cast(uint32_t, c));
                    }
            }
        }
    } else if constexpr (MODE == MODE_SWIGLU || MODE == MODE_PRODUCTS) {
        constexpr bool PROD = MODE == MODE_PRODUCTS;
        const rsrc_t ro = make_rsrc((PROD ? p.c1 : p.out) + (int64_t)m0 * p.N, out_bytes);
        const rsrc_t ro2 = make_rsrc(PROD ? p.c2 + (int64_t)m0 * p.N : p.out, PROD ? out_bytes : 0u);
#pragma unroll
        for (int i = 0; i < WMT; i++)
#pragma unroll
            for (int j = 0; j < WN; j++) {
                const int col = n0 + 64 * wn + 32 * j + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int row = 32 * WMT * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    const uint32_t off = col < p.N ? ((uint32_t)row * (uint32_t)p.N + (uint32_t)col) * 2u : OOB;
                    const float c1 = acc1[i][j][r], c2 = acc2[i][j][r];
                    if constexpr (PROD) {
                        bstore_b16<AUX_STREAM>(ro, off, f32_to_bf16(c1));
                        bstore_b16<AUX_STREAM>(ro2, off, f32_to_bf16(c2));
                    } else {
                        bstore_b16<AUX_STREAM>(ro, off, f32_to_bf16(silu(c1) * c2));
                    }
                }
            }
    } else {
        constexpr int ACT = MODE - MODE_BIAS;
        const rsrc_t ro = make_rsrc(p.out + (int64_t)m0 * p.N, out_bytes);
        const rsrc_t rbias = make_rsrc(p.bias ? p.bias : p.out, p.bias ? (uint32_t)p.N * 2u : 0u);  // none: zeros
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int j = 0; j < WN; j++) {
                const int col = n0 + 128 * h + 64 * wn + 32 * j + (lane & 31);
                const bool in = col < p.N;
                const float bv = bf16_to_f32(bload_b16(rbias, in ? (uint32_t)col * 2u : OOB));
#pragma unroll
                for (int i = 0; i < WMT; i++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int row = 32 * WMT * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        const uint32_t off = in ? ((uint32_t)row * (uint32_t)p.N + (uint32_t)col) * 2u : OOB;
                        const float c = h == 0 ? acc1[i][j][r] : acc2[i][j][r];
                        bstore_b16<AUX_STREAM>(ro, off, f32_to_bf16(activation<ACT>(c + bv)));
                    }
            }
    }
}

template <bool ALIGNED, int MODE>
__global__ void __launch_bounds__(THREADS, 1)
swiglu_kernel(DualArgs p) {
    const uint16_t *a = p.a, *b1 = p.b1, *b2 = p.b2;
    const int M = p.M, N = p.N, K = p.K;
    constexpr int STAGE = (BM + 2 * BN) * BK;  // bf16 elements per LDS stage (64 KiB)
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

    const Tile tile = tile_of(blockIdx.x, p.tiles_m, p.tiles_n, p.bn_step);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    floatx16 acc1[WM][WN], acc2[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; i++)
#pragma unroll
        for (int j = 0; j < WN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc1[i][j][r] = acc2[i][j][r] = 0.0f;

    const int kt_n = (K + BK - 1) / BK;
    uint4 ra[8], rb[8];
    load_stage<ALIGNED>(a, b1, b2, M, N, K, p.nlim2, tile.m0, tile.n0, 0, ra, rb);
    store_stage(lds, lds + BM * BK, lds + (BM + BN) * BK, ra, rb);
    if (kt_n > 1) load_stage<ALIGNED>(a, b1, b2, M, N, K, p.nlim2, tile.m0, tile.n0, BK, ra, rb);
    __syncthreads();

    Frags f[2];
    read_frags(lds, lds + BM * BK, lds + (BM + BN) * BK, wm, wn, lane, 0, f[0]);
    for (int kt = 0; kt < kt_n; kt++) {
        const uint16_t* la = lds + (kt & 1) * STAGE;
        const uint16_t* lb1 = la + BM * BK;
        const uint16_t* lb2 = lb1 + BN * BK;
#pragma unroll
        for (int kk = 0; kk < BK / 16; kk++) {
            // LDS reads of the next slice overlap this slice's MFMAs
            if (kk + 1 < BK / 16) read_frags(la, lb1, lb2, wm, wn, lane, kk + 1, f[(kk + 1) & 1]);
            mfma_slice(f[kk & 1], acc1, acc2);
            if (kk == 1 && kt + 1 < kt_n) {
                // stage kt+1 goes to the other buffer: nobody reads it until after the barrier
                // below, and its previous contents (stage kt-1) were consumed before the last one
                uint16_t* na = lds + ((kt + 1) & 1) * STAGE;
                store_stage(na, na + BM * BK, na + (BM + BN) * BK, ra, rb);
                if (kt + 2 < kt_n)
                    load_stage<ALIGNED>(a, b1, b2, M, N, K, p.nlim2, tile.m0, tile.n0, (kt + 2) * BK, ra, rb);
            }
        }
        __syncthreads();
        if (kt + 1 < kt_n) {
            const uint16_t* na = lds + ((kt + 1) & 1) * STAGE;
            read_frags(na, na + BM * BK, na + (BM + BN) * BK, wm, wn, lane, 0, f[0]);
        }
    }

    store_tile<MODE>(p, acc1, acc2, tile.m0, tile.n0, wm, wn, lane, 0);
}

// ------------------------------------------------------------------------------------------------
// Full-tile kernel (M % 256 == 0, N % 128 == 0, K % 32 == 0, 16-byte aligned operands): operands go
// from memory straight into LDS with global_load_lds_dwordx4 (no VGPR staging, no LDS store
// instructions), through a ring of S stages of one 32-deep K step each, and b1/b2 are transposed at
// fragment-read time with ds_read_b64_tr_b16.
//
// ds_read_b64_tr_b16, per group of 16 lanes: if lane j reads the four 16-bit values D[j][0..3], lane
// i receives D[i/4][i%4], D[4+i/4][i%4], D[8+i/4][i%4], D[12+i/4][i%4].  With lane j reading
// n = nb + 4 (j%4) .. +3 of row k = kb + j/4 of an n-contiguous tile, lane i receives
// B[kb..kb+3][nb+i]: four consecutive k of one column, the matrix-core B operand layout.
//
// LDS layouts.  gfx950's LDS has 64 four-byte banks (256 bytes per cycle); a ds_read_b128 is
// served 16 lanes at a time and a ds_read_b64 32 lanes at a time.  XOR swizzles on 16-byte chunks
// keep both free of bank conflicts (the asynchronous writes fill 1 KiB per wave instruction in
// lane order and never conflict):
//   a tile  [256][32]: chunk q of row r at q ^ ((r >> 2) & 3) (four 64-byte rows per 256 bytes)
//   b tiles [32][128]: chunk q of row k at q ^ 4 (k & 3): the 64 bytes the two 16-lane groups of
//                      a transposed read take from each of four consecutive rows land in four
//                      different 64-byte quarters of the bank space
//
// Pipeline.  The fragments of a K step's first 16-deep slice are read during the previous step,
// so the matrix cores resume right after the step's barrier: in step kt the MFMAs of slice 0
// (registers f0, stage kt) run while slice 1 of stage kt is read into f1, and the MFMAs of slice 1
// run while slice 0 of stage kt+1 is read into f0.  Each LDS read is issued after an MFMA, in the
// order the next slice consumes them; the eight loads of stage kt+S-1 go out between the later
// MFMAs.  The barrier closing step kt therefore needs stages kt+1 and kt+2 complete (this wave's
// loads via vmcnt, everyone's via the barrier) and retires stage kt, whose buffer the loads of
// step kt+1 overwrite.
// ------------------------------------------------------------------------------------------------

// TM = 256 (the tile), 128 or 64 (a half or a quarter of a tile of the last round, see the kernel).
template <int TM> struct DirectCfgT {
    static constexpr int BKD = 32;
    static constexpr int A_ROW_BYTES = 64, A_CHUNKS = 4;
    static constexpr int A_BYTES = TM * A_ROW_BYTES;  // 16, 8 or 4 KiB
    static constexpr int B_BYTES = BKD * BN * 2;      // 8 KiB per matrix
    static constexpr int STAGE_BYTES = A_BYTES + 2 * B_BYTES;
    static constexpr int WMT = TM / 64;               // 32-row blocks per wave (wave tile TM/2 x 64)
    // asynchronous load instructions per wave per stage: TM/64 of a rows (TM/4 rows per wave),
    // 2 each of b1 and b2 rows
    static constexpr int A_LOADS = TM / 64;
    static constexpr int LOADS_PER_STAGE = A_LOADS + 4;
    __device__ static int a_phys(int r, int q) { return q ^ ((r >> 2) & 3); }
};
using DirectCfg = DirectCfgT<BM>;

__device__ __forceinline__ int b_phys(int k, int q) { return q ^ (4 * (k & 3)); }

// s_waitcnt with vmcnt = N and no wait on the other counters (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// Asynchronous 16-byte-per-lane load from global memory straight into LDS: lane L's 16 bytes land
// at lds + 16 L (M0 holds the wave's LDS base; one wait state between the M0 write and its use).
// Issued as inline assembly so that the compiler adds no waits of its own around it: the caller
// orders it with an explicit s_waitcnt vmcnt and a barrier before the data is read.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}

// Load slot `slot` of K step k0 into the stage at LDS address `base`: the first A_LOADS slots fill
// a rows [TM/4 w, TM/4 w + TM/4) of wave w (16 rows of 64 bytes per instruction), the last four
// four rows each of the b1 and b2 tiles, wave w taking rows [8 w, 8 w + 8).  Called with
// compile-time slot numbers from unrolled loops, so the branch folds away.
template <int TM>
__device__ __forceinline__ void dma_slot(int slot, const uint16_t* a, const uint16_t* b1, const uint16_t* b2,
                                         int N, int K, int m0, int n0, int k0, uint32_t base, int wave, int lane) {
    using C = DirectCfgT<TM>;
    if (slot < C::A_LOADS) {
        const int r0 = (TM / 4) * wave + 16 * slot;
        const int r = r0 + lane / C::A_CHUNKS, p = lane % C::A_CHUNKS;
        dma16(a + (int64_t)(m0 + r) * K + k0 + 8 * C::a_phys(r, p), base + r0 * C::A_ROW_BYTES);
    } else {
        const int j = slot - C::A_LOADS, i = j >> 1, mat = j & 1;
        const int k0r = 8 * wave + 4 * i;
        const int kr = k0r + lane / 16, p = lane % 16;
        const int64_t off = (int64_t)(k0 + kr) * N + n0 + 8 * b_phys(kr, p);
        dma16((mat == 0 ? b1 : b2) + off, base + C::A_BYTES + mat * C::B_BYTES + k0r * 256);
    }
}

// One 16-byte piece of a B fragment (32 columns from nb, k = kb .. kb + 15): transposed read t of 2.
__device__ __forceinline__ v4i16 b_frag_half(const char* bt, int nb, int kb, int lane, int t) {
    const int g = lane >> 4, j = lane & 15;
    const int n = nb + 16 * (g & 1) + 4 * (j & 3);
    const int q = n >> 3, half = (n >> 2) & 1;
    const int k = kb + 8 * (g >> 1) + 4 * t + (j >> 2);
    const char* p = bt + k * 256 + b_phys(k, q) * 16 + half * 8;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(__attribute__((address_space(3))) const char*)p);
}

__device__ __forceinline__ bf16x8 join(v4i16 lo, v4i16 hi) {
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int TM>
__device__ __forceinline__ bf16x8 a_frag(const char* st, int wm, int lane, int kk, int i) {
    using C = DirectCfgT<TM>;
    const int r = (TM / 2) * wm + 32 * i + (lane & 31), qa = 2 * kk + (lane >> 5);
    return *reinterpret_cast<const bf16x8*>(st + r * C::A_ROW_BYTES + C::a_phys(r, qa) * 16);
}

template <int WMT> struct FragsD {
    bf16x8 a[WMT], b1[WN], b2[WN];
};

// The 4 WMT MFMAs of one k slice on fragments `f`, interleaved with the LDS reads of the fragments
// `nx` of slice rk of stage `rs`, issued after the first MFMAs in the order the next slice uses
// them (a0, b1[0], b2[0], b1[1], b2[1], then the other a rows; each b fragment is two transposed
// reads), and with this slice's share of the next stage's load slots (from slot0) after the later
// MFMAs.
template <int TM>
__device__ __forceinline__ void slice_step(const FragsD<TM / 64>& f, FragsD<TM / 64>& nx, const char* rs, int rk,
                                           floatx16 (&acc1)[TM / 64][WN], floatx16 (&acc2)[TM / 64][WN],
                                           int slot0, int nslots, const uint16_t* a, const uint16_t* b1,
                                           const uint16_t* b2,
                                           int N, int K, int m0, int n0, int k0, uint32_t base, int wm, int wn,
                                           int wave, int lane) {
    using C = DirectCfgT<TM>;
    constexpr int WMT = C::WMT, NM = 4 * WMT;
    const char* bt1 = rs + C::A_BYTES;
    const char* bt2 = rs + C::A_BYTES + C::B_BYTES;
    // read unit u: 0 = a0; 1..8 = the transposed halves of b1[0], b2[0], b1[1], b2[1]; 9.. = a1, a2, ...
    auto read_unit = [&](int u, v4i16 (&h)[8]) {
        if (u == 0) {
            nx.a[0] = a_frag<TM>(rs, wm, lane, rk, 0);
        } else if (u <= 8) {
            const int q = u - 1, frag = q >> 1, t = q & 1;  // frag: b1[0], b2[0], b1[1], b2[1]
            h[q] = b_frag_half((frag & 1) ? bt2 : bt1, 64 * wn + 32 * (frag >> 1), 16 * rk, lane, t);
            if (t == 1) {
                const bf16x8 v = join(h[q - 1], h[q]);
                if (frag == 0) nx.b1[0] = v;
                else if (frag == 1) nx.b2[0] = v;
                else if (frag == 2) nx.b1[1] = v;
                else nx.b2[1] = v;
            }
        } else {
            nx.a[u - 8] = a_frag<TM>(rs, wm, lane, rk, u - 8);
        }
    };
    constexpr int NU = 8 + WMT;                  // read units per slice
    constexpr int UPM = (NU + NM - 1) / NM;      // read units after each of the first MFMAs
    v4i16 h[8];
#pragma unroll
    for (int m = 0; m < NM; m++) {
        const int i = m >> 2, j = (m >> 1) & 1;
        if (m & 1) acc2[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b2[j], acc2[i][j], 0, 0, 0);
        else acc1[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b1[j], acc1[i][j], 0, 0, 0);
#pragma unroll
        for (int u = m * UPM; u < (m + 1) * UPM; u++)
            if (u < NU) read_unit(u, h);
        // the load slots: for the full tile after MFMAs 9, 11, 13, 15; otherwise one after each of
        // the last nslots MFMAs (nslots <= NM)
        if constexpr (WMT == 4) {
            if (m >= 9 && (m & 1) && (m - 9) / 2 < nslots)
                dma_slot<TM>(slot0 + (m - 9) / 2, a, b1, b2, N, K, m0, n0, k0, base, wave, lane);
        } else {
            if (m >= NM - nslots)
                dma_slot<TM>(slot0 + m - (NM - nslots), a, b1, b2, N, K, m0, n0, k0, base, wave, lane);
        }
        // keep this order: the scheduler would otherwise bunch the reads and the MFMAs
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One workgroup's tile (TM rows from m0, 128-column products from n0) over K steps
// [kt0, kt0 + kt_n), ring of S stages in `lds`.
template <int TM, int S, int MODE>
__device__ __forceinline__ void direct_tile(const DualArgs& p, char* lds, int m0, int n0, int kt0, int kt_n,
                                            int split) {
    const uint16_t *a = p.a, *b1 = p.b1, *b2 = p.b2;
    const int N = p.N, K = p.K;
    using C = DirectCfgT<TM>;
    constexpr int LPS = C::LOADS_PER_STAGE, WMT = C::WMT;
    // The thread index passes through an empty asm statement, so everything derived from it (the
    // per-lane load, fragment and store offsets) is formed again for each tile.  Otherwise, when
    // one workgroup walks several tiles, those values are hoisted out of its tile loop and held
    // across it, and with the accumulators in the AGPRs that spills VGPRs to scratch.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    floatx16 acc1[WMT][WN], acc2[WMT][WN];
#pragma unroll
    for (int i = 0; i < WMT; i++)
#pragma unroll
        for (int j = 0; j < WN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc1[i][j][r] = acc2[i][j][r] = 0.0f;

    // Prologue: stages 0 .. S-2.  With fewer K steps than that, the missing stages reload the last
    // one into a buffer nobody reads, which keeps the prologue's vmcnt count fixed.
#pragma unroll
    for (int s = 0; s < S - 1; s++) {
        const uint32_t base = lds_addr(lds + s * C::STAGE_BYTES);
        const int k0 = (kt0 + min(s, kt_n - 1)) * C::BKD;
#pragma unroll
        for (int l = 0; l < LPS; l++) dma_slot<TM>(l, a, b1, b2, N, K, m0, n0, k0, base, wave, lane);
    }
    wait_vmcnt<LPS * (S - 3)>();  // stages 0 and 1 are in
    __syncthreads();
    FragsD<WMT> f0, f1;
#pragma unroll
    for (int i = 0; i < WMT; i++) f0.a[i] = a_frag<TM>(lds, wm, lane, 0, i);
#pragma unroll
    for (int j = 0; j < WN; j++) {
        f0.b1[j] = join(b_frag_half(lds + C::A_BYTES, 64 * wn + 32 * j, 0, lane, 0),
                        b_frag_half(lds + C::A_BYTES, 64 * wn + 32 * j, 0, lane, 1));
        f0.b2[j] = join(b_frag_half(lds + C::A_BYTES + C::B_BYTES, 64 * wn + 32 * j, 0, lane, 0),
                        b_frag_half(lds + C::A_BYTES + C::B_BYTES, 64 * wn + 32 * j, 0, lane, 1));
    }

    // Steps that load stage kt + S - 1, then the last S - 1 steps, which load nothing and wait for
    // every load still in flight (the stage they need next is the newest one).
    int kt = 0;
    for (; kt + S - 1 < kt_n; kt++) {
        const char* st = lds + (kt % S) * C::STAGE_BYTES;
        const char* sn = lds + ((kt + 1) % S) * C::STAGE_BYTES;
        const uint32_t nbase = lds_addr(lds + ((kt + S - 1) % S) * C::STAGE_BYTES);
        const int nk0 = (kt0 + kt + S - 1) * C::BKD;
        slice_step<TM>(f0, f1, st, 1, acc1, acc2, 0, LPS / 2, a, b1, b2, N, K, m0, n0, nk0, nbase, wm, wn, wave,
                       lane);
        slice_step<TM>(f1, f0, sn, 0, acc1, acc2, LPS / 2, LPS - LPS / 2, a, b1, b2, N, K, m0, n0, nk0, nbase, wm, wn, wave,
                       lane);
        wait_vmcnt<LPS * (S - 3)>();
        __syncthreads();
    }
    for (; kt < kt_n; kt++) {
        const char* st = lds + (kt % S) * C::STAGE_BYTES;
        const char* sn = lds + ((kt + 1) % S) * C::STAGE_BYTES;
        slice_step<TM>(f0, f1, st, 1, acc1, acc2, 0, 0, a, b1, b2, N, K, m0, n0, 0, 0, wm, wn, wave, lane);
        slice_step<TM>(f1, f0, sn, 0, acc1, acc2, 0, 0, a, b1, b2, N, K, m0, n0, 0, 0, wm, wn, wave, lane);
        wait_vmcnt<0>();
        __syncthreads();
    }
    wait_vmcnt<0>();  // no load may still be writing this workgroup's LDS when it ends

    store_tile<MODE, WMT, true>(p, acc1, acc2, m0, n0, wm, wn, lane, split);
}

// Work units.  Split K (p.tail = 0): unit (split, tile) = (bid / tiles, bid % tiles) covers K
// steps [split * ksteps, split * ksteps + ksteps) of its tile.  Otherwise tiles - tail units are
// a whole tile each, and parts * tail units the remaining tiles as 128-row halves or 64-row
// quarters: when the tiles leave a last round that fills few CUs, that round is spread over more
// of them.  Where the slices go in the unit order spreads the whole tiles' output bursts, which
// otherwise all fall at the end of a round: the GEMM modes (about one round of whole tiles) run
// the slices first, the SwiGLU kernels (two and more rounds) right after the first round of
// whole tiles, one per workgroup of the grid.  Measured at 2048x8960x1536 (three alternating
// rounds each), GEMM + bias + ReLU against slices last: 67.4-67.6 against 69.1-69.4 us per
// synchronised dispatch, 63.4-64.0 against 64.7-64.8 us over 200 launches; SwiGLU against
// slices last, on two machines: 106.5-106.7 against 109.0-109.2 and 112.1-112.8 against
// 112.6-113.2 us per dispatch, 104.6-105.3 against 105.3-105.9 and 107.4-108.0 against
// 108.6-109.1 us over 200 launches (slices first: 2.5 us faster per dispatch, 1.5 us slower
// sustained).  Whole tiles after the slices run as unit t + parts * tail, on the XCD the tile
// map assigns tile t when parts * tail is a multiple of 8 (96 and 192 at these shapes), on a
// neighbouring one otherwise.  A grid of one workgroup per unit puts the SwiGLU slices last.  One workgroup per unit, or, with more units than CUs, a grid of one
// workgroup per CU (rounded down to a multiple of 8) walking units b, b + grid, ..., so that unit u
// still runs on XCD u % 8, the one the tile map assumes.
// Last-round slice q (of tail tiles cut in P row slices each): its tile among the tail tiles and
// its part.  When the tail is a whole number of groups of 8 tiles, the P slices of a tile are 8
// units apart, so they run on one XCD (unit u runs on XCD u % 8) and its L2 fetches the tile's b
// columns once for all of them instead of once per slice; otherwise the slices of a tile are
// consecutive units.  Each slice still sums every k in the same order: results do not change.
struct Slice {
    int tile, part;
};
template <int P> __device__ __forceinline__ Slice slice_of(int q, int tail) {
    if (tail % NUM_XCD == 0) {
        constexpr int G = NUM_XCD * P;  // units of one group of 8 tiles
        return {(q / G) * NUM_XCD + q % NUM_XCD, (q / NUM_XCD) % P};
    }
    return {q / P, q % P};
}

// Work unit `bid` of the full-tile kernel, in the ring `lds`.
template <int S, int MODE>
__device__ __forceinline__ void direct_unit(const DualArgs& p, char* lds, int bid) {
    constexpr bool SLICES_FIRST = MODE >= MODE_BIAS && MODE < MODE_PART_DUAL;
    const int ntiles = p.tiles_m * p.tiles_n;
    const int kt_all = p.K / DirectCfg::BKD;
    const int head = ntiles - p.tail;
    // q: the unit's index among the last-round slices; -1 for a whole tile (index bid)
    int q = -1;
    if (p.tail != 0) {
        const int nsl = p.parts * p.tail;
        if (SLICES_FIRST) {
            if (bid < nsl) q = bid;
            else bid -= nsl;
        } else {
            // slices after the first round of whole tiles: one per workgroup of the grid
            const int w1 = min(head, (int)gridDim.x);
            if (bid >= w1 && bid < w1 + nsl) q = bid - w1;
            else if (bid >= w1 + nsl) bid -= nsl;
        }
    }
    if (q < 0) {
        const int split = bid / ntiles;
        const Tile tile = tile_of(bid - split * ntiles, p.tiles_m, p.tiles_n, p.bn_step);
        const int kt0 = split * p.ksteps;
        direct_tile<BM, S, MODE>(p, lds, tile.m0, tile.n0, kt0, min(p.ksteps, kt_all - kt0), split);
    } else if (p.parts == 2) {
        const Slice sl = slice_of<2>(q, p.tail);
        const Tile tile = tile_of(head + sl.tile, p.tiles_m, p.tiles_n, p.bn_step);
        direct_tile<BM / 2, S, MODE>(p, lds, tile.m0 + (BM / 2) * sl.part, tile.n0, 0, kt_all, 0);
    } else {
        const Slice sl = slice_of<4>(q, p.tail);
        const Tile tile = tile_of(head + sl.tile, p.tiles_m, p.tiles_n, p.bn_step);
        direct_tile<BM / 4, S, MODE>(p, lds, tile.m0 + (BM / 4) * sl.part, tile.n0, 0, kt_all, 0);
    }
}

// One workgroup per work unit.
template <int S, int MODE>
__global__ void __launch_bounds__(THREADS, 1)
swiglu_direct_kernel(DualArgs p) {
    static_assert(S >= 3 && S * DirectCfg::STAGE_BYTES <= 160 * 1024, "ring of 3 to 5 stages of 32 KiB");
    __shared__ __attribute__((aligned(1024))) char lds[S * DirectCfg::STAGE_BYTES];
    direct_unit<S, MODE>(p, lds, blockIdx.x);
}

// One workgroup per CU walking units b, b + grid, ... (shapes with more units than CUs).  A kernel
// of its own: the loop costs 17-20 spilled VGPRs of per-unit state (none inside the K loops), which
// the one-unit kernel above, used for split K and for shapes that fit in one round, does not pay.
template <int S, int MODE>
__global__ void __launch_bounds__(THREADS, 1)
swiglu_persist_kernel(DualArgs p) {
    static_assert(S >= 3 && S * DirectCfg::STAGE_BYTES <= 160 * 1024, "ring of 3 to 5 stages of 32 KiB");
    __shared__ __attribute__((aligned(1024))) char lds[S * DirectCfg::STAGE_BYTES];
    for (int bid = blockIdx.x; bid < p.units; bid += gridDim.x) {
        if (bid > (int)blockIdx.x) __syncthreads();  // the previous unit's last LDS reads are done
        direct_unit<S, MODE>(p, lds, bid);
    }
}

// ------------------------------------------------------------------------------------------------
// Split-K form.  The fused kernel's time has a floor: one workgroup walks all of K for its tile, so
// a shape with few tiles leaves most CUs idle for that whole walk.  Below a tile count set from
// the CU count, K is divided among several workgroups per tile; each stores its fp32 partial
// products and a second kernel sums them (in split order, so results are reproducible) and
// applies the epilogue.  This is the pages' trade between one kernel with fewer blocks and more
// blocks with an intermediate in memory, decided per shape on the device at hand.
// ------------------------------------------------------------------------------------------------
template <int MODE, int ACT>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* part, const uint16_t* bias, uint16_t* out, int64_t mn, int N, int splits) {
    constexpr int PLANES = MODE == MODE_PART_DUAL ? 2 : 1;
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;  // mn is a multiple of 4
    if (e >= mn) return;
    float s1[4] = {0.0f, 0.0f, 0.0f, 0.0f}, s2[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    // With many splits, the partials of U splits are loaded before any of them is added, so their
    // memory latencies overlap instead of adding up; the additions still go in split order, so the
    // result is the same bit for bit.  Measured per synchronised dispatch (SwiGLU auto plan):
    // 256x256x1536 (12 splits) 17.6 -> 15.7 us, 256x512x1536 (8 splits) 18.6 -> 17.7 us; with 3 or 4
    // splits, where the partials are larger and bandwidth sets the time, no gain (2048x1024x4096:
    // 55.0 -> 56.4 us), so only plans of 8 splits or more take this path.
    constexpr int U = 4;
    auto add = [&](const float4& v, const float4& w) {
        s1[0] += v.x, s1[1] += v.y, s1[2] += v.z, s1[3] += v.w;
        if constexpr (PLANES == 2) s2[0] += w.x, s2[1] += w.y, s2[2] += w.z, s2[3] += w.w;
    };
    int s = 0;
    for (; splits >= 2 * U && s + U <= splits; s += U) {
        float4 v[U], w[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const float* q = part + (int64_t)(s + u) * PLANES * mn + e;
            v[u] = *reinterpret_cast<const float4*>(q);
            if constexpr (PLANES == 2) w[u] = *reinterpret_cast<const float4*>(q + mn);
        }
#pragma unroll
        for (int u = 0; u < U; u++) add(v[u], w[u]);
    }
    for (; s < splits; s++) {
        const float* q = part + (int64_t)s * PLANES * mn + e;
        const float4 v = *reinterpret_cast<const float4*>(q);
        float4 w = v;
        if constexpr (PLANES == 2) w = *reinterpret_cast<const float4*>(q + mn);
        add(v, w);
    }
    uint32_t o[4];
    const int col = (int)(e % N);
#pragma unroll
    for (int k = 0; k < 4; k++) {
        if constexpr (MODE == MODE_PART_DUAL) o[k] = f32_to_bf16(silu(s1[k]) * s2[k]);
        else o[k] = f32_to_bf16(activation<ACT>(s1[k] + (bias ? bf16_to_f32(bias[col + k]) : 0.0f)));
    }
    *reinterpret_cast<uint2*>(out + e) = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
}

int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Ring depth of the full-tile kernel (FUSE_SWIGLU_STAGES, 3 to 5, overrides the default for tuning
// sweeps; five stages take all 160 KiB of LDS).  0: no full-tile kernel for this shape.
int direct_stages(int M, int N, int K, bool aligned, int tile_cols) {
    if (!aligned || M % BM != 0 || N % tile_cols != 0 || K % DirectCfg::BKD != 0) return 0;
    if (getenv("FUSE_SWIGLU_GENERAL") != nullptr) return 0;
    const char* s = getenv("FUSE_SWIGLU_STAGES");
    const int st = s ? atoi(s) : 4;
    return (st >= 3 && st <= 5) ? st : 4;
}

// One resident workgroup per CU walking the work units (b, b + grid, ...) instead of one
// workgroup per unit: no workgroup ends and launches between a CU's tiles.  Measured per
// synchronised dispatch at 2048x8960x1536: SwiGLU 113.2-114.4 -> 111.5-113.3 us median (mean
// 115.4-118.2 -> 112.3-113.0), GEMM + bias + ReLU 70.8-71.0 -> 70.4-70.6 us.  Results are
// bit-identical.  FUSE_SWIGLU_PERSIST=0 launches one workgroup per unit, for measurement.
bool persistent() {
    const char* e = getenv("FUSE_SWIGLU_PERSIST");
    return !(e && atoi(e) == 0);
}

// Tiles of the last round that the full-tile kernel runs in row slices, and how many slices:
// when the tiles take two or more rounds over the CUs and the last round fills at most half of
// them, its tiles run as halves, or as quarters when even those fill at most a quarter (560
// tiles on 256 CUs: 48 tiles as 192 quarters).  FUSE_SWIGLU_TAIL=0 turns it off and =2 limits it
// to halves, for measurement.
struct TailPlan {
    int tail, parts;
};
TailPlan tail_plan(int ntiles) {
    const char* e = getenv("FUSE_SWIGLU_TAIL");
    const int lim = e ? atoi(e) : 4;
    const int cus = cu_count();
    const int rounds = (ntiles + cus - 1) / cus;
    const int last = ntiles - (rounds - 1) * cus;
    if (rounds < 2 || lim < 2) return {0, 0};
    if (lim >= 4 && 4 * last <= cus) return {last, 4};
    if (2 * last <= cus) return {last, 2};
    return {0, 0};
}

// Launch of the dual-product kernels: `tile_cols` output columns per tile (128 for SwiGLU, whose
// two products cover the same 128 columns; 256 for a GEMM, whose two halves are adjacent).
template <int MODE>
hipError_t launch(DualArgs p, int tile_cols, hipStream_t stream) {
    p.tiles_m = (p.M + BM - 1) / BM;
    p.tiles_n = (p.N + tile_cols - 1) / tile_cols;
    p.bn_step = tile_cols;
    p.ksteps = p.K / DirectCfg::BKD;
    if ((int64_t)p.tiles_m * p.tiles_n > 0x7fffffff) return hipErrorInvalidValue;
    const bool aligned = (p.K % 8 == 0) && (p.N % 8 == 0) &&
                         (((uintptr_t)p.a | (uintptr_t)p.b1 | (uintptr_t)p.b2) & 15u) == 0;
    const int st = direct_stages(p.M, p.N, p.K, aligned, tile_cols);
    const TailPlan tp = st != 0 ? tail_plan(p.tiles_m * p.tiles_n) : TailPlan{0, 0};
    p.tail = tp.tail;
    p.parts = tp.parts;
    p.units = p.tiles_m * p.tiles_n + (tp.parts - 1) * tp.tail;
    const dim3 grid((unsigned)p.units), block(THREADS);
    const int cus = cu_count(), g = cus >= NUM_XCD ? cus / NUM_XCD * NUM_XCD : cus;
    // the persistent kernel with the default ring only; the other ring depths (tuning sweeps)
    // run one workgroup per unit
    if (st == 4 && persistent() && p.units > g) {
        hipLaunchKernelGGL((swiglu_persist_kernel<4, MODE>), dim3((unsigned)g), block, 0, stream, p);
        return hipGetLastError();
    }
    if (st == 3) hipLaunchKernelGGL((swiglu_direct_kernel<3, MODE>), grid, block, 0, stream, p);
    else if (st == 4) hipLaunchKernelGGL((swiglu_direct_kernel<4, MODE>), grid, block, 0, stream, p);
    else if (st == 5) hipLaunchKernelGGL((swiglu_direct_kernel<5, MODE>), grid, block, 0, stream, p);
    else if (aligned) hipLaunchKernelGGL((swiglu_kernel<true, MODE>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((swiglu_kernel<false, MODE>), grid, block, 0, stream, p);
    return hipGetLastError();
}

DualArgs dual_args(const void* a, const void* b1, const void* b2, int M, int N, int K) {
    DualArgs p{};
    p.a = (const uint16_t*)a;
    p.b1 = (const uint16_t*)b1;
    p.b2 = (const uint16_t*)b2;
    p.M = M;
    p.N = N;
    p.K = K;
    p.nlim2 = N;
    return p;
}

// Split of K for a shape (1 = the single fused kernel).  Full tiles only, and only when the tiles
// cover fewer than SPLIT_BELOW_CU_FRACTION of the CUs (one partial round).  Each split count sp,
// 2 .. K steps / MIN_SPLIT_STEPS, is priced against the single kernel by a cost model fitted to
// measurements on MI355X (256 CUs; 13 shapes, M 256-2048, K 512-4096, every split count from 1 to
// 16; with the current kernels the model's choice is within 1 % of the fastest forced split count
// at 10 of the 13 and 2-8 % off at the other three):
//   time(sp) = ceil(units / CUs) x ceil(K steps / sp) x STEP_US
//            + (sp > 1) x (SPLIT_FIXED_US + 8 x planes x sp x M x N bytes / SPLIT_BYTES_PER_US)
// with units = tiles x sp: the K steps each workgroup walks, plus the second kernel and the fp32
// partial products written and read back (planes = 2 for the dual product, 1 for a GEMM).  The
// cheapest wins; no plan's partials exceed SPLIT_MAX_BYTES, the size of the allocation-free entry
// point's array, so every chosen plan fits there.  FUSE_SPLITK forces a split count (1 = never
// split) for tuning sweeps.
constexpr double SPLIT_BELOW_CU_FRACTION = 0.5;
constexpr int MIN_SPLIT_STEPS = 4;
constexpr double STEP_US = 0.7;             // one 32-deep K step of a full tile
constexpr double SPLIT_FIXED_US = 4.0;      // the reduction kernel's launch and tail
constexpr double SPLIT_BYTES_PER_US = 5.0e6;
constexpr double SPLIT_MAX_BYTES = (double)SWIGLU_NOALLOC_SCRATCH_BYTES;

struct SplitPlan {
    int splits, ksteps;
};

SplitPlan split_plan(int M, int N, int K, int tile_cols, bool aligned) {
    const int kt = K / DirectCfg::BKD;
    if (direct_stages(M, N, K, aligned, tile_cols) == 0) return {1, kt};
    const int tiles = (M / BM) * (N / tile_cols);
    const char* f = getenv("FUSE_SPLITK");
    int sp;
    if (f && atoi(f) >= 1) {
        sp = atoi(f);
    } else {
        const int cus = cu_count();
        if (tiles >= SPLIT_BELOW_CU_FRACTION * cus) return {1, kt};
        const double planes = tile_cols == BN ? 2.0 : 1.0;
        const double mn = (double)M * (double)N;
        auto cost = [&](int s) {
            const int steps = (kt + s - 1) / s;
            const double rounds = (double)((tiles * s + cus - 1) / cus);
            double t = rounds * steps * STEP_US;
            if (s > 1) t += SPLIT_FIXED_US + 8.0 * planes * s * mn / SPLIT_BYTES_PER_US;
            return t;
        };
        sp = 1;
        double best = cost(1);
        for (int s = 2; s <= kt / MIN_SPLIT_STEPS; s++) {
            if ((double)s * planes * mn * 4.0 > SPLIT_MAX_BYTES) break;
            const double c = cost(s);
            if (c < best) {
                best = c;
                sp = s;
            }
        }
    }
    sp = max(1, min(sp, kt));
    if (sp < 2) return {1, kt};
    const int ksteps = (kt + sp - 1) / sp;
    return {(kt + ksteps - 1) / ksteps, ksteps};  // no empty split
}

size_t split_bytes(const SplitPlan& sp, int M, int N, int planes) {
    return sp.splits < 2 ? 0 : (size_t)sp.splits * planes * (size_t)M * (size_t)N * 4u;
}

bool aligned_args(const void* a, const void* b, int N, int K) {
    return (K % 8 == 0) && (N % 8 == 0) && ((((uintptr_t)a | (uintptr_t)b) & 15u) == 0);
}

template <int PMODE, int ACT>
hipError_t launch_split(DualArgs p, int tile_cols, const SplitPlan& sp, float* part, hipStream_t stream) {
    p.tiles_m = p.M / BM;
    p.tiles_n = p.N / tile_cols;
    p.bn_step = tile_cols;
    p.ksteps = sp.ksteps;
    p.part = part;
    const int st = direct_stages(p.M, p.N, p.K, true, tile_cols);
    p.units = p.tiles_m * p.tiles_n * sp.splits;
    const dim3 grid((unsigned)p.units), block(THREADS);
    if (st == 3) hipLaunchKernelGGL((swiglu_direct_kernel<3, PMODE>), grid, block, 0, stream, p);
    else if (st == 5) hipLaunchKernelGGL((swiglu_direct_kernel<5, PMODE>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((swiglu_direct_kernel<4, PMODE>), grid, block, 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t mn = (int64_t)p.M * p.N;
    hipLaunchKernelGGL((splitk_reduce_kernel<PMODE, ACT>), dim3((unsigned)((mn / 4 + 255) / 256)), dim3(256), 0,
                       stream, (const float*)part, p.bias, p.out, mn, p.N, sp.splits);
    return hipGetLastError();
}

}  // namespace

// The split form also needs a 16-byte aligned output (the reduction stores 8 bytes per thread).
int swiglu_auto_splits(int M, int N, int K, const void* a, const void* b1, const void* b2, const void* out,
                       size_t* ws_bytes) {
    const SplitPlan sp =
        split_plan(M, N, K, BN, aligned_args(a, b1, N, K) && ((((uintptr_t)b2) | (uintptr_t)out) & 15u) == 0);
    if (ws_bytes) *ws_bytes = split_bytes(sp, M, N, 2);
    return sp.splits;
}

int gemm_auto_splits(int M, int N, int K, const void* x, const void* w, const void* y, size_t* ws_bytes) {
    const SplitPlan sp = split_plan(M, N, K, 2 * BN, aligned_args(x, w, N, K) && ((uintptr_t)y & 15u) == 0);
    if (ws_bytes) *ws_bytes = split_bytes(sp, M, N, 1);
    return sp.splits;
}

hipError_t launch_swiglu_auto(const void* a, const void* b1, const void* b2, void* out, int M, int N, int K,
                              void* ws, hipStream_t stream) {
    const SplitPlan sp =
        split_plan(M, N, K, BN, aligned_args(a, b1, N, K) && ((((uintptr_t)b2) | (uintptr_t)out) & 15u) == 0);
    if (sp.splits < 2) return launch_swiglu(a, b1, b2, out, M, N, K, stream);
    DualArgs p = dual_args(a, b1, b2, M, N, K);
    p.out = (uint16_t*)out;
    return launch_split<MODE_PART_DUAL, ACT_NONE>(p, BN, sp, (float*)ws, stream);
}

// ------------------------------------------------------------------------------------------------
// Allocation-free split-K SwiGLU, for callers that cannot allocate device memory.  The fp32 partial
// products go to `scratch`, a fixed array of the library, instead of a caller workspace.  Its size
// covers every split plan the library chooses: the split planner keeps the partials within it
// (SPLIT_MAX_BYTES); only a split count forced through FUSE_SPLITK can need more.  Each
// device holds its own copy from the first call on it until the process ends.  Every call on a
// device shares that copy, so calls that overlap on one device (two streams, two threads) race
// on it.  Every partial a launch reads is written earlier in the same launch, so nothing needs
// clearing between calls.
// ------------------------------------------------------------------------------------------------
static __device__ __align__(256) float scratch[SWIGLU_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int MAX_DEVICES = 64;
std::atomic<void*> scratch_addr[MAX_DEVICES];
std::mutex scratch_mu;

// Device address of `scratch` on the current device, looked up once per device.  The array's
// name in host code is only a stand-in for the symbol; this address is what kernels get.
hipError_t scratch_on_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    void* p = scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(scratch_mu);
        p = scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}
}  // namespace

size_t swiglu_noalloc_need(int M, int N, int K, const void* a, const void* b1, const void* b2, const void* out) {
    size_t need = 0;
    swiglu_auto_splits(M, N, K, a, b1, b2, out, &need);
    return need;
}

hipError_t launch_swiglu_auto_noalloc(const void* a, const void* b1, const void* b2, void* out, int M, int N, int K,
                                      hipStream_t stream) {
    const SplitPlan sp =
        split_plan(M, N, K, BN, aligned_args(a, b1, N, K) && ((((uintptr_t)b2) | (uintptr_t)out) & 15u) == 0);
    if (sp.splits < 2) return launch_swiglu(a, b1, b2, out, M, N, K, stream);
    if (split_bytes(sp, M, N, 2) > SWIGLU_NOALLOC_SCRATCH_BYTES) return hipErrorInvalidValue;  // checked by the caller
    void* part = nullptr;
    const hipError_t e = scratch_on_current_device(&part);
    if (e != hipSuccess) return e;
    DualArgs p = dual_args(a, b1, b2, M, N, K);
    p.out = (uint16_t*)out;
    return launch_split<MODE_PART_DUAL, ACT_NONE>(p, BN, sp, (float*)part, stream);
}

hipError_t launch_gemm_bias_act_auto(const void* x, const void* w, const void* bias, void* y, int M, int N, int K,
                                     int act, void* ws, hipStream_t stream) {
    const SplitPlan sp = split_plan(M, N, K, 2 * BN, aligned_args(x, w, N, K) && ((uintptr_t)y & 15u) == 0);
    if (sp.splits < 2) return launch_gemm_bias_act(x, w, bias, y, M, N, K, act, stream);
    DualArgs p = dual_args(x, w, (const uint16_t*)w + 128, M, N, K);
    p.out = (uint16_t*)y;
    p.bias = (const uint16_t*)bias;
    p.nlim2 = N - 128;
    switch (act) {
        case ACT_NONE: return launch_split<MODE_PART_GEMM, ACT_NONE>(p, 2 * BN, sp, (float*)ws, stream);
        case ACT_RELU: return launch_split<MODE_PART_GEMM, ACT_RELU>(p, 2 * BN, sp, (float*)ws, stream);
        case ACT_GELU: return launch_split<MODE_PART_GEMM, ACT_GELU>(p, 2 * BN, sp, (float*)ws, stream);
        case ACT_SILU: return launch_split<MODE_PART_GEMM, ACT_SILU>(p, 2 * BN, sp, (float*)ws, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_swiglu(const void* a, const void* b1, const void* b2, void* out, int M, int N, int K,
                         hipStream_t stream) {
    DualArgs p = dual_args(a, b1, b2, M, N, K);
    p.out = (uint16_t*)out;
    return launch<MODE_SWIGLU>(p, BN, stream);
}

hipError_t launch_swiglu_unfused(const void* a, const void* b1, const void* b2, void* out, int M, int N,
                                 int K, void* c1, void* c2, hipStream_t stream) {
    DualArgs p = dual_args(a, b1, b2, M, N, K);
    p.c1 = (uint16_t*)c1;
    p.c2 = (uint16_t*)c2;
    hipError_t e = launch<MODE_PRODUCTS>(p, BN, stream);
    if (e != hipSuccess) return e;
    // second kernel of scheme A: out = SiLU(c1) * c2, element-wise over M*N
    const bool vec = (N % 8 == 0) && (((uintptr_t)out | (uintptr_t)c1 | (uintptr_t)c2) & 15u) == 0;
    return launch_ew<DT::BF16>(EwOp::SiluMul, vec, c1, c2, nullptr, out, (int64_t)M * N, N, 4, stream);
}

// GEMM + bias + activation on the same kernels: each 256 x 256 output tile is computed as two
// 128-column halves, the second product reading the weight shifted by 128 columns.
hipError_t launch_gemm_bias_act(const void* x, const void* w, const void* bias, void* y, int M, int N, int K,
                                int act, hipStream_t stream) {
    DualArgs p = dual_args(x, w, (const uint16_t*)w + 128, M, N, K);
    p.out = (uint16_t*)y;
    p.bias = (const uint16_t*)bias;
    p.nlim2 = N > 128 ? N - 128 : 0;
    switch (act) {
        case ACT_NONE: return launch<MODE_BIAS + ACT_NONE>(p, 2 * BN, stream);
        case ACT_RELU: return launch<MODE_BIAS + ACT_RELU>(p, 2 * BN, stream);
        case ACT_GELU: return launch<MODE_BIAS + ACT_GELU>(p, 2 * BN, stream);
        case ACT_SILU: return launch<MODE_BIAS + ACT_SILU>(p, 2 * BN, stream);
    }
    return hipErrorInvalidValue;
}

// Unfused chain of [P1] §二.1's example: the GEMM kernel stores C, a bias kernel stores T = C + b,
// an activation kernel writes y (stored intermediates in bf16; no bias skips the bias kernel, no
// activation the activation kernel).
hipError_t launch_gemm_bias_act_unfused(const void* x, const void* w, const void* bias, void* y, int M, int N,
                                        int K, int act, void* c, void* t, hipStream_t stream) {
    const bool last_gemm = !bias && act == ACT_NONE;
    hipError_t e = launch_gemm_bias_act(x, w, nullptr, last_gemm ? y : c, M, N, K, ACT_NONE, stream);
    if (e != hipSuccess || last_gemm) return e;
    const int64_t n = (int64_t)M * N;
    const void* src = c;
    if (bias) {
        void* dst = act == ACT_NONE ? y : t;
        const bool vec = (N % 8 == 0) && (((uintptr_t)src | (uintptr_t)bias | (uintptr_t)dst) & 15u) == 0;
        e = launch_ew<DT::BF16>(EwOp::BiasAdd, vec, src, nullptr, bias, dst, n, N, 4, stream);
        if (e != hipSuccess || act == ACT_NONE) return e;
        src = t;
    }
    const bool vec = (N % 8 == 0) && (((uintptr_t)src | (uintptr_t)y) & 15u) == 0;
    const EwOp op = act == ACT_RELU ? EwOp::Relu : act == ACT_GELU ? EwOp::Gelu : EwOp::Silu;
    return launch_ew<DT::BF16>(op, vec, src, nullptr, nullptr, y, n, N, 4, stream);
}

}  // namespace fuse
