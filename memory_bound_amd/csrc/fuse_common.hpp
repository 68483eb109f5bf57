// fuse_common.hpp -- device helpers shared by the libfuse kernels (gfx950, wave64).
//
// Storage types, 128-bit vector I/O, round-to-nearest-even conversions, wave-wide reductions
// built on DPP lane permutations and one ds_swizzle, and the scalar math the fused epilogues
// need (exp through v_exp_f32, the normal CDF through a published erfc approximation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fuse {

// ------------------------------------------------------------------------------------------------
// storage types
// ------------------------------------------------------------------------------------------------

enum class DT : int { F32 = 0, F16 = 1, BF16 = 2 };

template <DT D> struct Elem;
template <> struct Elem<DT::F32> { using T = float;    static constexpr int VEC = 4; };
template <> struct Elem<DT::F16> { using T = uint16_t; static constexpr int VEC = 8; };
template <> struct Elem<DT::BF16> { using T = uint16_t; static constexpr int VEC = 8; };

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
    // v_cvt_f16_f32 rounds to nearest even in the default mode
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    // v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// One 128-bit word <-> VEC fp32 values.
template <DT D> __device__ __forceinline__ void unpack(const uint4& w, float* out) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    if constexpr (D == DT::F32) {
#pragma unroll
        for (int i = 0; i < 4; i++) out[i] = __builtin_bit_cast(float, u[i]);
    } else if constexpr (D == DT::F16) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            out[2 * i] = f16_to_f32(u[i] & 0xffffu);
            out[2 * i + 1] = f16_to_f32(u[i] >> 16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            out[2 * i] = __builtin_bit_cast(float, u[i] << 16);
            out[2 * i + 1] = __builtin_bit_cast(float, u[i] & 0xffff0000u);
        }
    }
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

// VEC fp32 values -> one 128-bit word.  16-bit types convert in pairs (v_cvt_pk_f16_f32,
// v_cvt_pk_bf16_f32: one instruction per two elements, round to nearest even).
template <DT D> __device__ __forceinline__ uint4 pack(const float* v) {
    uint32_t u[4];
    if constexpr (D == DT::F32) {
#pragma unroll
        for (int i = 0; i < 4; i++) u[i] = __builtin_bit_cast(uint32_t, v[i]);
    } else if constexpr (D == DT::F16) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const half2_t h = {(_Float16)v[2 * i], (_Float16)v[2 * i + 1]};
            u[i] = __builtin_bit_cast(uint32_t, h);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const bf162_t h = {(__bf16)v[2 * i], (__bf16)v[2 * i + 1]};
            u[i] = __builtin_bit_cast(uint32_t, h);
        }
    }
    return make_uint4(u[0], u[1], u[2], u[3]);
}

// round_f16(a0 * g.lo + b.lo) | round_f16(a1 * g.hi + b.hi) << 16, with g and b packed f16 pairs:
// v_fma_mixlo_f16 / v_fma_mixhi_f16 widen g and b, fuse the multiply-add and round once, from the
// exact result, to f16 (fp32 fmaf then a conversion would round twice).
__device__ __forceinline__ uint32_t fma_mix_f16x2(float a0, float a1, uint32_t g, uint32_t b) {
    uint32_t r;
    asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[0,1,1]" : "=v"(r) : "v"(a0), "v"(g), "v"(b));
    asm("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel:[0,1,1] op_sel_hi:[0,1,1]" : "+v"(r) : "v"(a1), "v"(g), "v"(b));
    return r;
}

// 1.0f that the compiler cannot fold away: fmaf(a, one, b) is exactly a + b (a * 1 is exact, one
// rounding), but left as a fused multiply-add it merges with the f16 -> fp32 widening of a and b
// into one mixed-precision instruction (v_fma_mix_f32) instead of two conversions and an add.
__device__ __forceinline__ float opaque_one() {
    float one;
    asm("s_mov_b32 %0, 1.0" : "=s"(one));
    return one;
}

// ------------------------------------------------------------------------------------------------
// Raw buffer access.  A buffer resource covers [base, base + bytes); a load at an offset at or
// beyond `bytes` returns zero and a store there is dropped, in hardware.  Kernels therefore issue
// every load of a row or block unconditionally (no per-load branch, so the loads are all in
// flight together) and let the range check mask the tails.  Offsets are 32-bit and relative to
// the base, so bases are taken per row / per block / per tile.
// ------------------------------------------------------------------------------------------------

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int RSRC_WORD3 = 0x00020000;  // gfx9-family raw (untyped) buffer access
constexpr uint32_t OOB = 0x80000000u;   // an offset no resource covers: loads 0, stores dropped

// Cache policy of the buffer instructions (gfx94x/gfx950 encoding: bit 0 sc0, bit 1 nt, bit 4
// sc1).  Tensors that are read or written exactly once per launch use the non-temporal hint so
// that they do not displace reused data (per-column parameters, other rows' tiles) in L2 and
// the Infinity Cache; everything else uses the default policy.
#ifndef FUSE_STREAM_AUX
#define FUSE_STREAM_AUX 2
#endif
constexpr int AUX_DEFAULT = 0;
constexpr int AUX_STREAM = FUSE_STREAM_AUX;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, RSRC_WORD3);
}
template <int AUX = AUX_DEFAULT> __device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX));
}
template <int AUX = AUX_DEFAULT>
__device__ __forceinline__ void bstore16(rsrc_t r, uint32_t off, const uint4& v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, AUX);
}
template <int AUX = AUX_DEFAULT> __device__ __forceinline__ uint32_t bload_b16(rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, AUX);
}
template <int AUX = AUX_DEFAULT>
__device__ __forceinline__ void bstore_b16(rsrc_t r, uint32_t off, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, (int)off, 0, AUX);
}
template <int AUX = AUX_DEFAULT> __device__ __forceinline__ uint32_t bload_b32(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, AUX);
}
template <int AUX = AUX_DEFAULT>
__device__ __forceinline__ void bstore_b32(rsrc_t r, uint32_t off, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, AUX);
}

// One element at element index i of the buffer, widened to fp32 (0 outside the buffer).
template <DT D, int AUX = AUX_DEFAULT> __device__ __forceinline__ float bload_elem(rsrc_t r, uint32_t i) {
    if constexpr (D == DT::F32) return __builtin_bit_cast(float, bload_b32<AUX>(r, i * 4u));
    else if constexpr (D == DT::F16) return f16_to_f32(bload_b16<AUX>(r, i * 2u));
    else return bf16_to_f32(bload_b16<AUX>(r, i * 2u));
}
template <DT D, int AUX = AUX_DEFAULT> __device__ __forceinline__ void bstore_elem(rsrc_t r, uint32_t i, float v) {
    if constexpr (D == DT::F32) bstore_b32<AUX>(r, i * 4u, __builtin_bit_cast(uint32_t, v));
    else if constexpr (D == DT::F16) bstore_b16<AUX>(r, i * 2u, f32_to_f16(v));
    else bstore_b16<AUX>(r, i * 2u, f32_to_bf16(v));
}

// ------------------------------------------------------------------------------------------------
// wave64 all-reduce: every lane ends with the same value, combined in a fixed order.
//
// Steps 1-4 are DPP permutations inside each 16-lane row (partner lane 1, 2, mirrored half
// row, mirrored row); step 5 exchanges the two 16-lane rows of each half wave with ds_swizzle
// (xor 16); step 6 adds lane 0 and lane 32.  Each step pairs lanes symmetrically, so all lanes
// compute bit-identical results.
// ------------------------------------------------------------------------------------------------

enum : int {
    DPP_QUAD_XOR1 = 0xB1,          // quad_perm [1,0,3,2]
    DPP_QUAD_XOR2 = 0x4E,          // quad_perm [2,3,0,1]
    DPP_ROW_HALF_MIRROR = 0x141,   // lane i <- lane 7-i within 8
    DPP_ROW_MIRROR = 0x140,        // lane i <- lane 15-i within 16
    SWZ_XOR16 = 0x401F             // ds_swizzle bit mode: and 0x1f, or 0, xor 0x10
};

template <int CTRL> __device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                              0xF, 0xF, false));
}
__device__ __forceinline__ float swz_xor16(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), SWZ_XOR16));
}
__device__ __forceinline__ float lane_read(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

struct SumOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct MaxOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

template <class Op> __device__ __forceinline__ float wave_allreduce(float v, Op op) {
    v = op(v, dpp<DPP_QUAD_XOR1>(v));
    v = op(v, dpp<DPP_QUAD_XOR2>(v));
    v = op(v, dpp<DPP_ROW_HALF_MIRROR>(v));
    v = op(v, dpp<DPP_ROW_MIRROR>(v));
    v = op(v, swz_xor16(v));
    return op(lane_read(v, 0), lane_read(v, 32));
}

// ------------------------------------------------------------------------------------------------
// scalar math
// ------------------------------------------------------------------------------------------------

constexpr float LOG2E = 1.4426950408889634f;

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// e^x as 2^(x log2 e).
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * LOG2E); }

// Complementary error function for z >= 0 with fractional error below 1.2e-7 everywhere:
// the Chebyshev-fitted form of Press, Teukolsky, Vetterling & Flannery, "Numerical Recipes"
// (2nd ed., §6.2, routine erfcc): erfc(z) ~ t * exp(-z^2 + P(t)), t = 1 / (1 + z/2), with P a
// degree-9 polynomial.  Relative (not just absolute) accuracy matters here: the GELU tail
// t * Phi(t) for negative t is built from erfc directly.
__host__ __device__ __forceinline__ float erfc_nonneg(float z, float t) {
    float p = 0.17087277f;
    p = p * t + -0.82215223f;
    p = p * t + 1.48851587f;
    p = p * t + -1.13520398f;
    p = p * t + 0.27886807f;
    p = p * t + -0.18628806f;
    p = p * t + 0.09678418f;
    p = p * t + 0.37409196f;
    p = p * t + 1.00002368f;
    p = p * t + -1.26551223f;
    return p - z * z;  // exponent; caller applies t * exp(.)
}

// GELU(t) = t * Phi(t), Phi(t) = erfc(-t / sqrt 2) / 2.
__device__ __forceinline__ float gelu_erf(float t) {
    const float z = fabsf(t) * 0.70710678118654752f;
    const float w = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
    const float ec = w * exp_fast(erfc_nonneg(z, w));  // erfc(|t|/sqrt 2)
    const float half_ec = 0.5f * ec;
    const float phi = t < 0.0f ? half_ec : 1.0f - half_ec;
    return t * phi;
}

// SiLU(c) = c / (1 + e^-c).
__device__ __forceinline__ float silu(float c) {
    return c * __builtin_amdgcn_rcpf(1.0f + exp_fast(-c));
}

}  // namespace fuse
