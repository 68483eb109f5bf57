// copy.hip -- plain device copy used to calibrate the roofline (achievable streaming bandwidth and
// the scale of the hardware byte counters), the matrix-core calibration kernel (achievable MFMA
// rate), and the empty kernel of the launch-cost probe.
#include "launch.hpp"
#include "stream_kernels.hpp"

namespace fuse {

// ------------------------------------------------------------------------------------------------
// Plain copy (roofline calibration): 16-byte chunks, CH per thread, plus a byte tail kernel.
// ------------------------------------------------------------------------------------------------
// Workgroup b copies 16-byte chunks [b*256*CH, (b+1)*256*CH) through buffer resources that end
// at the copy's end: every load is issued before the first store, no per-chunk branch.
template <int CH>
__global__ void __launch_bounds__(256)
copy16_kernel(const uint4* src, uint4* dst, uint64_t n16) {
    const uint64_t first = (uint64_t)blockIdx.x * (256u * CH);
    const uint64_t left = n16 - first;
    const uint32_t bytes = (uint32_t)(left < 256u * CH ? left : 256u * CH) * 16u;
    const rsrc_t rs = make_rsrc(src + first, bytes);
    const rsrc_t rd = make_rsrc(dst + first, bytes);
    uint4 v[CH];
#pragma unroll
    for (int j = 0; j < CH; j++) v[j] = bload16<AUX_STREAM>(rs, ((uint32_t)(j * 256) + threadIdx.x) * 16u);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < CH; j++) bstore16<AUX_STREAM>(rd, ((uint32_t)(j * 256) + threadIdx.x) * 16u, v[j]);
}

__global__ void __launch_bounds__(256)
copy_bytes_kernel(const uint8_t* src, uint8_t* dst, uint64_t n) {
    const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    constexpr int CH = 4;
    const bool a16 = ((((uintptr_t)src) | ((uintptr_t)dst)) & 15u) == 0;
    const uint64_t n16 = a16 ? bytes / 16 : 0;
    if (n16) {
        const uint64_t per_block = 256ull * CH;
        hipLaunchKernelGGL((copy16_kernel<CH>), dim3((unsigned)((n16 + per_block - 1) / per_block)), dim3(256),
                           0, stream, (const uint4*)src, (uint4*)dst, n16);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const uint64_t done = n16 * 16, tail = bytes - done;
    if (tail) {
        hipLaunchKernelGGL(copy_bytes_kernel, dim3((unsigned)((tail + 255) / 256)), dim3(256), 0, stream,
                           (const uint8_t*)src + done, (uint8_t*)dst + done, tail);
        return hipGetLastError();
    }
    return hipSuccess;
}

// ------------------------------------------------------------------------------------------------
// Matrix-core calibration: 8 independent 32x32x16 bf16 accumulations per wave (128 AGPRs, so two
// workgroups fit on a CU and each SIMD can hold two waves), operands in registers, nothing but
// MFMAs in the loop.  The operands are ones built from the thread index, which the compiler cannot
// fold through the matrix instruction; each accumulator element ends at 16 * iters.
// ------------------------------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256, 2) mfma_ceiling_kernel(int iters, float* out) {
    const float one = (float)(1 + (threadIdx.x >> 8));  // 1 for every thread of the launch
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; i++) a[i] = b[i] = (__bf16)one;
    floatx16_t acc[8];
#pragma unroll
    for (int j = 0; j < 8; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[j][r] = 0.0f;
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int j = 0; j < 8; j++) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) s += acc[j][r];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

hipError_t launch_mfma_ceiling(int workgroups, int iters, float* out, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_ceiling_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, iters, out);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Launch-cost probe: a kernel with no work, one 64-thread workgroup per launch, so that what is
// timed is the cost of getting a kernel from the host call to a finished dispatch.
// ------------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(64) empty_kernel() {}

hipError_t launch_empty(int64_t count, hipStream_t stream) {
    for (int64_t i = 0; i < count; i++) {
        hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace fuse
