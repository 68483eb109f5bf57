// copy.hip -- plain device copy used to calibrate the roofline (achievable streaming bandwidth and
// the scale of the hardware byte counters).
#include "launch.hpp"
#include "stream_kernels.hpp"

namespace fuse {

// ------------------------------------------------------------------------------------------------
// Plain copy (roofline calibration): 16-byte chunks, CH per thread, plus a byte tail kernel.
// ------------------------------------------------------------------------------------------------
template <int CH>
__global__ void __launch_bounds__(256)
copy16_kernel(const uint4* src, uint4* dst, uint64_t n16) {
    const uint64_t base = (uint64_t)blockIdx.x * (256 * CH) + threadIdx.x;
    uint4 v[CH];
#pragma unroll
    for (int j = 0; j < CH; j++) {
        const uint64_t i = base + (uint64_t)j * 256;
        if (i < n16) v[j] = src[i];
    }
#pragma unroll
    for (int j = 0; j < CH; j++) {
        const uint64_t i = base + (uint64_t)j * 256;
        if (i < n16) dst[i] = v[j];
    }
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

}  // namespace fuse
