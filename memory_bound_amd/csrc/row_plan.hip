// row_plan.hip -- choice of the compiled row-kernel instantiation (lane vector width, chunks per
// lane, waves per row) for a row length.  Kept apart from the entry points so that the code which
// decides the launch of the row kernels sits in the files those kernels are built from.
#include "row_plan.hpp"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>

namespace fuse {

RowPlan plan_row(int64_t n, int eb, bool aligned, int wpr_override) {
    const int V = 16 / eb;
    if (aligned && (n % V) == 0) {
        // About two 16-byte chunks per lane: more waves per row shorten each lane's load chain
        // and give the memory system more independent requests, which measured fastest for the
        // 48 MiB Add+LayerNorm and 512 MiB softmax workloads (4096 and 2048 fp16 per row).
        const int64_t c = n / V;
        int wpr = 1;
        while (c > 128 * wpr && wpr < 8) wpr *= 2;
        if (wpr_override == 1 || wpr_override == 2 || wpr_override == 4 || wpr_override == 8) {
            if (c <= (int64_t)64 * 16 * wpr_override) wpr = wpr_override;
        }
        int nv = 1;
        while ((int64_t)nv * 64 * wpr < c) nv *= 2;
        if (nv > 8 && wpr == 8) return {true, 8, 8};  // unreachable below the row-length limit
        return {true, nv, wpr};
    }
    if (n <= 64) return {false, 1, 1};
    if (n <= 256) return {false, 4, 1};
    if (n <= 1024) return {false, 16, 1};
    if (n <= 4096) return {false, 16, 4};
    return {false, 32, 8};
}

namespace {

int device_cus() {
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

// FUSE_ROW_STEPS = 1, 2 or 4, else 0.
int steps_override() {
    if (const char* e = getenv("FUSE_ROW_STEPS")) {
        const int v = atoi(e);
        if (v == 1 || v == 2 || v == 4) return v;
    }
    return 0;
}

}  // namespace

int row_steps(int64_t blocks) {
    if (const int v = steps_override()) return v;
    // Measured on MI355X (256 CUs), [R, 4096] fp16 Add+LayerNorm: 2048 rows (8 blocks per CU)
    // fastest with 4 steps (512 workgroups, 10.0 vs 10.4 us), 16384 rows (64 per CU) with 2
    // (66.3 vs 68.3 us); 4 steps start once they still leave two workgroups per CU, 2 steps
    // once they leave four.
    const int64_t cus = device_cus();
    if (blocks > 16 * cus) return 2;
    if (blocks >= 8 * cus) return 4;
    if (blocks >= 4 * cus) return 2;
    return 1;
}

int scan_steps(int64_t blocks) {
    if (const int v = steps_override()) return v;
    // Measured on MI355X (256 CUs), [2048, 4096] fp16 cumsum + scale (8 blocks per CU), three
    // alternating runs each: 2 steps 6.9-7.1 us, 1 step 7.2-7.3 us, 4 steps 7.4 us.  The scan
    // stores a block's words right after one LDS exchange, so it needs less of the read-ahead
    // that the LayerNorm's two reductions do; 2 steps once they still leave four workgroups per CU.
    return blocks >= 8 * device_cus() ? 2 : 1;
}

}  // namespace fuse
