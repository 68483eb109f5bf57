// row_plan.hip -- choice of the compiled row-kernel instantiation (lane vector width, chunks per
// lane, waves per row) for a row length.  Kept apart from the entry points so that the code which
// decides the launch of the row kernels sits in the files those kernels are built from.
#include "row_plan.hpp"

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

}  // namespace fuse
