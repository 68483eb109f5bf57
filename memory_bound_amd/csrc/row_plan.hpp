// row_plan.hpp -- launch shape of the register-resident row kernels.
#pragma once

#include <stdint.h>

namespace fuse {

// Shape of a register-resident row kernel launch: 128-bit or per-element access, chunks per
// lane (NV) and waves per row (WPR).
struct RowPlan {
    bool vec;
    int nv;
    int wpr;
};

// Plan for a row of n elements of elem_bytes each; `aligned` = every pointer is 16-byte aligned
// and n * elem_bytes is a multiple of 16.  `wpr_override` > 0 forces the waves per row on the
// 128-bit path when the resulting chunks per lane stay within the compiled set.
RowPlan plan_row(int64_t n, int elem_bytes, bool aligned, int wpr_override);

// Row blocks each workgroup of the LayerNorm kernels walks (1, 2 or 4) for a launch of `blocks`
// row blocks on the current device.  FUSE_ROW_STEPS = 1, 2 or 4 overrides it (tests, tuning).
int row_steps(int64_t blocks);

// The same for the cumsum + scale kernel (1 or 2; FUSE_ROW_STEPS overrides it the same way).
int scan_steps(int64_t blocks);

}  // namespace fuse
