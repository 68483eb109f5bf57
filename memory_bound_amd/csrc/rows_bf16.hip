// rows_bf16.hip -- row and streaming kernels instantiated for bf16 storage.
#include "row_launch.hpp"

namespace fuse {
FUSE_INSTANTIATE_ROWS(DT::BF16)
}  // namespace fuse
