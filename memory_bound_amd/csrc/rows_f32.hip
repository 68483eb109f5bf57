// rows_f32.hip -- row and streaming kernels instantiated for f32 storage.
#include "row_launch.hpp"

namespace fuse {
FUSE_INSTANTIATE_ROWS(DT::F32)
}  // namespace fuse
