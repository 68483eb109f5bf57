// rows_f16.hip -- row and streaming kernels instantiated for f16 storage.
#include "row_launch.hpp"

namespace fuse {
FUSE_INSTANTIATE_ROWS(DT::F16)
}  // namespace fuse
