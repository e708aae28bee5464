// route_s32.hip -- row pass and backward kernels for segments of 32 lanes.
#include "route_rows_impl.hpp"

namespace moe {
MOE_INSTANTIATE_SEGMENT(32)
}  // namespace moe
