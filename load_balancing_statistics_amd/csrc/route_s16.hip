// route_s16.hip -- row pass and backward kernels for segments of 16 lanes.
#include "route_rows_impl.hpp"

namespace moe {
MOE_INSTANTIATE_SEGMENT(16)
}  // namespace moe
