// route_s64.hip -- row pass and backward kernels for segments of 64 lanes.
#include "route_rows_impl.hpp"

namespace moe {
MOE_INSTANTIATE_SEGMENT(64)
}  // namespace moe
