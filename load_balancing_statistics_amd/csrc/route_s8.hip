// route_s8.hip -- row pass and backward kernels for segments of 8 lanes.
#include "route_rows_impl.hpp"

namespace moe {
MOE_INSTANTIATE_SEGMENT(8)
}  // namespace moe
