// route_s1.hip -- row pass and backward kernels for segments of 1 lanes.
#include "route_rows_impl.hpp"

namespace moe {
MOE_INSTANTIATE_SEGMENT(1)
}  // namespace moe
