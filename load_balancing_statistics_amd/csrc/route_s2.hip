// route_s2.hip -- row pass and backward kernels for segments of 2 lanes.
#include "route_rows_impl.hpp"

namespace moe {
MOE_INSTANTIATE_SEGMENT(2)
}  // namespace moe
