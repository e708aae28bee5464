// route_s4.hip -- row pass and backward kernels for segments of 4 lanes.
#include "route_rows_impl.hpp"

namespace moe {
MOE_INSTANTIATE_SEGMENT(4)
}  // namespace moe
