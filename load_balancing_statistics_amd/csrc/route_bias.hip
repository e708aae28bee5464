// route_bias.hip -- one update step of the selection bias.
//
// Page mhpq.cn/news/998159 section 4.3 (loss-free balancing): each expert has
// a scalar bias on its router logit; an overloaded expert's bias is pushed
// down and an idle expert's up, with no loss term.  The page fixes no step
// form; the step here is a fixed gamma against the sign of the load error:
//   load_e = sum over microbatches of counts[mb][e],
//   bias[e] -= gamma if load_e * E > T*k, += gamma if load_e * E < T*k.
// The comparison is exact (64-bit integers); the step is one fp32 add.
#include "route_common.hpp"

namespace moe {
namespace {

constexpr int kBiasThreads = 256;

__global__ void __launch_bounds__(kBiasThreads)
route_bias_update_kernel(const BiasArgs a)
{
    const int e = blockIdx.x * kBiasThreads + threadIdx.x;
    if (e >= a.E) return;
    int64_t load = 0;
    for (int mb = 0; mb < a.n_micro; ++mb) load += a.counts[int64_t(mb) * a.E + e];
    const int64_t lhs = load * a.E;
    const float b = a.bias[e];
    if (lhs > a.Tk) a.bias[e] = b - a.gamma;
    else if (lhs < a.Tk) a.bias[e] = b + a.gamma;
}

}  // namespace

hipError_t launch_bias_update(const BiasArgs& a, hipStream_t st) {
    const int blocks = (a.E + kBiasThreads - 1) / kBiasThreads;
    hipLaunchKernelGGL(route_bias_update_kernel, dim3(blocks), dim3(kBiasThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace moe
