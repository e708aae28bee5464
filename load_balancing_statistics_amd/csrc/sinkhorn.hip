// sinkhorn.hip -- single-workgroup Sinkhorn-Knopp flow plan (LoongForge TAOT
// blog at baidu-baige.github.io, section 2, Phase 1): the overload of each
// rank is the supply, the idle capacity the demand, and the entropy-
// regularised transport plan under a topology cost matrix C is
//   T = diag(u) K diag(v),  K = exp(-C / eps),
// found by alternating matrix-vector steps from u = v = 1:
//   u_i = a_i / max(sum_j K_ij v_j, tiny),  v_j = b_j / max(sum_i K_ij u_i, tiny)
// (tiny = 1e-300), sums in index order, fp64.  R <= 64 ranks: one wave, lane
// i owns rank i; K sits in LDS with row stride R+1 doubles so that both the
// row sums (lanes walk their own row) and the column sums (lanes walk
// consecutive columns) read it without bank conflicts to speak of; all
// rounds run in one launch with no host round trip.
#include "route_common.hpp"

namespace moe {
namespace {

constexpr int kMaxR = 64;

__global__ void __launch_bounds__(64)
sinkhorn_kernel(const SinkhornArgs a)
{
    __shared__ double K[kMaxR * (kMaxR + 1)];
    __shared__ double uv[2][kMaxR];
    const int R = a.R, S = R + 1;
    const int i = threadIdx.x;
    const bool own = i < R;
    for (int j = 0; j < R; ++j)
        if (own) K[i * S + j] = exp(-a.C[long(i) * R + j] / a.eps);
    double u = 1.0, v = 1.0;
    const double ai = own ? a.supply[i] : 0.0, bi = own ? a.demand[i] : 0.0;
    if (own) uv[1][i] = 1.0;
    const double tiny = 1e-300;
    for (int it = 0; it < a.iters; ++it) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (own) {
            double s = 0.0;
            for (int j = 0; j < R; ++j) s = fma(K[i * S + j], uv[1][j], s);
            u = ai / (s > tiny ? s : tiny);
            uv[0][i] = u;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (own) {
            double s = 0.0;
            for (int r = 0; r < R; ++r) s = fma(K[r * S + i], uv[0][r], s);
            v = bi / (s > tiny ? s : tiny);
            uv[1][i] = v;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (own) {
        a.u[i] = u;
        a.v[i] = v;
        for (int j = 0; j < R; ++j) a.T[long(i) * R + j] = u * K[i * S + j] * uv[1][j];
    }
}

}  // namespace

hipError_t launch_sinkhorn(const SinkhornArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(sinkhorn_kernel, dim3(1), dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace moe
