// sinkhorn.hip -- single-workgroup Sinkhorn-Knopp flow plan (LoongForge TAOT
// blog at baidu-baige.github.io, section 2, Phase 1): the overload of each
// rank is the supply, the idle capacity the demand, and the entropy-
// regularised transport plan under a topology cost matrix C is
//   T = diag(u) K diag(v),  K = exp(-C / eps),
// found by alternating matrix-vector steps from u = v = 1:
//   u_i = a_i / max(sum_j K_ij v_j, tiny),  v_j = b_j / max(sum_i K_ij u_i, tiny)
// (tiny = 1e-300), fp64.  R <= 64 ranks, one workgroup of four waves: lane i
// of wave q holds K[i][16q..16q+16) and K[16q..16q+16)[i] in registers and
// forms that quarter of the row and column products (four interleaved sums);
// the quarters meet in LDS and every wave combines them in the same order,
// so each keeps an identical copy of u and v (one barrier per half-round).
// The summation order differs from a left-to-right sum by rounding only.
// All rounds run in one launch with no host round trip.
#include "route_common.hpp"

namespace moe {
namespace {

constexpr int kMaxR = 64;
constexpr int kQ = 4;              // waves; wave q sums the columns [16q, 16q+16)
constexpr int kSpan = kMaxR / kQ;

// Partial product over the wave's 16 columns, four interleaved sums.
__device__ __forceinline__ double dot16(const double (&k)[kSpan], const double* x) {
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
#pragma unroll
    for (int j = 0; j < kSpan; j += 4) {
        s0 = fma(k[j], x[j], s0);
        s1 = fma(k[j + 1], x[j + 1], s1);
        s2 = fma(k[j + 2], x[j + 2], s2);
        s3 = fma(k[j + 3], x[j + 3], s3);
    }
    return (s0 + s1) + (s2 + s3);
}

__global__ void __launch_bounds__(kQ * 64)
sinkhorn_kernel(const SinkhornArgs a)
{
    __shared__ double red[2][kQ][kMaxR];  // partial products, ping-pong
    __shared__ double xs[kQ][kMaxR];      // each wave's copy of u or v
    const int R = a.R;
    const int i = threadIdx.x & 63, q = threadIdx.x >> 6;
    const bool own = i < R;
    // K[i][16q..16q+16) and K[16q..16q+16)[i] in registers (zero past R)
    double kr[kSpan], kc[kSpan];
#pragma unroll
    for (int t = 0; t < kSpan; ++t) {
        const int j = q * kSpan + t;
        kr[t] = (own && j < R) ? exp(-a.C[long(i) * R + j] / a.eps) : 0.0;
        kc[t] = (own && j < R) ? exp(-a.C[long(j) * R + i] / a.eps) : 0.0;
    }
    const double ai = own ? a.supply[i] : 0.0, bi = own ? a.demand[i] : 0.0;
    const double tiny = 1e-300;
    double* mine = xs[q];
    mine[i] = own ? 1.0 : 0.0;  // v = 1
    double u = 1.0, v = 1.0;
    int h = 0;
    for (int it = 0; it < a.iters; ++it) {
        // u_i = a_i / (K v)_i
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        red[h][q][i] = dot16(kr, mine + q * kSpan);
        __syncthreads();
        {
            const double su = ((red[h][0][i] + red[h][1][i]) + red[h][2][i]) + red[h][3][i];
            u = own ? ai / (su > tiny ? su : tiny) : 0.0;
        }
        mine[i] = u;
        h ^= 1;
        // v_j = b_j / (K^T u)_j
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        red[h][q][i] = dot16(kc, mine + q * kSpan);
        __syncthreads();
        {
            const double sv = ((red[h][0][i] + red[h][1][i]) + red[h][2][i]) + red[h][3][i];
            v = own ? bi / (sv > tiny ? sv : tiny) : 0.0;
        }
        mine[i] = v;
        h ^= 1;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (own) {
        if (q == 0) {
            a.u[i] = u;
            a.v[i] = v;
        }
        // wave q writes the columns of its span
#pragma unroll
        for (int t = 0; t < kSpan; ++t) {
            const int j = q * kSpan + t;
            if (j < R) a.T[long(i) * R + j] = u * kr[t] * mine[j];
        }
    }
}

}  // namespace

hipError_t launch_sinkhorn(const SinkhornArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(sinkhorn_kernel, dim3(1), dim3(kQ * 64), 0, st, a);
    return hipGetLastError();
}

}  // namespace moe
