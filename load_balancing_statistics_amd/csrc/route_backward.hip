// route_backward.hip -- gradient of the aux loss with respect to the logits.
//
// L_aux = alpha * E * sum_i f_i * P_i with P_i the mean softmax probability
// of expert i over the microbatch and f_i a constant observation (pages
// mhpq.cn/news/998159 section 4.2 and codechina.net article 413310 section
// 2.2: the gradient reaches the router through P only).  Differentiating the
// softmax gives, for token t of microbatch mb,
//   dL/dl[t,j] = g_mb * alpha * E / Tm * p[t,j] * (f_j - sum_i f_i p[t,i]).
// One streaming pass: read a row (and its saved softmax statistics when
// given), write the row of the gradient.  Same lane mapping as the row pass.
#include "route_common.hpp"

namespace moe {
namespace {

using namespace dev;

template <int S, int G, int NW>
__global__ void __launch_bounds__(NW * 64)
route_backward_kernel(const BackArgs a)
{
    constexpr int W = 64 / S;
    const int E = a.E;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int seg = lane / S, s = lane % S;
    const int mb = blockIdx.x / a.bpm, bi = blockIdx.x % a.bpm;
    const long row_begin = long(mb) * a.Tm + long(bi) * a.R;
    long row_end = row_begin + a.R;
    if (row_end > long(mb + 1) * a.Tm) row_end = long(mb + 1) * a.Tm;

    const float inv_total = 1.0f / (float(a.Tm) * float(a.k));
    float fcol[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int col = g * S + s;
        fcol[g] = (col < E) ? float(a.counts[long(mb) * E + col]) * inv_total : 0.f;
    }
    const float gup = a.d_aux ? a.d_aux[mb] : 1.0f;
    const float c = gup * a.alpha * float(E) / float(a.Tm);

    const long per_iter = long(NW) * W;
    for (long row = row_begin + long(wave) * W + seg;
         row - seg < row_end; row += per_iter) {
        const bool valid = row < row_end;
        const float* src = a.logits + row * E;
        float x[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int col = g * S + s;
            x[g] = (valid && col < E) ? __builtin_nontemporal_load(src + col) : -INFINITY;
        }
        float m, ssum;
        float ex[G];
        if (a.row_stats) {
            m = valid ? a.row_stats[2 * row] : 0.f;
            ssum = valid ? a.row_stats[2 * row + 1] : 1.f;
            const float mL = m * kLog2e;
#pragma unroll
            for (int g = 0; g < G; ++g) ex[g] = exp2f(fmaf(x[g], kLog2e, -mL));
        } else {
            float lmax = x[0];
#pragma unroll
            for (int g = 1; g < G; ++g) lmax = fmaxf(lmax, x[g]);
            m = seg_max<S>(lmax);
            const float mL = m * kLog2e;
            ssum = 0.f;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                ex[g] = exp2f(fmaf(x[g], kLog2e, -mL));
                ssum += ex[g];
            }
            ssum = seg_sum<S>(ssum);
        }
        const float inv = 1.0f / ssum;
        float dot = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            ex[g] *= inv;  // p
            dot = fmaf(fcol[g], ex[g], dot);
        }
        dot = seg_sum<S>(dot);
        if (valid) {
            float* dst = a.dlogits + row * E;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int col = g * S + s;
                if (col < E) __builtin_nontemporal_store(c * ex[g] * (fcol[g] - dot), dst + col);
            }
        }
    }
}

template <int S, int G>
hipError_t launch_sg(const RowCfg& c, const BackArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((route_backward_kernel<S, G, 8>), dim3(c.B), dim3(8 * 64), 0, st, a);
    return hipGetLastError();
}

template <int S>
hipError_t launch_s(const RowCfg& c, const BackArgs& a, hipStream_t st) {
    switch (c.G) {
        case 1: return launch_sg<S, 1>(c, a, st);
        case 2: return launch_sg<S, 2>(c, a, st);
        case 4: return launch_sg<S, 4>(c, a, st);
        case 8: return launch_sg<S, 8>(c, a, st);
        case 12: return launch_sg<S, 12>(c, a, st);
        case 16: return launch_sg<S, 16>(c, a, st);
        case 24: return launch_sg<S, 24>(c, a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_route_backward(const RowCfg& c, const BackArgs& a, hipStream_t st) {
    if (c.NW != 8) return hipErrorInvalidValue;
    switch (c.S) {
        case 1: return launch_s<1>(c, a, st);
        case 2: return launch_s<2>(c, a, st);
        case 4: return launch_s<4>(c, a, st);
        case 8: return launch_s<8>(c, a, st);
        case 16: return launch_s<16>(c, a, st);
        case 32: return launch_s<32>(c, a, st);
        case 64: return launch_s<64>(c, a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
