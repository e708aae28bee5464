// route_finalize.hip -- per-microbatch counts, offsets and balance statistics.
//
// One block per microbatch; fp64 internally, every sum in a fixed order:
//   counts_e (the histogram of page codechina.net article 413310 section 3.1,
//   zero-count experts kept), offsets = exclusive prefix sum of the counts,
//   f_e = counts_e/(Tm*k) and P_e = probability sum/Tm with
//   aux = alpha*E*sum_e f_e*P_e (page mhpq.cn/news/998159 sections 4.2, 4.4;
//   codechina.net section 2.2), CV = population std/mean and balance degree
//   1-(max-mean)/mean (page cnvsn.com/news/335486 sections 3.1, 5.1),
//   max/mean load (mhpq.cn section 5.4), entropy and max/min share of f
//   (codechina.net section 4.2), kept and dropped assignments under C.
#include "route_common.hpp"

namespace moe {
namespace {

using namespace dev;

constexpr int kFinThreads = 256;
constexpr int kFinWaves = kFinThreads / 64;
constexpr int kFinPer = (MOE_ROUTE_MAX_E + kFinThreads - 1) / kFinThreads;  // experts per thread
constexpr int kFinSplits = 8;  // split partials loaded together

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += shfl_xor_f64(v, m);
    return v;
}

__global__ void __launch_bounds__(kFinThreads)
route_finalize_kernel(const FinalArgs a)
{
    __shared__ double red[4][kFinWaves];
    __shared__ int wmax[kFinWaves], wmin[kFinWaves], wsum[kFinWaves];
    const int E = a.E;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int mb = blockIdx.x;
    const int per = (E + kFinThreads - 1) / kFinThreads;
    const int e0 = min(tid * per, E), e1 = min(e0 + per, E);
    const long so = long(mb) * a.nsplit * E;

    // counts and probability sums of my experts: all split partials loaded
    // before any is used
    int cnt[kFinPer];
    double ps[kFinPer];
#pragma unroll
    for (int u = 0; u < kFinPer; ++u) {
        cnt[u] = 0;
        ps[u] = 0.0;
    }
    for (int sp0 = 0; sp0 < a.nsplit; sp0 += kFinSplits) {
        int cv[kFinPer][kFinSplits];
        double pv[kFinPer][kFinSplits];
#pragma unroll
        for (int u = 0; u < kFinPer; ++u)
#pragma unroll
            for (int v = 0; v < kFinSplits; ++v) {
                const bool in = (e0 + u < e1) && (sp0 + v < a.nsplit);
                const long o = so + long(sp0 + v) * E + e0 + u;
                cv[u][v] = in ? a.split_tot[o] : 0;
                pv[u][v] = in ? a.split_P[o] : 0.0;
            }
#pragma unroll
        for (int u = 0; u < kFinPer; ++u)
#pragma unroll
            for (int v = 0; v < kFinSplits; ++v) {
                cnt[u] += cv[u][v];
                ps[u] += pv[u][v];
            }
    }

    const double total = double(a.Tm) * double(a.k);
    const double mean = total / double(E);
    const long cb = long(mb) * E;
    double dot = 0.0, var = 0.0, ent = 0.0, kept = 0.0;
    int cmax = -1, cmin = 0x7FFFFFFF, local = 0;
#pragma unroll
    for (int u = 0; u < kFinPer; ++u) {
        const int e = e0 + u;
        if (e < e1) {
            const int c = cnt[u];
            const double fe = double(c) / total;
            const double pe = ps[u] / double(a.Tm);
            a.counts[cb + e] = c;
            if (a.f) a.f[cb + e] = float(fe);
            if (a.P) a.P[cb + e] = float(pe);
            dot += fe * pe;
            var += (double(c) - mean) * (double(c) - mean);
            if (fe > 0.0) ent -= fe * log(fe);
            kept += double((a.capacity >= 0 && c > a.capacity) ? a.capacity : c);
            cmax = max(cmax, c);
            cmin = min(cmin, c);
            local += c;
        }
    }

    // offsets: exclusive scan of the counts in expert order
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(incl, d);
        if (lane >= d) incl += t;
    }
    // block reductions: butterflies inside the waves, then waves in order
    dot = wave_sum_f64(dot);
    var = wave_sum_f64(var);
    ent = wave_sum_f64(ent);
    kept = wave_sum_f64(kept);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        cmax = max(cmax, __shfl_xor(cmax, m));
        cmin = min(cmin, __shfl_xor(cmin, m));
    }
    if (lane == 63) wsum[wave] = incl;
    if (lane == 0) {
        red[0][wave] = dot;
        red[1][wave] = var;
        red[2][wave] = ent;
        red[3][wave] = kept;
        wmax[wave] = cmax;
        wmin[wave] = cmin;
    }
    __syncthreads();
    int run = incl - local;
    for (int w = 0; w < wave; ++w) run += wsum[w];
    for (int e = e0; e < e1; ++e) {
        a.offsets[long(mb) * (E + 1) + e] = run;
        run += cnt[e - e0];
    }
    if (tid == 0) {
        int tot = 0;
        double sdot = 0.0, svar = 0.0, sent = 0.0, skept = 0.0;
        int mx = -1, mn = 0x7FFFFFFF;
        for (int w = 0; w < kFinWaves; ++w) {
            tot += wsum[w];
            sdot += red[0][w];
            svar += red[1][w];
            sent += red[2][w];
            skept += red[3][w];
            mx = max(mx, wmax[w]);
            mn = min(mn, wmin[w]);
        }
        a.offsets[long(mb) * (E + 1) + E] = tot;
        a.aux[mb] = float(double(a.alpha) * double(E) * sdot);
        a.cv[mb] = float(sqrt(svar / double(E)) / mean);
        a.max_over_mean[mb] = float(double(mx) / mean);
        if (a.extra) {
            float* x = a.extra + long(mb) * 8;
            x[0] = float(double(mn) / mean);
            x[1] = float(1.0 - (double(mx) - mean) / mean);
            x[2] = float(sent);
            x[3] = float(skept);
            x[4] = float(total - skept);
            x[5] = float(a.capacity);
            x[6] = float(double(mx) / total);
            x[7] = float(double(mn) / total);
        }
    }
}

}  // namespace

hipError_t launch_route_finalize(const RowCfg& c, const FinalArgs& a, int n_micro, hipStream_t st) {
    (void)c;
    hipLaunchKernelGGL(route_finalize_kernel, dim3(n_micro), dim3(kFinThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace moe
