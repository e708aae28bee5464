// route_scan.hip -- combine the per-block partials of the row pass.
//
// For each microbatch and expert: the total count (the histogram of
// page codechina.net article 413310 section 3.1, zero-count experts kept),
// the exclusive prefix of the counts over the microbatch's blocks (the base
// at which each block's assignments to that expert start inside the expert's
// segment of the dispatch permutation), and the probability sum behind P_i
// (page mhpq.cn/news/998159 section 4.2), accumulated in fp64 in block order.
//
// Grid: (ceil(E/64), n_micro); 16 waves per block, lane = expert, each wave
// owns a contiguous range of the microbatch's row blocks.
#include "route_common.hpp"

namespace moe {
namespace {

constexpr int kScanWaves = 16;
constexpr int kScanChunk = 8;  // loads in flight per lane

__global__ void __launch_bounds__(kScanWaves * 64)
route_scan_kernel(const ScanArgs a)
{
    __shared__ int wc[kScanWaves][64];
    __shared__ double wp[kScanWaves][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + lane;
    const int mb = blockIdx.y;
    const bool ok = e < a.E;
    const int q = (a.bpm + kScanWaves - 1) / kScanWaves;
    const int j0 = min(wave * q, a.bpm), j1 = min(j0 + q, a.bpm);
    const long first = long(mb) * a.bpm;

    int csum = 0;
    double psum = 0.0;
    for (int j = j0; j < j1; j += kScanChunk) {
        int cv[kScanChunk];
        float pv[kScanChunk];
#pragma unroll
        for (int u = 0; u < kScanChunk; ++u) {
            const bool in = ok && (j + u < j1);
            const long o = (first + j + u) * a.E + e;
            cv[u] = in ? a.cnt_part[o] : 0;
            pv[u] = in ? a.P_part[o] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kScanChunk; ++u) {
            csum += cv[u];
            psum += double(pv[u]);
        }
    }
    wc[wave][lane] = csum;
    wp[wave][lane] = psum;
    __syncthreads();

    int base = 0;
    for (int w = 0; w < wave; ++w) base += wc[w][lane];
    if (wave == 0 && ok) {
        int tot = 0;
        double ps = 0.0;
        for (int w = 0; w < kScanWaves; ++w) {
            tot += wc[w][lane];
            ps += wp[w][lane];
        }
        a.totals[long(mb) * a.E + e] = tot;
        a.Psum[long(mb) * a.E + e] = ps;
    }

    int run = base;
    for (int j = j0; j < j1; j += kScanChunk) {
        int cv[kScanChunk];
#pragma unroll
        for (int u = 0; u < kScanChunk; ++u) {
            const bool in = ok && (j + u < j1);
            cv[u] = in ? a.cnt_part[(first + j + u) * a.E + e] : 0;
        }
#pragma unroll
        for (int u = 0; u < kScanChunk; ++u) {
            if (ok && j + u < j1) a.colprefix[(first + j + u) * a.E + e] = run;
            run += cv[u];
        }
    }

    // status word: OR of the row blocks' flags (one block does it)
    if (a.status && blockIdx.x == 0 && blockIdx.y == 0) {
        int fl = 0;
        for (int b = threadIdx.x; b < a.B; b += kScanWaves * 64) fl |= a.flag_part[b];
        fl = __syncthreads_or(fl & MOE_STATUS_NONFINITE) ? MOE_STATUS_NONFINITE : 0;
        if (threadIdx.x == 0) a.status[0] = fl;
    }
}

}  // namespace

hipError_t launch_route_scan(const RowCfg& c, const ScanArgs& a, hipStream_t st) {
    dim3 grid((a.E + 63) / 64, a.n_micro);
    hipLaunchKernelGGL(route_scan_kernel, grid, dim3(kScanWaves * 64), 0, st, a);
    (void)c;
    return hipGetLastError();
}

}  // namespace moe
