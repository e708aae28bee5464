// route_scan.hip -- combine the per-block partials of the row pass.
//
// For each microbatch, expert and split (a contiguous range of at most
// kScanWaves*kScanPerWave row blocks): the split's count and probability
// sum, and the exclusive prefix of the counts over the split's blocks -- the
// base at which a block's assignments to that expert start, relative to the
// split, inside the expert's segment of the dispatch permutation.  The
// counts form the histogram of page codechina.net article 413310 section 3.1
// (zero-count experts kept); the probability sums give P_i of page
// mhpq.cn/news/998159 section 4.2, accumulated in fp64 in block order.  The
// scatter that follows turns the split sums into the offsets and the
// balance statistics.
//
// Grid: (ceil(E/64), n_micro, nsplit); lane = expert; each of the 16 waves
// owns up to 8 consecutive row blocks, so every load is issued in one round.
#include "route_common.hpp"

namespace moe {
namespace {

using namespace dev;

constexpr int kScanThreads = kScanWaves * 64;

__global__ void __launch_bounds__(kScanThreads)
route_scan_kernel(const ScanArgs a)
{
    __shared__ int wc[kScanWaves][64];
    __shared__ double wp[kScanWaves][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + lane;
    const int mb = blockIdx.y, sp = blockIdx.z;
    const bool ok = e < a.E;
    const int per_split = kScanWaves * kScanPerWave;
    const int j0 = min(sp * per_split + wave * kScanPerWave, a.bpm);
    const int j1 = min(j0 + kScanPerWave, min((sp + 1) * per_split, a.bpm));
    const long first = long(mb) * a.bpm;

    int cv[kScanPerWave];
    float pv[kScanPerWave];
#pragma unroll
    for (int u = 0; u < kScanPerWave; ++u) {
        const bool in = ok && (j0 + u < j1);
        const long o = (first + j0 + u) * a.E + e;
        cv[u] = load_or(a.cnt_part, o, in, 0);
        pv[u] = load_or(a.P_part, o, in, 0.f);
    }
    int csum = 0;
    double psum = 0.0;
#pragma unroll
    for (int u = 0; u < kScanPerWave; ++u) {
        csum += cv[u];
        psum += double(pv[u]);
    }
    wc[wave][lane] = csum;
    wp[wave][lane] = psum;
    __syncthreads();

    // every wave reads all 16 partials at once (unrolled), keeping those of
    // the earlier waves
    int run = 0;
    {
        int c[kScanWaves];
#pragma unroll
        for (int w = 0; w < kScanWaves; ++w) c[w] = wc[w][lane];
#pragma unroll
        for (int w = 0; w < kScanWaves; ++w) run += (w < wave) ? c[w] : 0;
    }
#pragma unroll
    for (int u = 0; u < kScanPerWave; ++u) {
        if (ok && j0 + u < j1) a.colprefix[(first + j0 + u) * a.E + e] = run;
        run += cv[u];
    }
    if (wave == 0 && ok) {
        int c[kScanWaves];
        double q[kScanWaves];
#pragma unroll
        for (int w = 0; w < kScanWaves; ++w) {
            c[w] = wc[w][lane];
            q[w] = wp[w][lane];
        }
        int tot = 0;
        double ps = 0.0;
#pragma unroll
        for (int w = 0; w < kScanWaves; ++w) {
            tot += c[w];
            ps += q[w];
        }
        const long so = (long(mb) * a.nsplit + sp) * a.E + e;
        a.split_tot[so] = tot;
        a.split_P[so] = ps;
    }

    // status word: OR of the row blocks' flags (one block does it)
    if (a.status && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) {
        int fl = 0;
        for (int b = threadIdx.x; b < a.B; b += kScanThreads) fl |= a.flag_part[b];
        fl = __syncthreads_or(fl & MOE_STATUS_NONFINITE) ? MOE_STATUS_NONFINITE : 0;
        if (threadIdx.x == 0) a.status[0] = fl;
    }
}

}  // namespace

hipError_t launch_route_scan(const RowCfg& c, const ScanArgs& a, hipStream_t st) {
    dim3 grid((a.E + 63) / 64, a.n_micro, c.nsplit);
    hipLaunchKernelGGL(route_scan_kernel, grid, dim3(kScanThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace moe
