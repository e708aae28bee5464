// route_scan.hip -- combine the per-block partials of the row pass, then the
// per-microbatch counts, offsets and balance statistics.
//
// Part 1, every block.  For each microbatch, expert and split (a contiguous
// range of at most kScanWaves*kScanPerWave row blocks): the split's count and
// probability sum, and the exclusive prefix of the counts over the split's
// blocks -- the base at which a block's assignments to that expert start,
// relative to the split, inside the expert's segment of the dispatch
// permutation.  The counts form the histogram of page codechina.net article
// 413310 section 3.1 (zero-count experts kept); the probability sums give P_i
// of page mhpq.cn/news/998159 section 4.2, accumulated in fp64 in block order.
//
// Part 2, the last block of a microbatch to finish part 1 (an arrival counter
// per microbatch, zeroed by the row pass that precedes this kernel): fp64,
// every sum in a fixed order:
//   counts_e, offsets = exclusive prefix sum of the counts,
//   f_e = counts_e/(Tm*k) and P_e = probability sum/Tm (or /(Tm*k) for the
//   masked form of mhpq.cn section 4.4, whose sums cover the picks only) with
//   aux = alpha*E*sum_e f_e*P_e (mhpq.cn sections 4.2, 4.4; codechina.net
//   section 2.2), CV = population std/mean and balance degree
//   1-(max-mean)/mean (page cnvsn.com/news/335486 sections 3.1, 5.1),
//   max/mean load (mhpq.cn section 5.4), entropy and max/min share of f
//   (codechina.net section 4.2), kept and dropped assignments under C.
//
// Grid: (ceil(E/64), n_micro, nsplit); lane = expert; each of the 16 waves
// owns up to 8 consecutive row blocks, so every load is issued in one round.
#include <climits>

#include "route_common.hpp"

namespace moe {
namespace {

using namespace dev;

constexpr int kScanThreads = kScanWaves * 64;
constexpr int kStatSplits = 8;  // split partials loaded together
static_assert(MOE_ROUTE_MAX_E <= kScanThreads, "one expert per thread in the statistics");

// Statistics of microbatch mb from the split partials; one expert per
// thread, reductions per wave (only the waves that own experts) and then
// over those waves in order.
__device__ void microbatch_statistics(const ScanArgs& a, int mb) {
    __shared__ double red[4][kScanWaves];
    __shared__ int wmax[kScanWaves], wmin[kScanWaves], wsum[kScanWaves];
    const int E = a.E;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool own = tid < E;
    const bool wave_owns = wave * 64 < E;  // wave-uniform
    const int nwaves = (E + 63) / 64;
    const long so = long(mb) * a.nsplit * E + tid;

    int cnt = 0;
    double ps = 0.0;
    for (int sp0 = 0; sp0 < a.nsplit; sp0 += kStatSplits) {
        int cv[kStatSplits];
        double pv[kStatSplits];
#pragma unroll
        for (int v = 0; v < kStatSplits; ++v) {
            const bool in = own && (sp0 + v < a.nsplit);
            const long o = so + long(sp0 + v) * E;
            cv[v] = load_or(a.split_tot, o, in, 0);
            pv[v] = load_or(a.split_P, o, in, 0.0);
        }
#pragma unroll
        for (int v = 0; v < kStatSplits; ++v) {
            cnt += cv[v];
            ps += pv[v];
        }
    }

    const double total = double(a.Tm) * double(a.k);
    const double mean = total / double(E);
    const long cb = long(mb) * E;
    double dot = 0.0, var = 0.0, ent = 0.0, kept = 0.0;
    int cmax = -1, cmin = INT_MAX;
    if (own) {
        const double fe = double(cnt) / total;
        const double pe = ps / (a.p_masked ? total : double(a.Tm));
        a.counts[cb + tid] = cnt;
        if (a.f) a.f[cb + tid] = float(fe);
        if (a.P) a.P[cb + tid] = float(pe);
        dot = fe * pe;
        var = (double(cnt) - mean) * (double(cnt) - mean);
        if (fe > 0.0) ent = -fe * log(fe);
        kept = double((a.capacity >= 0 && cnt > a.capacity) ? a.capacity : cnt);
        cmax = cnt;
        cmin = cnt;
    }

    // offsets: exclusive scan of the counts in expert order
    int incl = 0;
    if (wave_owns) {
        incl = wave_incl_scan_i(cnt);
        dot = wave_sum_f64(dot);
        var = wave_sum_f64(var);
        ent = wave_sum_f64(ent);
        kept = wave_sum_f64(kept);
        cmax = wave_max_i(cmax);
        cmin = wave_min_i(cmin);
        if (lane == 63) wsum[wave] = incl;
        if (lane == 0) {
            red[0][wave] = dot;
            red[1][wave] = var;
            red[2][wave] = ent;
            red[3][wave] = kept;
            wmax[wave] = cmax;
            wmin[wave] = cmin;
        }
    }
    __syncthreads();
    if (own) {
        int run = incl - cnt;
        for (int w = 0; w < wave; ++w) run += wsum[w];
        a.offsets[long(mb) * (E + 1) + tid] = run;
    }
    if (tid == 0) {
        int tot = 0;
        double sdot = 0.0, svar = 0.0, sent = 0.0, skept = 0.0;
        int mx = -1, mn = INT_MAX;
        for (int w = 0; w < nwaves; ++w) {
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

__global__ void __launch_bounds__(kScanThreads)
route_scan_kernel(const ScanArgs a)
{
    __shared__ int wc[kScanWaves][64];
    __shared__ double wp[kScanWaves][64];
    __shared__ int last;
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

    int run = 0;
    for (int w = 0; w < wave; ++w) run += wc[w][lane];
#pragma unroll
    for (int u = 0; u < kScanPerWave; ++u) {
        if (ok && j0 + u < j1) a.colprefix[(first + j0 + u) * a.E + e] = run;
        run += cv[u];
    }
    if (wave == 0 && ok) {
        int tot = 0;
        double ps = 0.0;
        for (int w = 0; w < kScanWaves; ++w) {
            tot += wc[w][lane];
            ps += wp[w][lane];
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

    // arrival: the barrier orders the block's split stores before thread 0's
    // agent-scope acquire-release increment, which publishes them (one cache
    // write-back per block) and, in the block that completes the microbatch,
    // makes every other block's partials visible to the statistics after the
    // second barrier
    __syncthreads();
    if (threadIdx.x == 0) {
        const int blocks = int(gridDim.x * gridDim.z);
        const int prev = __hip_atomic_fetch_add(&a.arrive[mb], 1, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_AGENT);
        last = (prev == blocks - 1) ? 1 : 0;
    }
    __syncthreads();
    if (!last) return;
    microbatch_statistics(a, mb);
}

}  // namespace

hipError_t launch_route_scan(const RowCfg& c, const ScanArgs& a, hipStream_t st) {
    dim3 grid((a.E + 63) / 64, a.n_micro, c.nsplit);
    hipLaunchKernelGGL(route_scan_kernel, grid, dim3(kScanThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace moe
