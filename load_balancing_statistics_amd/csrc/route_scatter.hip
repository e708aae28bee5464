// route_scatter.hip -- expert offsets, the stable capacity-limited dispatch
// permutation, and the per-microbatch balance statistics.
//
// Dispatch order: inside each microbatch the assignments (t, j) are grouped by
// expert, experts ascending, and keep their (t, j) order inside an expert.
// The r-th assignment of an expert (r counted from 0) is dropped when r >= C
// (page mhpq.cn/news/998159 section 4.5: tokens beyond an expert's capacity
// are dropped).  Block b handles the same rows as row block b; its
// assignments to expert e start at offsets[e] + (count of e in the earlier
// blocks of the microbatch).  Inside the block each wave takes a contiguous
// slice; within a 64-assignment chunk the rank among equal experts comes from
// ballots over the expert-id bits, so the order is exact and deterministic.
//
// Statistics (first block of each microbatch, fp64 internally):
//   f_e = counts_e/(Tm*k), P_e = probability sum/Tm, aux = alpha*E*sum f*P
//   (page mhpq.cn/news/998159 sections 4.2 and 4.4; page codechina.net
//   article 413310 section 2.2), CV = population std/mean and balance degree
//   1-(max-mean)/mean (page cnvsn.com/news/335486 sections 3.1, 5.1),
//   max/mean (mhpq.cn section 5.4), entropy and max/min ratio of f
//   (codechina.net section 4.2), kept and dropped assignments.
#include "route_common.hpp"

namespace moe {
namespace {

using namespace dev;

constexpr int kScatWaves = 4;
constexpr int kScatThreads = kScatWaves * 64;

// Exclusive scan of n global ints into LDS out[0..n] (out[n] = total).
__device__ void block_excl_scan(const int32_t* in, int n, int* out, int* wsum) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (n + kScatThreads - 1) / kScatThreads;
    const int i0 = min(tid * per, n), i1 = min(i0 + per, n);
    int loc = 0;
    for (int i = i0; i < i1; ++i) loc += in[i];
    int incl = loc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int t = __shfl_up(incl, d);
        if (lane >= d) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += wsum[w];
    int run = wbase + incl - loc;
    for (int i = i0; i < i1; ++i) {
        out[i] = run;
        run += in[i];
    }
    if (tid == kScatThreads - 1) out[n] = run;
    __syncthreads();
}

__device__ double block_sum_f64(double v, double* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += shfl_xor_f64(v, m);
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    double t = 0.0;
    for (int w = 0; w < kScatWaves; ++w) t += red[w];
    return t;
}

__device__ void finalize_stats(const ScatterArgs& a, int mb, const int* offs, double* red) {
    const int E = a.E;
    const double total = double(a.Tm) * double(a.k);
    const double mean = total / double(E);
    const long cb = long(mb) * E;
    double dot = 0.0, var = 0.0, ent = 0.0;
    long long kept = 0;
    int cmax = -1, cmin = 0x7FFFFFFF;
    for (int e = threadIdx.x; e < E; e += kScatThreads) {
        const int c = a.totals[cb + e];
        const double fe = double(c) / total;
        const double pe = a.Psum[cb + e] / double(a.Tm);
        a.counts[cb + e] = c;
        if (a.f) a.f[cb + e] = float(fe);
        if (a.P) a.P[cb + e] = float(pe);
        dot += fe * pe;
        var += (double(c) - mean) * (double(c) - mean);
        if (fe > 0.0) ent -= fe * log(fe);
        kept += (a.capacity >= 0 && c > a.capacity) ? a.capacity : c;
        cmax = max(cmax, c);
        cmin = min(cmin, c);
    }
    for (int e = threadIdx.x; e <= E; e += kScatThreads) a.offsets[long(mb) * (E + 1) + e] = offs[e];
    dot = block_sum_f64(dot, red);
    var = block_sum_f64(var, red);
    ent = block_sum_f64(ent, red);
    const double keptd = block_sum_f64(double(kept), red);
    // integer max/min over the block
    __shared__ int smax, smin;
    if (threadIdx.x == 0) { smax = -1; smin = 0x7FFFFFFF; }
    __syncthreads();
    atomicMax(&smax, cmax);
    atomicMin(&smin, cmin);
    __syncthreads();
    if (threadIdx.x == 0) {
        const double mx = double(smax), mn = double(smin);
        a.aux[mb] = float(double(a.alpha) * double(E) * dot);
        a.cv[mb] = float(sqrt(var / double(E)) / mean);
        a.max_over_mean[mb] = float(mx / mean);
        if (a.extra) {
            float* x = a.extra + long(mb) * 8;
            x[0] = float(mn / mean);
            x[1] = float(1.0 - (mx - mean) / mean);
            x[2] = float(ent);
            x[3] = float(keptd);
            x[4] = float(total - keptd);
            x[5] = float(a.capacity);
            x[6] = float(mx / total);
            x[7] = float(mn / total);
        }
    }
}

__global__ void __launch_bounds__(kScatThreads)
route_scatter_kernel(const ScatterArgs a)
{
    extern __shared__ __align__(16) int sm[];
    const int E = a.E;
    int* offs = sm;                         // [E+1]
    int* wh = sm + ((E + 1 + 3) & ~3);      // [kScatWaves][E]
    __shared__ int wsum[kScatWaves];
    __shared__ double red[kScatWaves];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int mb = blockIdx.x / a.bpm, bi = blockIdx.x % a.bpm;
    const long row_begin = long(mb) * a.Tm + long(bi) * a.R;
    long row_end = row_begin + a.R;
    if (row_end > long(mb + 1) * a.Tm) row_end = long(mb + 1) * a.Tm;
    const long segment = long(mb) * a.Tm * a.k;  // start of the microbatch in perm
    const long seglen = long(a.Tm) * a.k;

    block_excl_scan(a.totals + long(mb) * E, E, offs, wsum);
    if (bi == 0) finalize_stats(a, mb, offs, red);

    for (int i = tid; i < kScatWaves * E; i += kScatThreads) wh[i] = 0;
    __syncthreads();

    // this block's assignments, split into one contiguous slice per wave
    const long a0 = row_begin * a.k, a1 = row_end * a.k;
    const long na = a1 - a0;
    long q = (na + kScatWaves - 1) / kScatWaves;
    q = (q + 63) & ~63L;
    const long s0 = min(a0 + wave * q, a1), s1 = min(s0 + q, a1);
    int* mywh = wh + wave * E;
    int internal = 0;

    for (long c = s0; c < s1; c += 64) {
        const long i = c + lane;
        if (i < s1) {
            const int e = a.topk_idx[i];
            if (e >= 0 && e < E) atomicAdd(&mywh[e], 1);
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kScatThreads) {
        int run = offs[e] + a.colprefix[long(blockIdx.x) * E + e];
        for (int w = 0; w < kScatWaves; ++w) {
            const int t = wh[w * E + e];
            wh[w * E + e] = run;
            run += t;
        }
    }
    __syncthreads();

    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (long c = s0; c < s1; c += 64) {
        const long i = c + lane;
        int e = (i < s1) ? a.topk_idx[i] : 0;
        bool valid = i < s1;
        if (valid && (e < 0 || e >= E)) {
            internal = 1;
            valid = false;
            e = 0;
        }
        uint64_t peers = __ballot(valid);
        for (int bt = 0; bt < nbits; ++bt) {
            const bool bit = (e >> bt) & 1;
            const uint64_t bal = __ballot(bit);
            peers &= bit ? bal : ~bal;
        }
        const int before = __popcll(peers & lt);
        const int cnt = __popcll(peers);
        const int basepos = mywh[e];
        const bool leader = valid && (63 - __clzll(peers)) == lane;
        if (leader) mywh[e] = basepos + cnt;
        if (valid) {
            const int pos = basepos + before;
            if (pos < 0 || pos >= seglen) {
                internal = 1;
            } else {
                const int r = pos - offs[e];
                a.dropped[i] = (a.capacity >= 0 && r >= a.capacity) ? 1 : 0;
                a.perm[segment + pos] = int32_t(i);
                if (a.inv_perm) a.inv_perm[i] = int32_t(segment + pos);
            }
        }
    }
    if (internal && a.status) atomicOr(a.status, MOE_STATUS_INTERNAL);
}

}  // namespace

hipError_t launch_route_scatter(const RowCfg& c, const ScatterArgs& a, hipStream_t st) {
    const size_t lds = (size_t((a.E + 1 + 3) & ~3) + size_t(kScatWaves) * a.E) * 4;
    hipLaunchKernelGGL(route_scatter_kernel, dim3(c.B), dim3(kScatThreads), lds, st, a);
    return hipGetLastError();
}

}  // namespace moe
