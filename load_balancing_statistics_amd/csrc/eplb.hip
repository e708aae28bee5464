// eplb.hip -- EPLB placement over the routing counts: replicate experts, then
// pack the replicas onto GPUs (page cnvsn.com/news/335486, section 4.1.2).
//
// replicate_experts: each logical expert starts with one replica; while the
// physical count is below num_phys the expert with the largest load per
// replica, weight[e] / logcnt[e], gets another (physical E + r is the r-th
// copy).  balanced_packing: the replicas, weighted weight / logcnt of their
// expert, are taken heaviest first and each goes to the lightest pack that is
// not yet full (num_phys / num_packs replicas per pack).
// Per-replica loads are compared exactly as 64-bit cross products; ties go to
// the lower expert / replica / pack index; pack loads are fp64 sums in
// placement order.  One workgroup: the two greedy loops are sequential by
// nature and run in wave 0 with the candidates spread over the lanes and
// DPP arg-max/arg-min reductions; the sort between them ranks every replica
// by counting, over the whole workgroup.
#include "route_common.hpp"

namespace moe {
namespace {

using namespace dev;

constexpr int kEplbThreads = 256;
constexpr int kPerLane = MOE_ROUTE_MAX_E / 64;  // experts (and packs) per lane of wave 0

// a/b > c/d for non-negative a, c and positive b, d (exact).
__device__ __forceinline__ bool ratio_gt(int64_t a, int64_t b, int64_t c, int64_t d) {
    return a * d > c * b;
}

// Wave all-reduce of a candidate (num, den, idx) under "larger ratio, then
// lower index"; invalid candidates carry idx = INT_MAX and lose to any valid.
__device__ __forceinline__ void better_of(int& num, int& den, int& idx, int n2, int d2, int i2) {
    const bool v1 = idx != 0x7FFFFFFF, v2 = i2 != 0x7FFFFFFF;
    bool take;
    if (!v2) take = false;
    else if (!v1) take = true;
    else if (ratio_gt(n2, d2, num, den)) take = true;
    else if (ratio_gt(num, den, n2, d2)) take = false;
    else take = i2 < idx;
    if (take) {
        num = n2;
        den = d2;
        idx = i2;
    }
}

template <int D>
__device__ __forceinline__ void argmax_step(int& num, int& den, int& idx) {
    const int n2 = xstepi<D>(num), d2 = xstepi<D>(den), i2 = xstepi<D>(idx);
    better_of(num, den, idx, n2, d2, i2);
}

__device__ __forceinline__ void wave_argmax(int& num, int& den, int& idx) {
    argmax_step<1>(num, den, idx);
    argmax_step<2>(num, den, idx);
    argmax_step<4>(num, den, idx);
    argmax_step<8>(num, den, idx);
    argmax_step<16>(num, den, idx);
    argmax_step<32>(num, den, idx);
    num = __builtin_amdgcn_readfirstlane(num);
    den = __builtin_amdgcn_readfirstlane(den);
    idx = __builtin_amdgcn_readfirstlane(idx);
}

// Wave all-reduce of (load, idx) under "smaller load, then lower index".
template <int D>
__device__ __forceinline__ void argmin_step(double& v, int& idx) {
    const double v2 = xstep_f64<D>(v);
    const int i2 = xstepi<D>(idx);
    if (v2 < v || (v2 == v && i2 < idx)) {
        v = v2;
        idx = i2;
    }
}

__device__ __forceinline__ void wave_argmin(double& v, int& idx) {
    argmin_step<1>(v, idx);
    argmin_step<2>(v, idx);
    argmin_step<4>(v, idx);
    argmin_step<8>(v, idx);
    argmin_step<16>(v, idx);
    argmin_step<32>(v, idx);
    idx = __builtin_amdgcn_readfirstlane(idx);
    v = readlane_f64(v, 0);
}

__global__ void __launch_bounds__(kEplbThreads)
eplb_kernel(const EplbArgs a)
{
    extern __shared__ __align__(16) int esm[];
    const int E = a.E, P = a.num_phys, NP = a.num_packs;
    int* w = esm;                 // [E] weights (negative read as 0)
    int* cnt = w + E;             // [E] replicas per expert
    int* p2l = cnt + E;           // [P] physical -> logical
    int* prank = p2l + P;         // [P] replica number
    int* order = prank + P;       // [P] replicas, heaviest first
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int e = tid; e < E; e += kEplbThreads) {
        const int v = a.weight[e];
        w[e] = v > 0 ? v : 0;
        p2l[e] = e;
        prank[e] = 0;
    }
    __syncthreads();

    // ---- replicate_experts (wave 0; lane l owns experts l, l+64, ...)
    if (wave == 0) {
        int wl[kPerLane], cl[kPerLane];
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int e = lane + 64 * j;
            wl[j] = e < E ? w[e] : 0;
            cl[j] = 1;
        }
        for (int i = E; i < P; ++i) {
            int num = 0, den = 1, idx = 0x7FFFFFFF;
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) {
                const int e = lane + 64 * j;
                if (e < E) better_of(num, den, idx, wl[j], cl[j], e);
            }
            wave_argmax(num, den, idx);
            if (lane == (idx & 63)) {
#pragma unroll
                for (int j = 0; j < kPerLane; ++j)
                    if (lane + 64 * j == idx) {
                        if (lane == (idx & 63)) {
                            p2l[i] = idx;
                            prank[i] = cl[j];
                        }
                        cl[j] += 1;
                    }
            }
        }
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int e = lane + 64 * j;
            if (e < E) cnt[e] = cl[j];
        }
    }
    __syncthreads();

    // ---- sort the replicas by per-replica load (heaviest first, then index)
    for (int i = tid; i < P; i += kEplbThreads) {
        const int li = p2l[i];
        const int64_t ni = w[li], di = cnt[li];
        int rank = 0;
        for (int j = 0; j < P; ++j) {
            const int lj = p2l[j];
            const int64_t nj = w[lj], dj = cnt[lj];
            const int64_t l = nj * di, r = ni * dj;
            rank += (l > r || (l == r && j < i)) ? 1 : 0;
        }
        order[rank] = i;
    }
    __syncthreads();

    // ---- balanced_packing (wave 0; lane l owns packs l, l+64, ...)
    if (wave == 0) {
        const int cap = P / NP;
        double ld[kPerLane];
        int fill[kPerLane];
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            ld[j] = 0.0;
            fill[j] = 0;
        }
        for (int n = 0; n < P; ++n) {
            const int i = order[n];
            const int li = p2l[i];
            double v = 1.0e308;
            int idx = 0x7FFFFFFF;
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) {
                const int b = lane + 64 * j;
                if (b < NP && fill[j] < cap && (ld[j] < v || (ld[j] == v && b < idx))) {
                    v = ld[j];
                    idx = b;
                }
            }
            wave_argmin(v, idx);
            if (lane == (idx & 63)) {
#pragma unroll
                for (int j = 0; j < kPerLane; ++j)
                    if (lane + 64 * j == idx) {
                        a.pack[i] = idx;
                        a.slot[i] = fill[j];
                        fill[j] += 1;
                        ld[j] += double(w[li]) / double(cnt[li]);
                    }
            }
        }
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int b = lane + 64 * j;
            if (b < NP) a.pack_load[b] = ld[j];
        }
    }
    __syncthreads();
    for (int i = tid; i < P; i += kEplbThreads) {
        a.phy2log[i] = p2l[i];
        a.phy_rank[i] = prank[i];
    }
    for (int e = tid; e < E; e += kEplbThreads) a.logcnt[e] = cnt[e];
}

}  // namespace

size_t eplb_lds_bytes(int E, int num_phys) { return (size_t(2) * E + size_t(3) * num_phys) * 4; }

hipError_t launch_eplb(const EplbArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(eplb_kernel, dim3(1), dim3(kEplbThreads), eplb_lds_bytes(a.E, a.num_phys), st, a);
    return hipGetLastError();
}

}  // namespace moe
