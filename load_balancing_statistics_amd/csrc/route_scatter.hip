// route_scatter.hip -- the stable capacity-limited dispatch permutation.
//
// Dispatch order: inside each microbatch the assignments (t, j) are grouped by
// expert, experts ascending, and keep their (t, j) order inside an expert.
// The r-th assignment of an expert (r counted from 0) is dropped when r >= C
// (page mhpq.cn/news/998159 section 4.5: tokens beyond an expert's capacity
// are dropped).  Block b handles the same rows as row block b; its
// assignments to expert e start at
//   offsets[e] + (count of e in the earlier splits) + (count of e in the
//   earlier blocks of its split).
// Inside the block each wave takes a contiguous slice; within a 64-assignment
// chunk the rank among equal experts comes from ballots over the expert-id
// bits, so the order is exact and deterministic.
#include "route_common.hpp"

namespace moe {
namespace {

using namespace dev;

constexpr int kScatWaves = 16;
constexpr int kScatThreads = kScatWaves * 64;
constexpr int kCachedChunks = 8;  // 64-assignment chunks kept in registers per wave

// In-place exclusive scan of n LDS ints v[0..n) into out[0..n] (out[n] = total).
__device__ void block_excl_scan(const int* v, int n, int* out, int* wsum) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (n + kScatThreads - 1) / kScatThreads;
    const int i0 = min(tid * per, n), i1 = min(i0 + per, n);
    int loc = 0;
    for (int i = i0; i < i1; ++i) loc += v[i];
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
        const int t = v[i];
        out[i] = run;
        run += t;
    }
    if (tid == kScatThreads - 1) out[n] = run;
    __syncthreads();
}

__global__ void __launch_bounds__(kScatThreads)
route_scatter_kernel(const ScatterArgs a)
{
    extern __shared__ __align__(16) int sm[];
    const int E = a.E;
    const int E4 = (E + 1 + 3) & ~3;
    int* offs = sm;             // [E+1]
    int* tot = sm + E4;         // [E]
    int* base = tot + E4;       // [E]
    int* wh = base + E4;        // [kScatWaves][E]
    __shared__ int wsum[kScatWaves];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int mb = blockIdx.x / a.bpm, bi = blockIdx.x - (blockIdx.x / a.bpm) * a.bpm;
    const int my_split = bi / (kScanWaves * kScanPerWave);
    long row_begin, row_end;
    block_rows(blockIdx.x, a.bpm, a.Tm, row_begin, row_end);
    const long segment = long(mb) * a.Tm * a.k;  // start of the microbatch in perm
    const long seglen = long(a.Tm) * a.k;

    // this block's assignments, one contiguous slice per wave
    const long a0 = row_begin * a.k, a1 = row_end * a.k;
    long q = (a1 - a0 + kScatWaves - 1) / kScatWaves;
    q = (q + 63) & ~63L;
    const long s0 = min(a0 + wave * q, a1), s1 = min(s0 + q, a1);

    // ---- issue every independent global load first
    int eid[kCachedChunks];
#pragma unroll
    for (int u = 0; u < kCachedChunks; ++u) {
        const long i = s0 + long(u) * 64 + lane;
        eid[u] = (i < s1) ? a.topk_idx[i] : -1;
    }
    for (int e = tid; e < E; e += kScatThreads) {
        tot[e] = 0;
        base[e] = a.colprefix[long(blockIdx.x) * E + e];
    }
    for (int i = tid; i < kScatWaves * E; i += kScatThreads) wh[i] = 0;
    __syncthreads();
    // per-split counts: all (split, expert) pairs loaded at once, summed with
    // integer LDS atomics (order-independent)
    {
        const int n = a.nsplit * E;
        const int32_t* st = a.split_tot + long(mb) * n;
        for (int i0 = 0; i0 < n; i0 += 4 * kScatThreads) {
            int v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * kScatThreads + tid;
                v[u] = (i < n) ? st[i] : 0;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * kScatThreads + tid;
                if (i < n) {
                    const int sp = i / E, e = i - sp * E;
                    atomicAdd(&tot[e], v[u]);
                    if (sp < my_split) atomicAdd(&base[e], v[u]);
                }
            }
        }
    }
    __syncthreads();

    block_excl_scan(tot, E, offs, wsum);
    for (int e = tid; e < E; e += kScatThreads) base[e] += offs[e];

    // ---- per-wave histogram of the slice, then per-wave bases
    int* mywh = wh + wave * E;
    int internal = 0;
#pragma unroll
    for (int u = 0; u < kCachedChunks; ++u) {
        const int e = eid[u];
        if (e >= 0 && e < E) atomicAdd(&mywh[e], 1);
    }
    for (long c = s0 + long(kCachedChunks) * 64; c < s1; c += 64) {
        const long i = c + lane;
        if (i < s1) {
            const int e = a.topk_idx[i];
            if (e >= 0 && e < E) atomicAdd(&mywh[e], 1);
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kScatThreads) {
        int run = base[e];
        for (int w = 0; w < kScatWaves; ++w) {
            const int t = wh[w * E + e];
            wh[w * E + e] = run;
            run += t;
        }
    }
    __syncthreads();

    // ---- stable ranks inside 64-assignment chunks, in order
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int u = 0;
    for (long c = s0; c < s1; c += 64, ++u) {
        const long i = c + lane;
        bool valid = i < s1;
        int e;
        if (u < kCachedChunks) {
            e = eid[0];
#pragma unroll
            for (int v = 1; v < kCachedChunks; ++v) e = (u == v) ? eid[v] : e;
        } else {
            e = valid ? a.topk_idx[i] : 0;
        }
        if (valid && (e < 0 || e >= E)) {
            internal = 1;
            valid = false;
        }
        if (!valid) e = 0;
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
    const size_t E4 = size_t((a.E + 1 + 3) & ~3);
    const size_t lds = (3 * E4 + size_t(kScatWaves) * a.E) * 4;
    hipLaunchKernelGGL(route_scatter_kernel, dim3(c.B), dim3(kScatThreads), lds, st, a);
    return hipGetLastError();
}

}  // namespace moe
