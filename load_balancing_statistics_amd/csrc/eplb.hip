// eplb.hip -- EPLB placement over the routing counts: replicate experts, then
// pack the replicas onto GPUs (page cnvsn.com/news/335486, section 4.1.2).
//
// replicate_experts: each logical expert starts with one replica; while the
// physical count is below num_phys the expert with the largest load per
// replica, weight[e] / logcnt[e], gets another (physical E + r is the r-th
// copy).  balanced_packing: the replicas, weighted weight / logcnt of their
// expert, are taken heaviest first and each goes to the lightest pack that is
// not yet full (num_phys / num_packs replicas per pack).
// Per-replica loads are compared exactly as cross products (below 2^43:
// weights < 2^31, replica counts <= 2^12); ties go to the lower expert /
// replica / pack index; pack loads are fp64 sums in placement order.
//
// One workgroup.  The two greedy loops are sequential by nature; each runs in
// wave 0 over candidates spread across the lanes, and keeps every candidate's
// rank in the loop's order (rank 0 is the next pick), so a step is one ballot
// to find rank 0 and one ballot-popcount to re-rank the candidate that just
// changed -- no reduction tree per step.
//
// The replication picks, in order, the K = num_phys - E largest of the values
// w_e / c (c = 1, 2, ...; ties to the lower expert): each expert's values
// fall with c, so the greedy choice is a merge of sorted lists.  Only the K
// heaviest experts can therefore ever be picked (each of them has its w_e / 1
// ahead of every lighter expert's values), and they alone are candidates.
// The experts are ordered by weight and the replicas by per-replica load with
// a bitonic sort over the workgroup whose partners closer than a wave are
// exchanged between lanes and the others through LDS.
#include "route_common.hpp"

namespace moe {
namespace {

using namespace dev;

constexpr int kEplbThreads = 1024;
constexpr int kMaxSortPerThread = MOE_EPLB_MAX_PHYS / kEplbThreads;
constexpr int kNoRank = 0x7FFFFFFF;
static_assert(MOE_ROUTE_MAX_E <= kEplbThreads && MOE_ROUTE_MAX_E <= 1024, "one expert per thread, 10-bit index");
static_assert(MOE_EPLB_MAX_PHYS % kEplbThreads == 0, "whole sort slots per thread");

template <int D>
MOE_DEV int xl_i(int v) { return __float_as_int(xor_lane<D>(__int_as_float(v))); }

// Expert sort element: (weight << 10 | (1023 - expert)) + 1, larger first, so
// heavier experts lead and equal weights keep the lower index first; 0 pads.
struct EKey {
    int lo, hi;
    MOE_DEV uint64_t v() const { return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo); }
    MOE_DEV bool before(const EKey& b) const { return v() > b.v(); }
    template <int D>
    MOE_DEV EKey xl() const { return {xl_i<D>(lo), xl_i<D>(hi)}; }
    MOE_DEV void store(int* s0, int* s1, int*, int p) const { s0[p] = lo; s1[p] = hi; }
    static MOE_DEV EKey load(const int* s0, const int* s1, const int*, int p) { return {s0[p], s1[p]}; }
};

// Replica sort element: load n / d of its expert (n = -1 pads, sorting
// last) and the replica index; larger load first, then lower index.
struct Rep {
    int n, d, i;
    MOE_DEV bool before(const Rep& b) const {
        const double l = double(n) * double(b.d), r = double(b.n) * double(d);
        return l > r || (l == r && i < b.i);
    }
    template <int D>
    MOE_DEV Rep xl() const { return {xl_i<D>(n), xl_i<D>(d), xl_i<D>(i)}; }
    MOE_DEV void store(int* s0, int* s1, int* s2, int p) const { s0[p] = n; s1[p] = d; s2[p] = i; }
    static MOE_DEV Rep load(const int* s0, const int* s1, const int* s2, int p) { return {s0[p], s1[p], s2[p]}; }
};

// One compare-exchange of element i (held: me, partner's: other) in the
// stage of block size k and distance j: the pair ends in "before" order when
// the block ascends ((i & k) == 0), reversed otherwise.  Keys are distinct
// (equal ones are identical pads), so one comparison decides: the lower
// element of an ascending pair takes the partner when the partner comes
// first, and every other case is that decision flipped.
template <class T>
MOE_DEV T bitonic_cx(const T& me, const T& other, int i, int j, int k) {
    const bool flip = ((i & j) != 0) != ((i & k) != 0);
    return (other.before(me) != flip) ? other : me;
}

template <int D, class T, int M>
MOE_DEV void bitonic_lanes(T (&x)[M], int n2, int k) {
    const int t = threadIdx.x, wave_first = t & ~63;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        if (wave_first + m * kEplbThreads < n2) {  // wave-uniform
            const T y = x[m].template xl<D>();
            x[m] = bitonic_cx(x[m], y, t + m * kEplbThreads, D, k);
        }
    }
}

// Bitonic sort of n2 (a power of two, <= M * kEplbThreads) elements into
// "before" order; thread t holds elements t + m * kEplbThreads in x[m].
// s0..s2: LDS exchange arrays of n2 ints.  Every thread of the block calls it.
template <class T, int M>
MOE_DEV void block_bitonic(T (&x)[M], int n2, int* s0, int* s1, int* s2) {
    const int t = threadIdx.x;
    for (int k = 2; k <= n2; k <<= 1) {
        for (int j = k >> 1; j >= 64; j >>= 1) {
            T y[M];
            if (j >= kEplbThreads) {
                // partner in the same thread
                const int mj = j / kEplbThreads;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    y[m] = x[m];
#pragma unroll
                    for (int c = 0; c < M; ++c)
                        if ((m ^ mj) == c) y[m] = x[c];
                }
            } else {
                // partner in another wave: through LDS
#pragma unroll
                for (int m = 0; m < M; ++m)
                    if (t + m * kEplbThreads < n2) x[m].store(s0, s1, s2, t + m * kEplbThreads);
                __syncthreads();
#pragma unroll
                for (int m = 0; m < M; ++m)
                    if (t + m * kEplbThreads < n2) y[m] = T::load(s0, s1, s2, (t + m * kEplbThreads) ^ j);
                __syncthreads();
            }
#pragma unroll
            for (int m = 0; m < M; ++m)
                if (t + m * kEplbThreads < n2) x[m] = bitonic_cx(x[m], y[m], t + m * kEplbThreads, j, k);
        }
        // partners in the same wave
        if (k > 32) bitonic_lanes<32>(x, n2, k);
        if (k > 16) bitonic_lanes<16>(x, n2, k);
        if (k > 8) bitonic_lanes<8>(x, n2, k);
        if (k > 4) bitonic_lanes<4>(x, n2, k);
        if (k > 2) bitonic_lanes<2>(x, n2, k);
        bitonic_lanes<1>(x, n2, k);
    }
}

template <int CTRL>
MOE_DEV double dpp_inf_f64(double v) {
    // DPP move of a double; lanes without a source read +inf
    const uint64_t u = uint64_t(__double_as_longlong(v));
    const int lo = __builtin_amdgcn_update_dpp(0, int(uint32_t(u)), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0x7FF00000, int(uint32_t(u >> 32)), CTRL, 0xF, 0xF, false);
    return __longlong_as_double((long long)((uint64_t(uint32_t(hi)) << 32) | uint32_t(lo)));
}

// Minimum of v over the lanes below this one (+inf on lane 0): scans inside
// each 16-lane row (row_shr 1, 2, 4, 8), then the rows' totals in order.
MOE_DEV double wave_excl_prefix_min(double v) {
    const int lane = threadIdx.x & 63;
    double in = v;
    in = fmin(in, dpp_inf_f64<0x111>(in));
    in = fmin(in, dpp_inf_f64<0x112>(in));
    in = fmin(in, dpp_inf_f64<0x114>(in));
    in = fmin(in, dpp_inf_f64<0x118>(in));
    const double ex = dpp_inf_f64<0x111>(in);  // exclusive inside the row
    const double r1 = readlane_f64(in, 15);
    const double r2 = fmin(r1, readlane_f64(in, 31));
    const double r3 = fmin(r2, readlane_f64(in, 47));
    const int row = lane >> 4;
    const double before = row == 0 ? INFINITY : (row == 1 ? r1 : (row == 2 ? r2 : r3));
    return fmin(ex, before);
}

MOE_DEV double shfl_down_f64(double v) {
    const uint64_t u = uint64_t(__double_as_longlong(v));
    const int lo = __shfl_down(int(uint32_t(u)), 1), hi = __shfl_down(int(uint32_t(u >> 32)), 1);
    return __longlong_as_double((long long)((uint64_t(uint32_t(hi)) << 32) | uint32_t(lo)));
}

// Pack on a lane: load, index, fill; order (load, index) ascending.
struct PackSlot {
    double ld;
    int pid, fl;
    MOE_DEV bool before(const PackSlot& b) const { return ld < b.ld || (ld == b.ld && pid < b.pid); }
    template <int D>
    MOE_DEV PackSlot xl() const {
        const uint64_t u = uint64_t(__double_as_longlong(ld));
        const int lo = xl_i<D>(int(uint32_t(u))), hi = xl_i<D>(int(uint32_t(u >> 32)));
        return {__longlong_as_double((long long)((uint64_t(uint32_t(hi)) << 32) | uint32_t(lo))), xl_i<D>(pid),
                xl_i<D>(fl)};
    }
};

template <int D>
MOE_DEV void wave_sort_stage(PackSlot& x, int k) {
    const int lane = threadIdx.x & 63;
    x = bitonic_cx(x, x.template xl<D>(), lane, D, k);
}

// Bitonic sort of the wave's 64 lanes by (load, index).
MOE_DEV void wave_sort_packs(double& ld, int& pid, int& fl) {
    PackSlot x{ld, pid, fl};
    wave_sort_stage<1>(x, 2);
    wave_sort_stage<2>(x, 4); wave_sort_stage<1>(x, 4);
    wave_sort_stage<4>(x, 8); wave_sort_stage<2>(x, 8); wave_sort_stage<1>(x, 8);
    wave_sort_stage<8>(x, 16); wave_sort_stage<4>(x, 16); wave_sort_stage<2>(x, 16); wave_sort_stage<1>(x, 16);
    wave_sort_stage<16>(x, 32); wave_sort_stage<8>(x, 32); wave_sort_stage<4>(x, 32);
    wave_sort_stage<2>(x, 32); wave_sort_stage<1>(x, 32);
    wave_sort_stage<32>(x, 64); wave_sort_stage<16>(x, 64); wave_sort_stage<8>(x, 64);
    wave_sort_stage<4>(x, 64); wave_sort_stage<2>(x, 64); wave_sort_stage<1>(x, 64);
    ld = x.ld;
    pid = x.pid;
    fl = x.fl;
}

MOE_DEV int wave_sum_i(int v) {
    v += xstepi<1>(v);
    v += xstepi<2>(v);
    v += xstepi<4>(v);
    v += xstepi<8>(v);
    return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
           (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// EPL / PPL: candidate experts / packs per lane of wave 0 (powers of two).
template <int EPL, int PPL>
__global__ void __launch_bounds__(kEplbThreads)
eplb_kernel(const EplbArgs a)
{
    extern __shared__ __align__(16) int esm[];
    const int E = a.E, P = a.num_phys, NP = a.num_packs;
    const int K = P - E;         // replicas to add
    const int Kc = min(K, E);    // experts that can receive one
    int N2 = 1, NE = 1;
    while (N2 < P) N2 <<= 1;
    while (NE < E) NE <<= 1;
    double* wsorted = reinterpret_cast<double*>(esm);  // [P] replica weight, heaviest first
    int* w = reinterpret_cast<int*>(wsorted + P);      // [E] weights (negative read as 0)
    int* cnt = w + E;             // [E] replicas per expert
    int* p2l = cnt + E;           // [P] physical -> logical
    int* prank = p2l + P;         // [P] replica number
    int* s0 = prank + P;          // [N2] sort exchange; then the candidates,
    int* s1 = s0 + N2;            // [N2]   and the sorted replica indices
    int* s2 = s1 + N2;            // [N2]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    EKey ek[1] = {{0, 0}};
    if (tid < E) {
        const int v = a.weight[tid];
        const int wv = v > 0 ? v : 0;
        w[tid] = wv;
        cnt[tid] = 1;
        p2l[tid] = tid;
        prank[tid] = 0;
        const uint64_t key = ((uint64_t(wv) << 10) | uint64_t(1023 - tid)) + 1;
        ek[0] = {int(uint32_t(key)), int(uint32_t(key >> 32))};
    }
    if (K > 0) {
        block_bitonic(ek, NE, s0, s1, s2);
        // the Kc heaviest experts, heaviest first (s0 is free after the sort)
        if (tid < Kc) s0[tid] = 1023 - int((ek[0].v() - 1) & 1023);
    }
    __syncthreads();

    // ---- replicate_experts (wave 0; candidate of rank r starts on lane
    // r % 64, slot r / 64).  Pipelined: the next pick is the current one
    // again when no other candidate gets ahead of its new load, else the
    // current rank 1, whose values are gathered before the ranks change.
    if (wave == 0 && K > 0) {
        int ce[EPL], rk[EPL], ci[EPL], wi[EPL];
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int r = lane + 64 * j;
            const bool in = r < Kc;
            ce[j] = in ? s0[r] : 0;
            wi[j] = in ? w[ce[j]] : 0;
            ci[j] = 1;
            rk[j] = in ? r : kNoRank;
        }
        // the current pick: expert, replicas so far, weight, place (lane + 64 * slot)
        int be = __builtin_amdgcn_readlane(ce[0], 0), cb = 1, pb = 0;
        int wb = __builtin_amdgcn_readlane(wi[0], 0);
        for (int i0 = 0; i0 < K; i0 += 64) {
            const int nn = min(64, K - i0);
            int myexp = 0, mycopy = 0;
            for (int q = 0; q < nn; ++q) {
                int g_e = 0, g_c = 0, g_p = 0, g_w = 0;
                bool has = false;
#pragma unroll
                for (int j = 0; j < EPL; ++j) {
                    const bool m = rk[j] == 1;
                    g_e = m ? ce[j] : g_e;
                    g_c = m ? ci[j] : g_c;
                    g_w = m ? wi[j] : g_w;
                    g_p = m ? lane + 64 * j : g_p;
                    has |= m;
                }
                const uint64_t hm = __ballot(has);
                const int l1 = hm ? int(__builtin_ctzll(hm)) : 0;
                myexp = (lane == q) ? be : myexp;
                mycopy = (lane == q) ? cb : mycopy;
                // the others ahead of its new load wb / (cb + 1): exact
                // products below 2^43
                const int cn = cb + 1;
                int count = 0;
                if constexpr (EPL <= 2) {
#pragma unroll
                    for (int j = 0; j < EPL; ++j) {
                        const uint64_t l = uint64_t(uint32_t(wi[j])) * uint32_t(cn);
                        const uint64_t r = uint64_t(uint32_t(wb)) * uint32_t(ci[j]);
                        const bool ahead = (unsigned(rk[j] - 1) < unsigned(kNoRank - 1)) &
                                           ((l > r) | ((l == r) & (ce[j] < be)));
                        count += __popcll(__ballot(ahead));
                    }
                } else {
                    int c = 0;
#pragma unroll
                    for (int j = 0; j < EPL; ++j) {
                        const uint64_t l = uint64_t(uint32_t(wi[j])) * uint32_t(cn);
                        const uint64_t r = uint64_t(uint32_t(wb)) * uint32_t(ci[j]);
                        c += int((unsigned(rk[j] - 1) < unsigned(kNoRank - 1)) &
                                 ((l > r) | ((l == r) & (ce[j] < be))));
                    }
                    count = wave_sum_i(c);
                }
                const int bsel = (lane == (pb & 63)) ? (pb >> 6) : -1;
#pragma unroll
                for (int j = 0; j < EPL; ++j) {
                    const bool me = bsel == j;
                    const int r = rk[j];
                    ci[j] = me ? cn : ci[j];
                    rk[j] = me ? count : r - int((r >= 1) & (r <= count));
                }
                if (count > 0) {
                    be = __builtin_amdgcn_readlane(g_e, l1);
                    cb = __builtin_amdgcn_readlane(g_c, l1);
                    pb = __builtin_amdgcn_readlane(g_p, l1);
                    wb = __builtin_amdgcn_readlane(g_w, l1);
                } else {
                    cb = cn;
                }
            }
            if (lane < nn) {
                p2l[E + i0 + lane] = myexp;
                prank[E + i0 + lane] = mycopy;
            }
        }
#pragma unroll
        for (int j = 0; j < EPL; ++j)
            if (lane + 64 * j < Kc) cnt[ce[j]] = ci[j];
    }
    __syncthreads();

    // ---- replicas heaviest first
    if (N2 <= kEplbThreads) {
        Rep xr[1];
        xr[0] = {-1, 1, kNoRank};
        if (tid < P) {
            const int e = p2l[tid];
            xr[0] = {w[e], cnt[e], tid};
        }
        block_bitonic(xr, N2, s0, s1, s2);
        if (tid < P) {
            s2[tid] = xr[0].i;
            wsorted[tid] = double(xr[0].n) / double(xr[0].d);
        }
    } else {
        Rep xr[kMaxSortPerThread];
#pragma unroll
        for (int m = 0; m < kMaxSortPerThread; ++m) {
            const int i = tid + m * kEplbThreads;
            if (i < P) {
                const int e = p2l[i];
                xr[m] = {w[e], cnt[e], i};
            } else {
                xr[m] = {-1, 1, kNoRank};
            }
        }
        block_bitonic(xr, N2, s0, s1, s2);
#pragma unroll
        for (int m = 0; m < kMaxSortPerThread; ++m) {
            const int i = tid + m * kEplbThreads;
            if (i < P) {
                s2[i] = xr[m].i;
                wsorted[i] = double(xr[m].n) / double(xr[m].d);
            }
        }
    }
    __syncthreads();

    // ---- balanced_packing
    if constexpr (PPL == 1) {
        // Up to 64 packs (wave 0): the open packs sorted by (load, index)
        // across the lanes, lightest on lane 0; closed packs and lanes past
        // num_packs hold +inf and sort last.  A run of t items goes at once:
        // item n + r to the pack on lane r, which is the lightest open pack
        // when its turn comes as long as every pack filled earlier in the run
        // is now strictly heavier than lane r's (a prefix minimum over the
        // lanes; a tie ends the run, which only makes it shorter).  A pack's
        // load is stored when it fills -- every pack ends full.
        if (wave == 0) {
            const int cap = P / NP;
            int pid = lane, fl = 0;
            double ld = lane < NP ? 0.0 : INFINITY;
            int m = NP;  // open packs: lanes 0..m-1
            for (int n = 0; n < P;) {
                const int tmax = min(m, P - n);
                const bool in = lane < tmax;
                const int it = in ? s2[n + lane] : 0;
                const double wt = in ? wsorted[n + lane] : 0.0;
                const double lnew = ld + wt;
                const bool closes = fl + 1 == cap;
                const double pm = wave_excl_prefix_min(in && !closes ? lnew : INFINITY);
                const uint64_t inval = ~__ballot(in && pm > ld);
                const int t = inval ? int(__builtin_ctzll(inval)) : 64;
                const bool take = lane < t;
                if (take && it >= 0 && it < P) {
                    a.pack[it] = pid;
                    a.slot[it] = fl;
                }
                if (take && closes) a.pack_load[pid] = lnew;
                ld = take ? (closes ? INFINITY : lnew) : ld;
                fl += int(take);
                const int m_old = m;
                m -= __popcll(__ballot(take && closes));
                n += t;
                if (t == 1) {
                    // lane 0 moved: behind the open packs now lighter, the
                    // lanes between shift down one
                    const double l0 = readlane_f64(ld, 0);
                    const int p0 = __builtin_amdgcn_readlane(pid, 0), f0 = __builtin_amdgcn_readlane(fl, 0);
                    const bool ahead = (lane >= 1) & (lane < m_old) & ((ld < l0) | ((ld == l0) & (pid < p0)));
                    const int g = __popcll(__ballot(ahead));
                    const double ldn = shfl_down_f64(ld);
                    const int pidn = __shfl_down(pid, 1), fln = __shfl_down(fl, 1);
                    ld = lane < g ? ldn : (lane == g ? l0 : ld);
                    pid = lane < g ? pidn : (lane == g ? p0 : pid);
                    fl = lane < g ? fln : (lane == g ? f0 : fl);
                } else {
                    wave_sort_packs(ld, pid, fl);
                }
            }
        }
    } else if (wave == 0) {
        // More packs: ranks kept per pack, one item per step.
        const int cap = P / NP;
        double ld[PPL];
        int fill[PPL], rk[PPL];
#pragma unroll
        for (int j = 0; j < PPL; ++j) {
            const int b = lane + 64 * j;
            ld[j] = 0.0;
            fill[j] = 0;
            rk[j] = b < NP ? b : kNoRank;
        }
        int open = NP;
        int best = 0, fb = 0;  // the current pack and its fill
        double lold = 0.0;     // and its load
        for (int n0 = 0; n0 < P; n0 += 64) {
            // the next 64 replicas in order, one per lane, then broadcast
            const int myi = (n0 + lane < P) ? s2[n0 + lane] : 0;
            const double myw = (n0 + lane < P) ? wsorted[n0 + lane] : 0.0;
            const int nn = min(64, P - n0);
            int mypack = 0, myslot = 0;
            for (int q = 0; q < nn; ++q) {
                const double wt = readlane_f64(myw, q);
                double g_l = 0.0;
                int g_f = 0, g_b = 0;
                bool has = false;
#pragma unroll
                for (int j = 0; j < PPL; ++j) {
                    const bool m = rk[j] == 1;
                    g_l = m ? ld[j] : g_l;
                    g_f = m ? fill[j] : g_f;
                    g_b = m ? lane + 64 * j : g_b;
                    has |= m;
                }
                const uint64_t hm = __ballot(has);
                const int l1 = hm ? int(__builtin_ctzll(hm)) : 0;
                mypack = (lane == q) ? best : mypack;
                myslot = (lane == q) ? fb : myslot;
                const double lnew = lold + wt;
                const bool fills = fb + 1 == cap;
                int count = 0;
                if constexpr (PPL <= 2) {
#pragma unroll
                    for (int j = 0; j < PPL; ++j) {
                        const int b = lane + 64 * j;
                        const bool ahead = (unsigned(rk[j] - 1) < unsigned(kNoRank - 1)) &
                                           ((ld[j] < lnew) | ((ld[j] == lnew) & (b < best)));
                        count += __popcll(__ballot(ahead));
                    }
                } else {
                    int c = 0;
#pragma unroll
                    for (int j = 0; j < PPL; ++j) {
                        const int b = lane + 64 * j;
                        c += int((unsigned(rk[j] - 1) < unsigned(kNoRank - 1)) &
                                 ((ld[j] < lnew) | ((ld[j] == lnew) & (b < best))));
                    }
                    count = wave_sum_i(c);
                }
                // ranks 1..upto move up one; this pack takes rank `mine`
                const int upto = fills ? open - 1 : count;
                const int mine = fills ? kNoRank : count;
                const int bsel = (lane == (best & 63)) ? (best >> 6) : -1;
#pragma unroll
                for (int j = 0; j < PPL; ++j) {
                    const bool me = bsel == j;
                    const int r = rk[j];
                    ld[j] = me ? lnew : ld[j];
                    fill[j] = me ? fb + 1 : fill[j];
                    rk[j] = me ? mine : r - int((r >= 1) & (r <= upto));
                }
                open -= int(fills);
                if (fills || count > 0) {
                    best = __builtin_amdgcn_readlane(g_b, l1);
                    fb = __builtin_amdgcn_readlane(g_f, l1);
                    lold = readlane_f64(g_l, l1);
                } else {
                    fb += 1;
                    lold = lnew;
                }
            }
            if (n0 + lane < P && myi >= 0 && myi < P) {
                a.pack[myi] = mypack;
                a.slot[myi] = myslot;
            }
        }
#pragma unroll
        for (int j = 0; j < PPL; ++j) {
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

size_t eplb_lds_bytes(int E, int num_phys) {
    size_t n2 = 1;
    while (n2 < size_t(num_phys)) n2 <<= 1;
    return size_t(num_phys) * 8 + (size_t(2) * E + size_t(2) * num_phys + 3 * n2) * 4;
}

template <int EPL, int PPL>
static hipError_t launch_eplb_t(const EplbArgs& a, size_t lds, hipStream_t st) {
    auto kern = eplb_kernel<EPL, PPL>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(1), dim3(kEplbThreads), lds, st, a);
    return hipGetLastError();
}

template <int EPL>
static hipError_t launch_eplb_e(const EplbArgs& a, size_t lds, hipStream_t st) {
    const int ppl = (a.num_packs + 63) / 64;
    if (ppl <= 1) return launch_eplb_t<EPL, 1>(a, lds, st);
    if (ppl <= 2) return launch_eplb_t<EPL, 2>(a, lds, st);
    if (ppl <= 4) return launch_eplb_t<EPL, 4>(a, lds, st);
    if (ppl <= 8) return launch_eplb_t<EPL, 8>(a, lds, st);
    return launch_eplb_t<EPL, 16>(a, lds, st);
}

hipError_t launch_eplb(const EplbArgs& a, hipStream_t st) {
    const size_t lds = eplb_lds_bytes(a.E, a.num_phys);
    const int kc = std::min(a.num_phys - a.E, a.E);
    const int epl = std::max(1, (kc + 63) / 64);
    if (epl <= 1) return launch_eplb_e<1>(a, lds, st);
    if (epl <= 2) return launch_eplb_e<2>(a, lds, st);
    if (epl <= 4) return launch_eplb_e<4>(a, lds, st);
    if (epl <= 8) return launch_eplb_e<8>(a, lds, st);
    return launch_eplb_e<16>(a, lds, st);
}

}  // namespace moe
