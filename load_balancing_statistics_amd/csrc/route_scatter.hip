// route_scatter.hip -- the stable capacity-limited dispatch permutation.
//
// Dispatch order: inside each microbatch the assignments (t, j) are grouped by
// expert, experts ascending, and keep their (t, j) order inside an expert.
// The r-th assignment of an expert (r counted from 0) is dropped when r >= C
// (page mhpq.cn/news/998159 section 4.5: tokens beyond an expert's capacity
// are dropped).  Block b handles the same rows as row block b; its
// assignments to expert e start at
//   offsets[e] + (count of e in the earlier splits) + (count of e in the
//   earlier blocks of its split),
// offsets being the exclusive prefix sum, in expert order, of the
// microbatch's counts (the sums of its split counts), which every block
// forms for itself.  The first six blocks of each microbatch also share
// the counts, the offsets and the balance statistics, one reduced quantity
// each -- or, when the row blocks and one more workgroup per microbatch can
// run at once, that extra workgroup forms them all, so that no block adds
// them to its share of the rows.
//
// A token picks an expert at most once (its top-k are distinct), so inside an
// expert the (t, j) order is the token order.  The block walks its rows in
// windows; in a window each wave owns a contiguous run of rows, row r of the
// run being bit r of a 64-bit mask per (wave, expert).  The lanes of a row
// hold contiguous chunks of its k slots, read as 16-byte vectors when the
// chunks are whole vectors (every load instruction then covers contiguous
// bytes).  Every slot (r, j) ORs its bit into the mask of its expert; a
// slot's rank among the wave's assignments to that expert is then the
// popcount of the mask below its bit, and the wave's count is the whole
// popcount.  An exclusive scan over the waves and one over the experts place
// every slot in an LDS copy of the window sorted by expert, which is written
// to the permutation in that order: the block's assignments to one expert
// land in consecutive words, so the stores coalesce.  dropped and inv_perm
// are indexed by the assignment and are stored from the ranking pass.
#include <climits>

#include "route_common.hpp"

namespace moe {
namespace {

using namespace dev;

constexpr int kScatMaxWaves = 16;
constexpr int kSplitBatch = 8;
constexpr int kFoldLoads = 16;  // row blocks a thread sums when the scatter folds the combine in
constexpr int kFoldGroups = 16;  // at most this many row-block groups per expert

// Exclusive scan of n LDS ints v[0..n) into out[0..n] (out[n] = total).
__device__ void block_excl_scan(const int* v, int n, int* out, int* wsum) {
    const int nthr = blockDim.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (n + nthr - 1) / nthr;
    const int i0 = min(tid * per, n), i1 = min(i0 + per, n);
    const bool busy = wave * 64 * per < n;  // wave-uniform: the wave holds entries
    int loc = 0;
    for (int i = i0; i < i1; ++i) loc += v[i];
    int incl = 0;
    if (busy) {
        incl = wave_incl_scan_i(loc);
        if (lane == 63) wsum[wave] = incl;
    }
    __syncthreads();
    if (busy) {
        int run = incl - loc;
        for (int w = 0; w < wave; ++w) run += wsum[w];
        for (int i = i0; i < i1; ++i) {
            const int t = v[i];
            out[i] = run;
            run += t;
        }
        if (i1 == n && i0 < n) out[n] = run;
    }
    if (n == 0 && tid == 0) out[0] = 0;
    __syncthreads();
}

// Logical block of a workgroup: workgroups are dealt to the 8 XCDs in turn,
// so consecutive logical blocks -- whose runs of each expert are adjacent in
// the permutation -- are given to workgroups of one XCD, and the partial
// cache lines they share meet in one L2.
__device__ __forceinline__ int logical_block(int n) {
    const int b = blockIdx.x;
    return (n % 8 == 0) ? (b % 8) * (n / 8) + b / 8 : b;
}

// Slots (r, j) a lane ranks per window: rows get 64/rows-per-wave lanes, and
// the host caps rows per wave at 64/next_pow2(ceil(k/KM)), so ceil(k/lanes)
// never exceeds KM.
constexpr int KM = 8;

// NW waves per block (the launch uses exactly NW * 64 threads).
template <int NW>
__global__ void __launch_bounds__(NW * 64)
route_scatter_kernel(const ScatterArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int E = a.E, k = a.k;
    const int E4 = (E + 1 + 3) & ~3;
    uint64_t* gm = reinterpret_cast<uint64_t*>(smem);      // [NW][E] row masks
    int* wpre = reinterpret_cast<int*>(gm + NW * E);        // [NW][E] e's assignments in the earlier waves
    int2* st = reinterpret_cast<int2*>(wpre + NW * E);      // [stage] {assignment, segment place}, expert order
    int* base = reinterpret_cast<int*>(st + NW * a.rows_per_wave * k);  // [E] the block's next place for e
    int* lim = base + E4;                                   // [E] first dropped place of e
    int* tot = lim + E4;                                    // [E4] window counts
    int* lofs = tot + E4;                                   // [E4] window-local expert starts
    __shared__ int wsum[kScatMaxWaves];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // With stats_sep, workgroups B .. B + n_micro - 1 only form their
    // microbatch's offsets and statistics (as its first row block would).
    const bool stats_only = a.stats_sep && int(blockIdx.x) >= a.B;
    const int b = stats_only ? (int(blockIdx.x) - a.B) * a.bpm : logical_block(a.B);
    const int mb = b / a.bpm, bi = b - mb * a.bpm;
    const int my_split = bi / (kScanWaves * kScanPerWave);
    long row_begin, row_end;
    block_rows(b, a.bpm, a.Tm, row_begin, row_end);
    const long segment = long(mb) * a.Tm * k;  // start of the microbatch in perm
    const long seglen = long(a.Tm) * k;
    const int WR = NW * a.rows_per_wave;       // rows per window

    // slot layout of a window: rows per wave, lanes per row, and lane g of a
    // row holds slots j = g*KC + u, u < KC
    int ev[KM];
    long row = 0;
    int rl = 0, g = 0, KC = 1;
    bool active = false;
    auto load_window = [&](long w0) {
        const long w1 = min(w0 + long(WR), row_end);
        const int nrows = int(w1 - w0);
        const int rpw = (nrows + NW - 1) / NW;
        int rp = 1;
        while (rp < rpw) rp <<= 1;
        const int lpr = 64 / rp;
        KC = (k + lpr - 1) / lpr;
        rl = lane & (rp - 1);
        g = lane / rp;
        row = w0 + long(wave) * rpw + rl;
        active = rl < rpw && row < w1;
        const long i0 = row * k + long(g) * KC;
        if (a.vec_idx && (KC & 3) == 0) {
            // k and KC multiples of 4: a lane's chunk is KC/4 aligned vectors
#pragma unroll
            for (int q = 0; q < KM / 4; ++q) {
                const bool in = active && 4 * q < KC && g * KC + 4 * q < k;
                const int4 v = *reinterpret_cast<const int4*>(a.topk_idx + (in ? i0 + 4 * q : 0));
                ev[4 * q] = in ? v.x : -1;
                ev[4 * q + 1] = in ? v.y : -1;
                ev[4 * q + 2] = in ? v.z : -1;
                ev[4 * q + 3] = in ? v.w : -1;
            }
        } else {
#pragma unroll
            for (int u = 0; u < KM; ++u)
                ev[u] = load_or(a.topk_idx, i0 + u, active && u < KC && g * KC + u < k, -1);
        }
    };
    if (!stats_only) load_window(row_begin);
    // per expert: the microbatch's count tot[e], this block's start relative
    // to the expert's offset base[e] (the count in the microbatch's earlier
    // row blocks) and, for the statistics, the probability sum psum
    constexpr int EPT = (MOE_ROUTE_MAX_E + NW * 64 - 1) / (NW * 64);  // experts per thread
    // the statistics: all of them in the statistics workgroup, else spread
    // over the microbatch's first six row blocks (one reduced quantity
    // each; block 0 also the per-expert outputs and the aux loss), so no
    // block adds more than a sixth of them to its rows
    const int parts = a.stats_sep ? (stats_only ? kStatsAll : 0)
                    : a.bpm >= 6  ? (bi < 6 ? (1 << bi) : 0)
                                  : (bi == 0 ? kStatsAll : 0);
    const bool stats_block = parts != 0;
    const bool need_p = (parts & 1) != 0;  // only part 0 reads the probability sums
    double psum[EPT];
#pragma unroll
    for (int it = 0; it < EPT; ++it) psum[it] = 0.0;
    if (a.fold_q > 0) {
        // Few row blocks per microbatch: every block sums the row pass's
        // partials itself and no combine kernel runs.  Thread t < Q*E takes
        // expert t % E over the row blocks [q*bpm/Q, (q+1)*bpm/Q), q = t / E
        // (at most kFoldLoads of them, loaded in one round); the Q groups meet
        // in LDS -- the row masks' area, free until the first window -- and
        // are added in group order.
        const int Q = a.fold_q;
        int* fpre = reinterpret_cast<int*>(gm);
        int* ftot = fpre + Q * E;
        double* fps = reinterpret_cast<double*>(ftot + Q * E);
        const long pb = long(mb) * a.bpm;  // the microbatch's first row block
        for (int t = tid; t < Q * E; t += NW * 64) {
            const int e = t % E, q = t / E;
            const int b0 = (q * a.bpm) / Q, b1 = ((q + 1) * a.bpm) / Q;
            int cv[kFoldLoads];
            float pv[kFoldLoads];
#pragma unroll
            for (int v = 0; v < kFoldLoads; ++v) {
                const long o = (pb + ((b0 + v < b1) ? b0 + v : b0)) * E + e;
                cv[v] = a.cnt_part[o];
                pv[v] = a.P_part[o];
            }
            int pre = 0, tt = 0;
            double ps = 0.0;
#pragma unroll
            for (int v = 0; v < kFoldLoads; ++v) {
                if (b0 + v < b1) {
                    tt += cv[v];
                    pre += (b0 + v < bi) ? cv[v] : 0;
                    ps += double(pv[v]);
                }
            }
            fpre[t] = pre;
            ftot[t] = tt;
            fps[t] = ps;
        }
        // status: the flags of every row block, by logical block 0 or, with
        // statistics workgroups, by the first of them (the row pass zeroed
        // the word; the scatter only ORs bits into it)
        if (a.status && b == 0 && (stats_only || !a.stats_sep)) {
            int fl = 0;
            for (int j = tid; j < a.B; j += NW * 64) fl |= a.flag_part[j];
            if (__syncthreads_or(fl & MOE_STATUS_NONFINITE) && tid == 0)
                atomicOr(a.status, MOE_STATUS_NONFINITE);
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < EPT; ++it) {
            const int e = tid + it * NW * 64;
            if (e >= E) break;
            int pre = 0, tt = 0;
            double ps = 0.0;
            for (int q = 0; q < Q; ++q) {
                pre += fpre[q * E + e];
                tt += ftot[q * E + e];
                ps += fps[q * E + e];
            }
            tot[e] = tt;
            base[e] = pre;
            psum[it] = ps;
        }
    } else {
        // From the combine kernel: the split sums and this block's prefix
        // inside its split; the first kSplitBatch splits are loaded with the
        // prefix, in one round, and in the first block of the microbatch
        // the probability sums with them (one round trip, not two).
#pragma unroll
        for (int it = 0; it < EPT; ++it) {
            const int e = tid + it * NW * 64;
            if (e >= E) break;
            const long sb = long(mb) * a.nsplit * E + e;
            const int cp = a.colprefix[long(b) * E + e];
            int t = 0, pre = 0;
            for (int sp0 = 0; sp0 < a.nsplit; sp0 += kSplitBatch) {
                int sv[kSplitBatch];
                double pv[kSplitBatch];
#pragma unroll
                for (int v = 0; v < kSplitBatch; ++v)
                    sv[v] = load_or(a.split_tot, sb + long(sp0 + v) * E, sp0 + v < a.nsplit, 0);
                if (need_p) {
#pragma unroll
                    for (int v = 0; v < kSplitBatch; ++v)
                        pv[v] = load_or(a.split_P, sb + long(sp0 + v) * E, sp0 + v < a.nsplit, 0.0);
                }
#pragma unroll
                for (int v = 0; v < kSplitBatch; ++v) {
                    t += sv[v];
                    pre += (sp0 + v < my_split) ? sv[v] : 0;
                }
                if (need_p) {
#pragma unroll
                    for (int v = 0; v < kSplitBatch; ++v) psum[it] += pv[v];
                }
            }
            tot[e] = t;
            base[e] = pre + cp;
        }
    }
    __syncthreads();
    // offsets: exclusive prefix of the counts in expert order
    block_excl_scan(tot, E, lofs, wsum);  // ends with a barrier
    for (int e = tid; e < E; e += NW * 64) {
        const int o = lofs[e];
        base[e] += o;
        const long l = a.capacity >= 0 ? long(o) + a.capacity : long(INT32_MAX);
        lim[e] = int(l < INT32_MAX ? l : INT32_MAX);
    }
    // tot and lofs are reused by the windows only after their first
    // barrier; the row masks' LDS is free until the first window
    if (stats_block) microbatch_statistics<NW, EPT>(a, mb, tot, lofs, psum, reinterpret_cast<double*>(gm), parts);
    if (a.upd_bias && (parts & 1)) {
        // one loss-free balancing step from this (only) microbatch's counts,
        // the rule of the separate update kernel: the bias of an expert
        // loaded above the mean goes down by gamma, below it up (exact
        // integer comparison of load*E with T*k)
        const int64_t Tk = int64_t(a.Tm) * a.k;
        for (int e = tid; e < E; e += NW * 64) {
            const int64_t lhs = int64_t(tot[e]) * E;
            const float bv = a.upd_bias[e];
            if (lhs > Tk) a.upd_bias[e] = bv - a.upd_gamma;
            else if (lhs < Tk) a.upd_bias[e] = bv + a.upd_gamma;
        }
    }
    if (stats_only) return;

    uint64_t* mym = gm + wave * E;
    const int* mypre = wpre + wave * E;
    int internal = 0;
    for (long w0 = row_begin; w0 < row_end; w0 += WR) {
        if (w0 != row_begin) load_window(w0);
        // this wave's masks (wave-private until the barrier)
        for (int e = lane; e < E; e += 64) mym[e] = 0;
        const uint64_t bit = 1ull << rl;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < KM; ++u) {
            const int e = ev[u];
            if (e >= 0 && e < E) atomicOr(reinterpret_cast<unsigned long long*>(&mym[e]), bit);
            else if (active && u < KC && g * KC + u < k) internal = 1;
        }
        __syncthreads();
        // window count of every expert, and per wave the count in the
        // earlier waves
        for (int e = tid; e < E; e += NW * 64) {
            int c[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w) c[w] = __popcll(gm[w * E + e]);
            int t = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                wpre[w * E + e] = t;
                t += c[w];
            }
            tot[e] = t;
        }
        __syncthreads();
        block_excl_scan(tot, E, lofs, wsum);  // ends with a barrier
        const int nvalid = lofs[E];

        // every slot: rank among the wave's assignments to its expert, places
        const uint64_t below = bit - 1;
        const long ibase = row * k;
#pragma unroll
        for (int u = 0; u < KM; ++u) {
            const int e = ev[u];
            if (e < 0 || e >= E) continue;
            const int j = g * KC + u;
            const int rank = __popcll(mym[e] & below) + mypre[e];
            const int lp = lofs[e] + rank;          // place in the window
            const long pos = long(base[e]) + rank;  // place in the segment
            const long i = ibase + j;
            const bool in_seg = pos >= 0 && pos < seglen;
            if (lp < 0 || lp >= nvalid || !in_seg) internal = 1;
            if (lp >= 0 && lp < nvalid) st[lp] = make_int2(int(i), in_seg ? int(pos) : -1);
            if (in_seg) {
                a.dropped[i] = (pos >= lim[e]) ? 1 : 0;
                if (a.inv_perm) a.inv_perm[i] = int32_t(segment + pos);
            }
        }
        __syncthreads();
        // the window in expert order: runs of consecutive places
        for (int p = tid; p < nvalid; p += blockDim.x) {
            const int2 v = st[p];
            if (v.y >= 0 && v.y < seglen) a.perm[segment + v.y] = v.x;
        }
        for (int e = tid; e < E; e += blockDim.x) base[e] += tot[e];
        __syncthreads();
    }
    if (internal && a.status) atomicOr(a.status, MOE_STATUS_INTERNAL);
}


int rows_cap_for_k(int k) {
    int lanes = 1;
    while (lanes * KM < k) lanes <<= 1;
    return 64 / lanes;
}

size_t lds_for(int E, int NW, int rpw, int k) {
    const size_t E4 = size_t((E + 1 + 3) & ~3);
    const size_t stage = size_t(NW) * rpw * k;
    return size_t(NW) * E * 12 + stage * 8 + 4 * E4 * 4;
}

}  // namespace

// Row-block groups for folding the block combine into the scatter: enough
// groups that a thread sums at most kFoldLoads row blocks, when that takes at
// most kFoldGroups groups, the groups of every expert fit the block's
// threads and their sums (16 bytes each) the LDS free before the first
// window; 0 otherwise (the combine kernel runs).  Measured per call: 16384
// tokens, E=8 top-2 (4 groups) 14.3 -> 11.9 us; 131072 tokens, E=8 top-1 (16
// groups) 15.6 -> 13.9 us; 32768 tokens, E=32 top-2 (6 groups) 21.1 ->
// 18.3 us.  With more (group, expert) pairs than threads (65536 tokens, E=64:
// 1024 pairs, two rounds of loads) it was 19.7 against 19.2 us, so such
// shapes keep the combine kernel.
int scatter_fold_groups(int E, int k, int bpm, int NW) {
    const long Q = (bpm + kFoldLoads - 1) / kFoldLoads;
    const size_t room = size_t(NW) * E * 12 + size_t(NW) * scatter_rows_per_wave(E, k, NW) * k * 8;
    if (Q < 1 || Q > kFoldGroups || Q * E > long(NW) * 64 || size_t(16) * Q * E > room) return 0;
    return int(Q);
}

// Rows per wave and window: 64 (one mask bit per row), halved until the
// block's LDS fits.
int scatter_rows_per_wave(int E, int k, int NW) {
    int rpw = rows_cap_for_k(k);
    // (2 KB of the 160 KB left for the static LDS arrays)
    while (rpw > 1 && lds_for(E, NW, rpw, k) > 158 * 1024) rpw >>= 1;
    return rpw;
}

size_t scatter_lds_bytes(int E, int k, int NW) {
    return lds_for(E, NW, scatter_rows_per_wave(E, k, NW), k);
}

// Waves per scatter block, following the row pass's blocks (the scatter's
// block b takes row block b's rows): eight when the row pass runs two blocks
// of eight per compute unit -- half the rows a block, and two scatter blocks
// share a compute unit and overlap their LDS-bound phases and barriers --,
// sixteen when it runs one block, so that one window covers a row block;
// eight above E = 512, where sixteen waves' row masks do not fit the LDS.
int scatter_waves(int E, int row_nw) { return (row_nw == 8 || E > 512) ? 8 : 16; }

template <int NW>
hipError_t launch_scatter_nw(const RowCfg& c, const ScatterArgs& a, size_t lds, hipStream_t st) {
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(route_scatter_kernel<NW>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(route_scatter_kernel<NW>, dim3(c.B + (a.stats_sep ? a.n_micro : 0)), dim3(NW * 64), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_route_scatter(const RowCfg& c, const ScatterArgs& a, hipStream_t st) {
    const int NW = a.nw;
    const size_t lds = lds_for(a.E, NW, a.rows_per_wave, a.k);
    if (a.k > MOE_ROUTE_MAX_K || a.E > MOE_ROUTE_MAX_E || a.rows_per_wave < 1 ||
        a.rows_per_wave > rows_cap_for_k(a.k))
        return hipErrorInvalidValue;
    if (NW == 16) return launch_scatter_nw<16>(c, a, lds, st);
    if (NW == 8) return launch_scatter_nw<8>(c, a, lds, st);
    return hipErrorInvalidValue;
}

}  // namespace moe
