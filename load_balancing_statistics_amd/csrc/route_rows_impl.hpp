// route_rows_impl.hpp -- kernel templates of the two per-token streaming
// passes: the forward row pass and the aux-loss backward.  Instantiated per
// segment width S by route_s<S>.hip.
//
// Forward row pass.  For every token (row of logits [T,E]) one streaming read
// produces:
//   * the softmax statistics m = max_e l, s = sum_e exp(l - m)
//     (page mhpq.cn/news/998159 section 4.2: the router probabilities are a
//     softmax over the experts);
//   * the top-k experts in (logit desc, expert asc) order and their gate
//     weights (section 4.4 of that page: every token is dispatched to k
//     experts), optionally renormalised over the k picks;
//   * the block's expert histogram (LDS integer atomics) and the block's
//     per-expert sums of softmax probabilities, used for f_i and P_i.
// With a selection bias (BIAS; page mhpq.cn/news/998159 section 4.3) the
// experts are ranked by the fp32 sums l + b_e while the softmax, the weights
// and the probability sums use l: the block keeps a copy of the bias in LDS,
// from which each lane reads the bias of its columns for every row
// (threshold and candidate mask; registers it would otherwise hold for the
// whole pass) and the candidates theirs (keys); the LDS row copy stays
// unbiased, so a winner's weight is read from it exactly.
//
// Top-k without sorting.  Lane s of a segment owns G columns.  The k-th
// largest of the S lane maxima, tau, is a lower bound of the row's k-th
// largest logit (k lanes each hold a value >= tau), so the logits >= tau
// contain the top k.  For the routing workloads that is about 7-10 of 256-384
// logits; they are compacted into LDS as 64-bit order keys and ranked by
// counting, which yields the exact top-k with ties to the lower expert.  A
// row with more candidates than the list holds (massive ties) takes an exact
// k-round arg-max over its logits instead.
//
// Backward.  L_aux = alpha*E*sum_i f_i*P_i with f a constant observation
// (pages mhpq.cn/news/998159 section 4.2 and codechina.net article 413310
// section 2.2: the gradient reaches the router through P only):
//   dL/dl[t,j] = g_mb * alpha * E / Tm * p[t,j] * (f_j - sum_i f_i p[t,i]).
//
// Layout: lane s of a segment owns the columns VEC*(j*S + s) + v, j < G/VEC,
// v < VEC, so each vector load of a segment reads S*VEC consecutive floats.
// Determinism: integer histogram; every float sum has a fixed order.
#pragma once

#include "route_common.hpp"

namespace moe {
namespace rows_impl {

using namespace dev;

// 1 + the number of other lanes of the segment whose maximum is >= lmax.
template <int S, int R>
__device__ __forceinline__ int count_ge(float lmax) {
    if constexpr (R >= S) {
        return 1;
    } else {
        return ((seg_other<S, R>(lmax) >= lmax) ? 1 : 0) + count_ge<S, R + 1>(lmax);
    }
}

// Order-preserving integer key of a float (monotone for non-NaN values,
// -0.0 just below +0.0) and its inverse: integer max/min need no NaN
// canonicalisation and fuse with the DPP move of their operand.
__device__ __forceinline__ int order_key(float f) {
    const int b = __float_as_int(f);
    return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float from_order_key(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }

// One compare-exchange: lanes set in keep (a fixed pattern of the wave, held
// in a scalar mask) keep the larger of (v, partner), the others the smaller.
__device__ __forceinline__ int cx_keep(int v, int p, uint64_t keep) {
    const int mx = max(v, p), mn = min(v, p);
    return __builtin_amdgcn_inverse_ballot_w64(keep) ? mx : mn;
}

// Bitonic sort, descending, of one value per lane within each 16-lane row:
// merges of 2, 4, 8, 16 lanes, each opened by a mirror compare (the lower
// half keeps the larger) and closed by half-cleaners at distances 4, 2, 1.
__device__ __forceinline__ int sort16_desc(int v) {
    constexpr uint64_t kEven = 0x5555555555555555ull;  // (i & 1) == 0
    constexpr uint64_t kLow2 = 0x3333333333333333ull;  // (i & 2) == 0
    constexpr uint64_t kLow4 = 0x0F0F0F0F0F0F0F0Full;  // (i & 4) == 0
    constexpr uint64_t kLow8 = 0x00FF00FF00FF00FFull;  // (i & 8) == 0
    v = cx_keep(v, dppi<0xB1>(v), kEven);    // 2: lane i <-> i^1
    v = cx_keep(v, dppi<0x1B>(v), kLow2);    // 4: quad_perm [3,2,1,0], mirror
    v = cx_keep(v, dppi<0xB1>(v), kEven);
    v = cx_keep(v, dppi<0x141>(v), kLow4);   // 8: row_half_mirror
    v = cx_keep(v, dppi<0x4E>(v), kLow2);    //    i^2
    v = cx_keep(v, dppi<0xB1>(v), kEven);    //    i^1
    v = cx_keep(v, dppi<0x140>(v), kLow8);   // 16: row_mirror
    {
        // i^4: lane i reads i + 4 (row_ror:12) or i - 4 (row_ror:4)
        const int up = dppi<0x12C>(v), dn = dppi<0x124>(v);
        v = cx_keep(v, __builtin_amdgcn_inverse_ballot_w64(kLow4) ? up : dn, kLow4);
    }
    v = cx_keep(v, dppi<0x4E>(v), kLow2);    //    i^2
    v = cx_keep(v, dppi<0xB1>(v), kEven);    //    i^1
    return v;
}

// Minimum over each 16-lane row.
__device__ __forceinline__ int seg16_min(int v) {
    v = min(v, dppi<0xB1>(v));
    v = min(v, dppi<0x4E>(v));
    v = min(v, dppi<0x141>(v));
    v = min(v, dppi<0x140>(v));
    return v;
}

template <int S, int VEC>
__device__ __forceinline__ int col_of(int g, int s) {
    return VEC * ((g / VEC) * S + s) + (g % VEC);
}

// Load the G owned logits of a row.  The row index is clamped into the
// block's range and padding columns are clamped to the row, so every load is
// in bounds and unconditional; padding values become -inf.
template <int S, int G, int VEC, bool PAD>
__device__ __forceinline__ void load_row(float (&x)[G], const float* __restrict__ logits,
                                         long row, int E, int s) {
    const float* src = logits + row * E;
    if constexpr (VEC == 4) {
#pragma unroll
        for (int j = 0; j < G / 4; ++j) {
            int c0 = 4 * (j * S + s);
            const bool in = !PAD || c0 < E;
            if constexpr (PAD) c0 = in ? c0 : E - 4;
            const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + c0));
            x[4 * j + 0] = in ? v[0] : -INFINITY;
            x[4 * j + 1] = in ? v[1] : -INFINITY;
            x[4 * j + 2] = in ? v[2] : -INFINITY;
            x[4 * j + 3] = in ? v[3] : -INFINITY;
        }
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            int c = g * S + s;
            const bool in = !PAD || c < E;
            if constexpr (PAD) c = in ? c : E - 1;
            const float v = __builtin_nontemporal_load(src + c);
            x[g] = in ? v : -INFINITY;
        }
    }
}

// Masked P sums (page mhpq.cn/news/998159 section 4.4's top-k form: only a
// token's picks count) are accumulated like the all-token sums -- per-lane
// fp32 in row order, then fixed-order combines -- so they keep fp32's
// relative precision however small a pick's probability is.  A column is
// picked when its selection key is at least the row's k-th key: larger
// value, or equal value (-0.0 == +0.0) and a column no higher.
__device__ __forceinline__ bool picked_col(float y, int col, float kv, int kc) {
    return y > kv || (y == kv && col <= kc);
}

template <int S, int G, int VEC, bool PAD, int NW, bool BIAS, bool MASKED>
struct RowPass {
    static constexpr int W = 64 / S;               // rows per wave at a time
    static constexpr int RS = row_stride(S, G);    // LDS row-copy stride (floats)
    static constexpr int CAP = cand_cap(S, G);     // candidate list capacity
    static constexpr int CS = cand_stride(S, G);   // candidate row stride (keys)
    static constexpr int NP = (CAP + S - 1) / S;   // ranking passes at most

    // Exact top-k of a row from its LDS copy: k rounds of arg-max of the
    // order keys over the segment (rows whose candidate list overflows).
    __device__ __forceinline__ static uint64_t fallback_select(
        const float* rowbuf, const float* blds, uint64_t* sel, int E, int k, int s) {
        uint64_t prev = ~0ull;
        for (int j = 0; j < k; ++j) {
            uint64_t best = 0;
            for (int g = 0; g < G; ++g) {
                const int col = col_of<S, VEC>(g, s);
                if (!PAD || col < E) {
                    const float v = BIAS ? rowbuf[col] + blds[col] : rowbuf[col];
                    const uint64_t key = make_key(v, col);
                    if (key < prev && key > best) best = key;
                }
            }
            best = seg_max_u64<S>(best);
            if (s == 0) sel[j] = best;
            prev = best;
        }
        return prev;  // the k-th key (segment-uniform)
    }

    __device__ __forceinline__ static int col_from_bit(int g, int s) {
        return (VEC == 4) ? (4 * ((g >> 2) * S + s) + (g & 3)) : (g * S + s);
    }

    // One row (per segment): everything the forward needs from it.
    //
    // LDS traffic is arranged so that no step waits on a fresh round trip
    // more than necessary: the row copy is written and the lane's first
    // candidates are read back before the softmax arithmetic, which hides
    // the read latency; candidates then rank themselves against the whole
    // list (one batch of reads) and the winners write the outputs directly.
    __device__ __forceinline__ static void process(
        const RowsArgs& a, const float (&x)[G], long row, bool valid, int s,
        float* rowbuf, uint64_t* cand, int* hist, float (&acc)[G], int& bad,
        int* queue, int& qn, long row_begin, const float* blds,
        uint64_t* sel)
    {
        const int E = a.E, k = a.k;
        // the bias of the lane's columns, from the block's LDS copy (0 for
        // padding columns; unused without BIAS)
        float bz[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int col = col_of<S, VEC>(g, s);
            bz[g] = (BIAS && (!PAD || col < E)) ? blds[col] : 0.f;
        }
        // ---- row maximum (softmax) and the candidate threshold tau
        // (selection values: the logits, or the biased logits)
        float lmax = x[0];
#pragma unroll
        for (int g = 1; g < G; ++g) lmax = fmaxf(lmax, x[g]);
        float ymax = lmax;
        if constexpr (BIAS) {
            ymax = x[0] + bz[0];
#pragma unroll
            for (int g = 1; g < G; ++g) ymax = fmaxf(ymax, x[g] + bz[g]);
        }
        float m, tau;
        if constexpr (S == 16 && G <= 16) {
            // the segment's lane maxima sorted (descending) across its 16
            // lanes: tau is the k-th, and without a bias m is the first
            // (24-column lanes keep the rank count: the sort's temporaries
            // would push them past the 12-wave register budget)
            const int sk = sort16_desc(order_key(ymax));
            tau = from_order_key(seg16_min((s < k) ? sk : 0x7FFFFFFF));
            m = BIAS ? seg_max<S>(lmax) : from_order_key(dppi<0x150>(sk));  // row_newbcast:0
        } else {
            m = seg_max<S>(lmax);
            tau = BIAS ? seg_max<S>(ymax) : m;
            if constexpr (S > 1) {
                if (k > 1) {
                    const int ge = count_ge<S, 1>(ymax);
                    // the largest lane maximum reached by at least k lane maxima
                    tau = seg_max<S>(ge >= k ? ymax : -INFINITY);
                }
            }
        }

        // ---- candidates y >= tau (bit g of mask), real columns only
        unsigned mask = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const bool real = !PAD || col_of<S, VEC>(g, s) < E;
            const float y = BIAS ? x[g] + bz[g] : x[g];
            mask |= (y >= tau && real) ? (1u << g) : 0u;
        }
        if (!valid) mask = 0;
        const int n = __popc(mask);
        const int incl = seg_incl_scan<S>(n, s);
        const int C = seg_sumi<S>(n);

        // ---- row copy (LDS), then read back this lane's first candidates
        if constexpr (VEC == 4) {
#pragma unroll
            for (int j = 0; j < G / 4; ++j)
                *reinterpret_cast<f32x4*>(rowbuf + 4 * (j * S + s)) =
                    f32x4{x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]};
        } else {
#pragma unroll
            for (int g = 0; g < G; ++g) rowbuf[g * S + s] = x[g];
        }
        constexpr int XB = 4;  // candidates extracted per lane up front
        unsigned mm = mask;
        int ecol[XB];
        float ev[XB];
#pragma unroll
        for (int u = 0; u < XB; ++u) {
            const int g = mm ? __ffs(mm) - 1 : 0;
            mm &= mm - 1;
            ecol[u] = col_from_bit(g, s);
        }
#pragma unroll
        for (int u = 0; u < XB; ++u) ev[u] = BIAS ? rowbuf[ecol[u]] + blds[ecol[u]] : rowbuf[ecol[u]];

        // ---- softmax statistics and probability sums (hides the reads)
        const float mL = m * kLog2e;
        float ex[G];
        float ssum = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            ex[g] = __builtin_amdgcn_exp2f(fmaf(x[g], kLog2e, -mL));
            ssum += ex[g];
        }
        ssum = seg_sum<S>(ssum);
        const float inv = __builtin_amdgcn_rcpf(ssum);
        if (valid) {
            if constexpr (!MASKED) {
#pragma unroll
                for (int g = 0; g < G; ++g) acc[g] = fmaf(ex[g], inv, acc[g]);
            }
            if (!(ssum > 0.f && ssum <= 3.0e38f)) bad = 1;
        }

        // ---- exact top-k: winners as (rank, expert, exp) per ranking pass
        int wrank[NP], wcol[NP];
        float we[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) wrank[p] = -1;

        // Rows whose candidate list would overflow (massive ties) are queued
        // and resolved after the streaming loop; the rest rank here.
        const bool need_fb = valid && (C > CAP || C < k);
        const uint64_t fbmask = __ballot(need_fb && s == 0);
        if (__builtin_expect(fbmask != 0, 0)) {
            if (need_fb && s == 0) {
                const uint64_t lt = (__lane_id() == 0) ? 0ull : (~0ull >> (64 - __lane_id()));
                queue[qn + __popcll(fbmask & lt)] = int(row - row_begin);
            }
            qn += __popcll(fbmask);
        }
        if (!need_fb) {
            // compact the candidates' order keys into the row's list
            const int o = incl - n;
#pragma unroll
            for (int u = 0; u < XB; ++u)
                if (u < n) cand[o + u] = make_key(ev[u], ecol[u]);
            if (__builtin_expect(__any(n > XB), 0)) {
                int o2 = o + XB;
                while (mm) {
                    const int g = __ffs(mm) - 1;
                    mm &= mm - 1;
                    const int col = col_from_bit(g, s);
                    cand[o2++] = make_key(BIAS ? rowbuf[col] + blds[col] : rowbuf[col], col);
                }
            }
            // pad the list to a multiple of 4 keys
            const int C4 = (C + 3) & ~3;
            for (int p = C + s; p < C4; p += S) cand[p] = 0ull;
            // candidate c ranks itself against the whole list
            const ulonglong2* cand2 = reinterpret_cast<const ulonglong2*>(cand);
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int c = p * S + s;
                if (p * S < C) {
                    const uint64_t my = (c < C) ? cand[c] : 0ull;
                    int rank = 0;
                    for (int c2 = 0; c2 < C4; c2 += 4) {
                        const ulonglong2 k01 = cand2[c2 / 2];
                        const ulonglong2 k23 = cand2[c2 / 2 + 1];
                        rank += (k01.x > my) ? 1 : 0;
                        rank += (k01.y > my) ? 1 : 0;
                        rank += (k23.x > my) ? 1 : 0;
                        rank += (k23.y > my) ? 1 : 0;
                    }
                    if (c < C && rank < k) {
                        wrank[p] = rank;
                        wcol[p] = key_col(my);
                        const float lv = BIAS ? rowbuf[wcol[p]] : key_val(my);
                        we[p] = __builtin_amdgcn_exp2f(fmaf(lv, kLog2e, -mL));
                        if (MASKED && rank == k - 1) sel[0] = my;  // the k-th key, for masked P
                    }
                }
            }
        }

        // ---- gate weights, outputs, histogram
        float esum = 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p) esum += (wrank[p] >= 0) ? we[p] : 0.f;
        const float rden = a.renorm ? __builtin_amdgcn_rcpf(seg_sum<S>(esum)) : inv;
        if (valid) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                if (wrank[p] >= 0) {
                    a.topk_idx[row * k + wrank[p]] = wcol[p];
                    a.topk_w[row * k + wrank[p]] = we[p] * rden;
                    atomicAdd(&hist[wcol[p]], 1);
                }
            }
            if (s == 0 && a.save_stats) {
                a.row_stats[2 * row] = m;
                a.row_stats[2 * row + 1] = ssum;
            }
        }

        if constexpr (MASKED) {
          if (!need_fb) {
            // masked P: each owner adds the probabilities of its picked
            // columns, recomputed from the LDS row copy (x[] and ex[]
            // stay short-lived, so the all-token path keeps its
            // registers)
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const uint64_t kth = sel[0];
            const float kv = key_val(kth);
            const int kc = key_col(kth);
            if (valid) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int col = col_of<S, VEC>(g, s);
                    const float xv = rowbuf[(!PAD || col < E) ? col : 0];
                    const float y = BIAS ? xv + bz[g] : xv;
                    const float pv = __builtin_amdgcn_exp2f(fmaf(xv, kLog2e, -mL));
                    const bool pk = (!PAD || col < E) && picked_col(y, col, kv, kc);
                    acc[g] = pk ? fmaf(pv, inv, acc[g]) : acc[g];
                }
            }
          }
        }
    }

    // Queued rows (candidate-list overflow): reload, softmax statistics, exact
    // top-k by k rounds of arg-max, outputs.  The all-token probability sums
    // were already accumulated by the streaming pass; the masked ones, which
    // need the picks, are added here.
    __device__ __forceinline__ static void resolve_queue(
        const RowsArgs& a, const int* queue, int qn, long row_begin, int s, int seg,
        float* rowbuf, uint64_t* sel, int* hist, const float* blds, float (&acc)[G])
    {
        const int E = a.E, k = a.k;
        for (int q0 = 0; q0 < qn; q0 += W) {
            const bool has = q0 + seg < qn;
            const long row = row_begin + (has ? queue[q0 + seg] : queue[q0]);
            float x[G];
            load_row<S, G, VEC, PAD>(x, a.logits, row, E, s);
            float lmax = x[0];
#pragma unroll
            for (int g = 1; g < G; ++g) lmax = fmaxf(lmax, x[g]);
            const float m = seg_max<S>(lmax);
            const float mL = m * kLog2e;
            float ssum = 0.f;
#pragma unroll
            for (int g = 0; g < G; ++g) ssum += __builtin_amdgcn_exp2f(fmaf(x[g], kLog2e, -mL));
            ssum = seg_sum<S>(ssum);
#pragma unroll
            for (int g = 0; g < G; ++g) rowbuf[col_of<S, VEC>(g, s)] = x[g];
            const uint64_t kth = fallback_select(rowbuf, blds, sel, E, k, s);
            if (MASKED && has) {
                const float kv = key_val(kth), inv = __builtin_amdgcn_rcpf(ssum);
                const int kc = key_col(kth);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int col = col_of<S, VEC>(g, s);
                    const float y = BIAS ? x[g] + ((!PAD || col < E) ? blds[col] : 0.f) : x[g];
                    const float pv = __builtin_amdgcn_exp2f(fmaf(x[g], kLog2e, -mL));
                    const bool pk = (!PAD || col < E) && picked_col(y, col, kv, kc);
                    acc[g] = pk ? fmaf(pv, inv, acc[g]) : acc[g];
                }
            }
            float e = 0.f;
            int col = 0;
            if (s < k) {
                const uint64_t key = sel[s];
                col = key_col(key);
                const float lv = BIAS ? rowbuf[col] : key_val(key);
                e = __builtin_amdgcn_exp2f(fmaf(lv, kLog2e, -mL));
            }
            const float rden = a.renorm ? __builtin_amdgcn_rcpf(seg_sum<S>(s < k ? e : 0.f))
                                        : __builtin_amdgcn_rcpf(ssum);
            if (has && s < k) {
                a.topk_idx[row * k + s] = col;
                a.topk_w[row * k + s] = e * rden;
                atomicAdd(&hist[col], 1);
            }
        }
    }
};

// Waves per SIMD the row pass must fit: 4 for the eight-wave blocks that run
// two per compute unit (128 registers, as one block of 16 had), else 1.
template <int NW, int G>
constexpr int rows_min_waves_per_simd() { return rows_blocks_per_cu(NW, G) == 2 ? 4 : 1; }

// MASKED: P from each token's picks only (flag MOE_P_MASKED), a compile-time
// variant so that the all-token kernels keep their register budget.
template <int S, int G, int VEC, bool PAD, int NW, bool BIAS, bool MASKED>
__global__ void __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(rows_min_waves_per_simd<NW, G>())))
route_rows_kernel(const RowsArgs a)
{
    using RP = RowPass<S, G, VEC, PAD, NW, BIAS, MASKED>;
    constexpr int W = RP::W, RS = RP::RS, CS = RP::CS;

    extern __shared__ __align__(16) unsigned char smem[];
    const int E = a.E, k = a.k;
    int* hist = reinterpret_cast<int*>(smem);
    float* blds = reinterpret_cast<float*>(smem + ((E * 4 + 15) & ~15));  // [E] when BIAS
    float* rowbuf_all = reinterpret_cast<float*>(
        reinterpret_cast<unsigned char*>(blds) + (BIAS ? ((E * 4 + 15) & ~15) : 0));
    uint64_t* cand_all = reinterpret_cast<uint64_t*>(
        reinterpret_cast<unsigned char*>(rowbuf_all) + ((NW * W * RS * 4 + 15) & ~15));
    uint64_t* sel_all = cand_all + NW * W * CS;
    int* queue_all = reinterpret_cast<int*>(sel_all + NW * W * k);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int seg = lane / S, s = lane % S;
    long row_begin, row_end;
    block_rows(blockIdx.x, a.bpm, a.Tm, row_begin, row_end);

    for (int e = tid; e < E; e += NW * 64) hist[e] = 0;
    if (a.status && blockIdx.x == 0 && tid == 0) a.status[0] = 0;
    if constexpr (BIAS)
        for (int e = tid; e < E; e += NW * 64) blds[e] = a.bias[e];
    __syncthreads();

    float* rowbuf = rowbuf_all + (wave * W + seg) * RS;
    uint64_t* cand = cand_all + (wave * W + seg) * CS;
    uint64_t* sel = sel_all + (wave * W + seg) * k;
    int* queue = queue_all + wave * a.qcap;
    int qn = 0;

    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
    int bad = 0;
    const long per_iter = long(NW) * W;
    const int iters = int((row_end - row_begin + per_iter - 1) / per_iter);
    const long row0 = row_begin + long(wave) * W + seg;
    auto row_at = [&](int it) { return row0 + long(it) * per_iter; };
    auto clamp = [&](long r) { return r < row_end ? r : row_end - 1; };

    // Two register buffers: load the next row group while processing one.
    // Inside the loop every prefetch is unconditional (clamped rows), so the
    // wait before processing a buffer covers only that buffer's loads.
    float xa[G], xb[G];
    load_row<S, G, VEC, PAD>(xa, a.logits, clamp(row_at(0)), E, s);
    int it = 0;
    // Two blocks per compute unit: workgroups are dealt out in order, so the
    // second half of the grid holds each compute unit's second block, whose
    // waves the arbiter (oldest first) issues less often; left alone it ends
    // about a fifth of the kernel later and streams its last rows at half the
    // memory parallelism.  Its waves take the higher priority for the first
    // half of their iterations, which brings the two ends together (measured
    // at v3_shape: 31.3 us against 33.3 us).
    const bool second = gridDim.x == 2 * kAssumedCUs && blockIdx.x >= kAssumedCUs;
    const int cut = iters / 2;
    if (second && cut > 0) __builtin_amdgcn_s_setprio(1);
    for (; it + 2 < iters; it += 2) {
        if (second && it >= cut && it < cut + 2) __builtin_amdgcn_s_setprio(0);
        load_row<S, G, VEC, PAD>(xb, a.logits, clamp(row_at(it + 1)), E, s);
        RP::process(a, xa, row_at(it), row_at(it) < row_end, s, rowbuf, cand, hist, acc, bad, queue, qn, row_begin, blds, sel);
        load_row<S, G, VEC, PAD>(xa, a.logits, clamp(row_at(it + 2)), E, s);
        RP::process(a, xb, row_at(it + 1), row_at(it + 1) < row_end, s, rowbuf, cand, hist,
                    acc, bad, queue, qn, row_begin, blds, sel);
    }
    if (it + 1 < iters) {
        load_row<S, G, VEC, PAD>(xb, a.logits, clamp(row_at(it + 1)), E, s);
        RP::process(a, xa, row_at(it), row_at(it) < row_end, s, rowbuf, cand, hist, acc, bad, queue, qn, row_begin, blds, sel);
        RP::process(a, xb, row_at(it + 1), row_at(it + 1) < row_end, s, rowbuf, cand, hist,
                    acc, bad, queue, qn, row_begin, blds, sel);
    } else if (it < iters) {
        RP::process(a, xa, row_at(it), row_at(it) < row_end, s, rowbuf, cand, hist, acc, bad, queue, qn, row_begin, blds, sel);
    }

    if (__builtin_expect(qn > 0, 0))
        RP::resolve_queue(a, queue, qn, row_begin, s, seg, rowbuf, sel, hist, blds, acc);

    // ---- block partials: probability sums (fixed order) and histogram.
    // Lanes with the same s in different segments own the same columns.
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if constexpr (S <= 1) acc[g] += xor_lane<1>(acc[g]);
        if constexpr (S <= 2) acc[g] += xor_lane<2>(acc[g]);
        if constexpr (S <= 4) acc[g] += xor_lane<4>(acc[g]);
        if constexpr (S <= 8) acc[g] += xor_lane<8>(acc[g]);
        if constexpr (S <= 16) acc[g] += xor_lane<16>(acc[g]);
        if constexpr (S <= 32) acc[g] += xor_lane<32>(acc[g]);
    }
    const int any_bad = __syncthreads_or(bad);
    float* pbuf = rowbuf_all;  // reused: [NW][E]
    if (seg == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int col = col_of<S, VEC>(g, s);
            if (!PAD || col < E) pbuf[wave * E + col] = acc[g];
        }
    }
    __syncthreads();
    const long bo = long(blockIdx.x) * E;
    for (int e = tid; e < E; e += NW * 64) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) t += pbuf[w * E + e];
        a.P_part[bo + e] = t;
        a.cnt_part[bo + e] = hist[e];
    }
    if (tid == 0) a.flag_part[blockIdx.x] = any_bad ? MOE_STATUS_NONFINITE : 0;
}

// Backward.  Dense part (every column):  p_i * (alpha_i - beta_t);
// sparse part (the k picked columns):     gamma_i.
//   all-token aux:  alpha_i = c f_i,  beta_t += c sum_e f_e p_e,  c = g alpha E / Tm
//   masked aux:     gamma_i += c' f_i p_i,  beta_t += c' sum_picked f_e p_e,
//                   c' = g alpha E / (Tm k)
//   weights:        gamma_i += p_i dW_j,  beta_t += sum_j dW_j p_{idx_j}
//   renormalised:   gamma_i += w_j (dW_j - D_t),  D_t = sum_j dW_j w_j
// (j = the slot that picked column i; the forms follow from the softmax
// Jacobian p_i (delta_ij - p_j) and, for the renormalised weights
// w_j = p_{idx_j} / sum_picked p, the quotient rule).  SP enables the sparse
// part: the segment's probabilities go to an LDS row buffer, the slot lanes
// (s < k) form the picked columns' terms and write them into a second
// per-segment buffer, which the column owners read and clear again.
template <int S, int G, int VEC, bool PAD, int NW, bool SP>
__global__ void __launch_bounds__(NW * 64)
route_backward_kernel(const BackArgs a)
{
    constexpr int W = 64 / S;
    extern __shared__ __align__(16) unsigned char bsmem[];
    const int E = a.E, k = a.k;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int seg = lane / S, s = lane % S;
    const int mb = blockIdx.x / a.bpm;
    long row_begin, row_end;
    block_rows(blockIdx.x, a.bpm, a.Tm, row_begin, row_end);

    const float inv_total = 1.0f / (float(a.Tm) * float(a.k));
    float fcol[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int col = col_of<S, VEC>(g, s);
        fcol[g] = (!PAD || col < E) ? float(a.counts[long(mb) * E + col]) * inv_total : 0.f;
    }
    const float gup = a.d_aux ? a.d_aux[mb] : 1.0f;
    const float c = gup * a.alpha * float(E) / float(a.Tm);
    const float cm = c / float(k);
    const bool dense_aux = !(SP && a.p_masked);

    // SP buffers: f of every expert, then per segment [E4] probabilities and
    // [E4] sparse terms (kept zero between rows)
    const int E4 = (E + 3) & ~3;
    float* fl = reinterpret_cast<float*>(bsmem);
    float* pb = fl + E4 + (wave * W + seg) * 2 * E4;
    float* gb = pb + E4;
    if constexpr (SP) {
        for (int e = tid; e < E; e += NW * 64) fl[e] = float(a.counts[long(mb) * E + e]) * inv_total;
        for (int e = s; e < E; e += S) gb[e] = 0.f;
        __syncthreads();
    }

    // The block's rows from the last: the forward's row pass walked the same
    // rows upwards, so the ones it read last -- the likeliest still to be in
    // the Infinity Cache -- come first (v4 shape: 165.7 -> 164.9 us).  Every
    // row's gradient stands alone, so the order changes no result.
    const long per_iter = long(NW) * W;
    const long n_it = (row_end - row_begin + per_iter - 1) / per_iter;
    for (long it = n_it - 1; it >= 0; --it) {
        const long base = row_begin + it * per_iter + long(wave) * W;  // wave-uniform
        if (base >= row_end) continue;
        const long row = base + seg;
        const bool valid = row < row_end;
        const long lr = valid ? row : row_end - 1;
        float x[G];
        load_row<S, G, VEC, PAD>(x, a.logits, lr, E, s);
        float m, ssum;
        float ex[G];
        if (a.row_stats) {
            m = a.row_stats[2 * lr];
            ssum = a.row_stats[2 * lr + 1];
            const float mL = m * kLog2e;
#pragma unroll
            for (int g = 0; g < G; ++g) ex[g] = __builtin_amdgcn_exp2f(fmaf(x[g], kLog2e, -mL));
        } else {
            float lmax = x[0];
#pragma unroll
            for (int g = 1; g < G; ++g) lmax = fmaxf(lmax, x[g]);
            m = seg_max<S>(lmax);
            const float mL = m * kLog2e;
            ssum = 0.f;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                ex[g] = __builtin_amdgcn_exp2f(fmaf(x[g], kLog2e, -mL));
                ssum += ex[g];
            }
            ssum = seg_sum<S>(ssum);
        }
        const float inv = __builtin_amdgcn_rcpf(ssum);
        float dot = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            ex[g] *= inv;  // p
            dot = fmaf(fcol[g], ex[g], dot);
        }
        float beta = 0.f;
        if (dense_aux) beta = c * seg_sum<S>(dot);
        float gam[G];
#pragma unroll
        for (int g = 0; g < G; ++g) gam[g] = 0.f;
        if constexpr (SP) {
            // owners publish the row's probabilities
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int col = col_of<S, VEC>(g, s);
                if (!PAD || col < E) pb[col] = ex[g];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // slot lanes: the picked columns
            int cs = -1;
            float ps = 0.f, fs = 0.f, dws = 0.f;
            if (valid && s < k) {
                const int e = a.topk_idx[row * k + s];
                if (e >= 0 && e < E) {
                    cs = e;
                    ps = pb[e];
                    fs = fl[e];
                    dws = a.d_topk_w ? a.d_topk_w[row * k + s] : 0.f;
                }
            }
            const float Z = seg_sum<S>(ps);
            const float Sm = seg_sum<S>(fs * ps);
            const float Dn = seg_sum<S>(dws * ps);
            if (a.p_masked) beta += cm * Sm;
            if (a.d_topk_w && !a.renorm) beta += Dn;
            if (cs >= 0) {
                float gv = 0.f;
                if (a.p_masked) gv += cm * fs * ps;
                if (a.d_topk_w) {
                    if (a.renorm) {
                        const float rz = 1.0f / Z;
                        gv += ps * rz * (dws - Dn * rz);
                    } else {
                        gv += ps * dws;
                    }
                }
                gb[cs] = gv;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // owners take their columns' terms and clear them for the next row
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int col = col_of<S, VEC>(g, s);
                if (!PAD || col < E) {
                    gam[g] = gb[col];
                    gb[col] = 0.f;
                }
            }
        }
        if (valid) {
            float* dst = a.dlogits + row * E;
            if constexpr (VEC == 4) {
#pragma unroll
                for (int j = 0; j < G / 4; ++j) {
                    const int c0 = 4 * (j * S + s);
                    if (!PAD || c0 < E) {
                        f32x4 v;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int g = 4 * j + q;
                            const float al = dense_aux ? c * fcol[g] : 0.f;
                            v[q] = ex[g] * (al - beta) + gam[g];
                        }
                        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst + c0));
                    }
                }
            } else {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int col = g * S + s;
                    const float al = dense_aux ? c * fcol[g] : 0.f;
                    if (!PAD || col < E) __builtin_nontemporal_store(ex[g] * (al - beta) + gam[g], dst + col);
                }
            }
        }
    }
}

template <int S, int G, int VEC, bool PAD, bool BIAS, bool MASKED>
hipError_t launch_rows_v(const RowCfg& c, const RowsArgs& a, hipStream_t st, const LaunchEvents* ev) {
    constexpr int NW = rows_waves(S, G, BIAS, MASKED, VEC, PAD);
    if (c.NW != NW) return hipErrorInvalidValue;
    const size_t lds = rows_lds_bytes(c, a.E, a.k, BIAS);
    auto kern = route_rows_kernel<S, G, VEC, PAD, NW, BIAS, MASKED>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
    }
    if (ev && (ev->start || ev->stop))
        hipExtLaunchKernelGGL(kern, dim3(c.B), dim3(NW * 64), lds, st, ev->start, ev->stop, 0u, a);
    else
        hipLaunchKernelGGL(kern, dim3(c.B), dim3(NW * 64), lds, st, a);
    return hipGetLastError();
}

template <int S, int G, int VEC, bool PAD>
hipError_t launch_rows(const RowCfg& c, const RowsArgs& a, hipStream_t st, const LaunchEvents* ev) {
    if (a.bias)
        return a.p_masked ? launch_rows_v<S, G, VEC, PAD, true, true>(c, a, st, ev)
                          : launch_rows_v<S, G, VEC, PAD, true, false>(c, a, st, ev);
    return a.p_masked ? launch_rows_v<S, G, VEC, PAD, false, true>(c, a, st, ev)
                      : launch_rows_v<S, G, VEC, PAD, false, false>(c, a, st, ev);
}

template <int S, int G, int VEC, bool PAD, int NW, bool SP>
hipError_t launch_backward_nw(const RowCfg& c, const BackArgs& a, hipStream_t st) {
    auto kern = route_backward_kernel<S, G, VEC, PAD, NW, SP>;
    const size_t lds = SP ? backward_lds_bytes(c, a.E) : 0;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(c.B), dim3(NW * 64), lds, st, a);
    return hipGetLastError();
}

template <int S, int G, int VEC, bool PAD>
hipError_t launch_backward(const RowCfg& c, const BackArgs& a, hipStream_t st, const LaunchEvents*) {
    // the backward's blocks are the forward's row blocks (no selection bias)
    constexpr int NW = rows_waves(S, G, false, false, VEC);
    if (c.NW != NW) return hipErrorInvalidValue;
    const bool sp = a.p_masked || a.d_topk_w;
    return sp ? launch_backward_nw<S, G, VEC, PAD, NW, true>(c, a, st)
              : launch_backward_nw<S, G, VEC, PAD, NW, false>(c, a, st);
}

// Dispatch over (G, VEC, PAD) for one S.
template <int S, typename ArgsT, template <int, int, bool> class Launch>
hipError_t dispatch(const RowCfg& c, const ArgsT& a, hipStream_t st, const LaunchEvents* ev) {
#define MOE_CASE(GG, VV, PP) \
    if (c.G == GG && c.VEC == VV && c.PAD == PP) return Launch<GG, VV, PP>::run(c, a, st, ev);
    MOE_CASE(4, 4, 0) MOE_CASE(8, 4, 0) MOE_CASE(16, 4, 0) MOE_CASE(24, 4, 0)
    MOE_CASE(4, 4, 1) MOE_CASE(8, 4, 1) MOE_CASE(16, 4, 1) MOE_CASE(24, 4, 1)
    MOE_CASE(1, 1, 1) MOE_CASE(2, 1, 1) MOE_CASE(4, 1, 1) MOE_CASE(8, 1, 1)
    MOE_CASE(16, 1, 1) MOE_CASE(24, 1, 1)
#undef MOE_CASE
    return hipErrorInvalidValue;
}

}  // namespace rows_impl

#define MOE_INSTANTIATE_SEGMENT(SV)                                                        \
    namespace {                                                                            \
    template <int G, int V, bool P>                                                        \
    struct RowsL {                                                                         \
        static hipError_t run(const RowCfg& c, const RowsArgs& a, hipStream_t st,          \
                              const LaunchEvents* ev) {                                    \
            return rows_impl::launch_rows<SV, G, V, P>(c, a, st, ev);                      \
        }                                                                                  \
    };                                                                                     \
    template <int G, int V, bool P>                                                        \
    struct BackL {                                                                         \
        static hipError_t run(const RowCfg& c, const BackArgs& a, hipStream_t st,          \
                              const LaunchEvents* ev) {                                    \
            return rows_impl::launch_backward<SV, G, V, P>(c, a, st, ev);                  \
        }                                                                                  \
    };                                                                                     \
    }                                                                                      \
    template <>                                                                            \
    hipError_t launch_rows_s<SV>(const RowCfg& c, const RowsArgs& a, hipStream_t st,       \
                                 const LaunchEvents* ev) {                                 \
        return rows_impl::dispatch<SV, RowsArgs, RowsL>(c, a, st, ev);                     \
    }                                                                                      \
    template <>                                                                            \
    hipError_t launch_backward_s<SV>(const RowCfg& c, const BackArgs& a, hipStream_t st) { \
        return rows_impl::dispatch<SV, BackArgs, BackL>(c, a, st, nullptr);                \
    }

}  // namespace moe
