// route_rows.hip -- the fused per-token pass of MoE routing on gfx950.
//
// For every token (row of logits [T,E]) one streaming read produces:
//   * the softmax statistics m = max_e l, s = sum_e exp(l - m)
//     (page mhpq.cn/news/998159 section 4.2: the router probabilities are a
//     softmax over the experts);
//   * the top-k experts in (logit desc, expert asc) order and their gate
//     weights (section 4.4 of that page: every token is dispatched to k
//     experts), optionally renormalised over the k picks;
//   * the block's expert histogram (LDS atomics on integers) and the block's
//     per-expert sums of softmax probabilities, used for f_i and P_i.
//
// Top-k without sorting.  Lane s of a segment owns G columns.  Let mu_s be
// the lane's maximum.  The k-th largest of the S lane maxima, tau, is a lower
// bound of the row's k-th largest logit (k lanes each hold a value >= tau).
// Only the few logits >= tau are candidates (about 7-10 of 256-384 for the
// routing workloads); they are compacted into LDS as 64-bit order keys and
// ranked by counting, which gives the exact top-k, ties to the lower expert.
// A row with more candidates than the list holds (massive ties) takes an
// exact k-round arg-max over all its logits instead.
//
// Determinism: the histogram is integer; every floating-point sum has a fixed
// order (butterflies within the wave, fixed wave order in LDS).
#include "route_common.hpp"

namespace moe {
namespace {

using namespace dev;

// 1 + the number of other lanes r of the segment with maximum >= lmax.
template <int S, int R>
__device__ __forceinline__ int count_ge(float lmax) {
    if constexpr (R >= S) {
        return 1;
    } else {
        return ((seg_other<S, R>(lmax) >= lmax) ? 1 : 0) + count_ge<S, R + 1>(lmax);
    }
}

template <int S, int G, int NW>
__global__ void __launch_bounds__(NW * 64)
route_rows_kernel(const RowsArgs a)
{
    constexpr int W = 64 / S;                 // rows per wave at a time
    constexpr int RS = row_stride(S, G);      // LDS row-copy stride (floats)
    constexpr int CAP = cand_cap(S, G);       // candidate list capacity
    constexpr int CS = CAP + 1;               // candidate row stride (keys)

    extern __shared__ __align__(16) unsigned char smem[];
    const int E = a.E, k = a.k;
    int* hist = reinterpret_cast<int*>(smem);
    float* rowbuf_all = reinterpret_cast<float*>(smem + ((E * 4 + 15) & ~15));
    uint64_t* cand_all = reinterpret_cast<uint64_t*>(
        reinterpret_cast<unsigned char*>(rowbuf_all) + ((NW * W * RS * 4 + 15) & ~15));
    uint64_t* sel_all = cand_all + NW * W * CS;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int seg = lane / S, s = lane % S;
    const int mb = blockIdx.x / a.bpm, bi = blockIdx.x % a.bpm;
    const long row_begin = long(mb) * a.Tm + long(bi) * a.R;
    long row_end = row_begin + a.R;
    if (row_end > long(mb + 1) * a.Tm) row_end = long(mb + 1) * a.Tm;

    for (int e = tid; e < E; e += NW * 64) hist[e] = 0;
    __syncthreads();

    float* rowbuf = rowbuf_all + (wave * W + seg) * RS;
    uint64_t* cand = cand_all + (wave * W + seg) * CS;
    uint64_t* sel = sel_all + (wave * W + seg) * k;

    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
    int bad = 0;

    const long per_iter = long(NW) * W;
    const int iters = int((row_end - row_begin + per_iter - 1) / per_iter);

    // rows of this wave: row_begin + (it*NW + wave)*W + seg
    auto load_row = [&](float (&x)[G], long row) {
        const bool ok = row < row_end;
        const float* src = a.logits + row * E;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int col = g * S + s;
            x[g] = (ok && col < E) ? __builtin_nontemporal_load(src + col) : -INFINITY;
        }
    };

    float xn[G];
    load_row(xn, row_begin + long(wave) * W + seg);

    for (int it = 0; it < iters; ++it) {
        const long row = row_begin + (long(it) * NW + wave) * W + seg;
        const bool valid = row < row_end;
        float x[G];
#pragma unroll
        for (int g = 0; g < G; ++g) x[g] = xn[g];
        if (it + 1 < iters) load_row(xn, row + per_iter);

        // ---- row maximum and the threshold tau
        float lmax = x[0];
#pragma unroll
        for (int g = 1; g < G; ++g) lmax = fmaxf(lmax, x[g]);
        const float m = seg_max<S>(lmax);
        float tau = m;
        if (k > 1) {
            if constexpr (S > 1) {
                // number of lanes of the segment whose maximum is >= mine
                const int ge = count_ge<S, 1>(lmax);
                // tau = the largest lane maximum that at least k lane maxima reach
                tau = seg_max<S>(ge >= k ? lmax : -INFINITY);
            }
        }

        // ---- candidates: logits >= tau (bit g of mask for column g*S+s)
        unsigned mask = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int col = g * S + s;
            mask |= ((x[g] >= tau) && (col < E)) ? (1u << g) : 0u;
        }
        if (!valid) mask = 0;
        const int n = __popc(mask);
        const int incl = seg_incl_scan<S>(n, s);
        const int C = seg_sumi<S>(n);

        // row copy for candidate extraction
#pragma unroll
        for (int g = 0; g < G; ++g) rowbuf[g * S + s] = x[g];

        // ---- softmax statistics and probability sums
        const float mL = m * kLog2e;
        float ex[G];
        float ssum = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            ex[g] = exp2f(fmaf(x[g], kLog2e, -mL));
            ssum += ex[g];
        }
        ssum = seg_sum<S>(ssum);
        const float inv = 1.0f / ssum;
        if (valid) {
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] = fmaf(ex[g], inv, acc[g]);
            if (!(ssum > 0.f && ssum <= 3.0e38f)) bad = 1;
        }

        // ---- exact top-k among the candidates
        const bool need_fb = valid && (C > CAP || C < k);
        if (__any(need_fb)) {
            // k rounds of arg-max over every logit of the row
            uint64_t prev = ~0ull;
            for (int j = 0; j < k; ++j) {
                uint64_t best = 0;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int col = g * S + s;
                    if (col < E) {
                        const uint64_t key = make_key(x[g], col);
                        if (key < prev && key > best) best = key;
                    }
                }
                best = seg_max_u64<S>(best);
                if (s == 0) sel[j] = best;
                prev = best;
            }
        } else {
            int o = incl - n;
            unsigned mm = mask;
            while (mm) {
                const int g = __ffs(mm) - 1;
                mm &= mm - 1;
                const int col = g * S + s;
                cand[o++] = make_key(rowbuf[col], col);
            }
            const int Cmax = wave_max_over_segments<S>(C);
            for (int p = C + s; p < Cmax; p += S) cand[p] = 0ull;
            for (int base = 0; base < Cmax; base += S) {
                const int c = base + s;
                const uint64_t my = (c < C) ? cand[c] : 0ull;
                int rank = 0;
                for (int c2 = 0; c2 < Cmax; ++c2) rank += (cand[c2] > my) ? 1 : 0;
                if (c < C && rank < k) sel[rank] = my;
            }
        }

        // ---- gate weights, outputs, histogram
        float e_pick = 0.f;
        int col_pick = 0;
        if (s < k) {
            const uint64_t key = sel[s];
            col_pick = key_col(key);
            e_pick = exp2f(fmaf(key_val(key), kLog2e, -mL));
        }
        const float denom = a.renorm ? seg_sum<S>(s < k ? e_pick : 0.f) : ssum;
        if (valid && s < k) {
            a.topk_idx[row * k + s] = col_pick;
            a.topk_w[row * k + s] = e_pick / denom;
            atomicAdd(&hist[col_pick], 1);
        }
        if (valid && s == 0 && a.save_stats) {
            a.row_stats[2 * row] = m;
            a.row_stats[2 * row + 1] = ssum;
        }
    }

    // ---- block partials: probability sums (fixed order) and histogram
    // lanes with the same s in different segments own the same columns
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
            const int col = g * S + s;
            if (col < E) pbuf[wave * E + col] = acc[g];
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

template <int S, int G>
hipError_t launch_sg(const RowCfg& c, const RowsArgs& a, hipStream_t st) {
    const size_t lds = rows_lds_bytes(c, a.E, a.k);
    auto kern = route_rows_kernel<S, G, 8>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(c.B), dim3(8 * 64), lds, st, a);
    return hipGetLastError();
}

template <int S>
hipError_t launch_s(const RowCfg& c, const RowsArgs& a, hipStream_t st) {
    switch (c.G) {
        case 1: return launch_sg<S, 1>(c, a, st);
        case 2: return launch_sg<S, 2>(c, a, st);
        case 4: return launch_sg<S, 4>(c, a, st);
        case 8: return launch_sg<S, 8>(c, a, st);
        case 12: return launch_sg<S, 12>(c, a, st);
        case 16: return launch_sg<S, 16>(c, a, st);
        case 24: return launch_sg<S, 24>(c, a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_route_rows(const RowCfg& c, const RowsArgs& a, hipStream_t st) {
    if (c.NW != 8) return hipErrorInvalidValue;
    switch (c.S) {
        case 1: return launch_s<1>(c, a, st);
        case 2: return launch_s<2>(c, a, st);
        case 4: return launch_s<4>(c, a, st);
        case 8: return launch_s<8>(c, a, st);
        case 16: return launch_s<16>(c, a, st);
        case 32: return launch_s<32>(c, a, st);
        case 64: return launch_s<64>(c, a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
