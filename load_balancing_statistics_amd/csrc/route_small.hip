// route_small.hip -- the whole forward of a small microbatch in one launch.
//
// A microbatch of at most kSmallMaxLogits logits over a power-of-two number
// of experts up to 8, with k*E at most 16 (Switch top-1 over 4096 tokens and
// 8 experts is one), costs the multi-kernel path its launches and their
// first memory round trips, not its bytes -- the launch-count lesson of the
// LoongForge TAOT blog, section 3.
// Here no workgroup waits for another: every workgroup of a microbatch reads
// all of it (at most 128 KB, from L2 after the first) and selects every
// token's experts itself, which gives it the counts before its own rows and
// the whole histogram, hence its bases and the offsets:
//   - row block b (kSmallRows tokens, one per thread) writes the top-k, the
//     gate weights, the row statistics, the permutation, inv_perm and the
//     drop mask of its own tokens (page mhpq.cn/news/998159 sections 4.2,
//     4.4, 4.5);
//   - one more workgroup per microbatch also forms the softmax probability
//     sums and writes the counts, offsets, f, P, the balance statistics and
//     the status word, with the same code as the multi-kernel path.
// Each workgroup's selection costs about k*E steps per row of the whole
// microbatch, so the path stops where the multi-kernel path is faster
// (measured: 16 experts top-2 over 2048 tokens, 16.4 against 12.5 us).
// The order is the library's: larger logit (plus the selection bias when
// given) first, ties to the lower expert, -0.0 equal to +0.0.  A thread
// keeps each of its rows in registers; the k picks are k rounds of arg-max
// over the row's order keys.  Inside an expert the permutation keeps token
// order (a token picks an expert at most once): a token's rank is the
// count in the earlier rows of the microbatch, in the earlier waves of the
// block (ballot counts) and in the earlier lanes of its wave (popcount of
// the ballot below it).
#include "route_common.hpp"

namespace moe {
namespace {

using namespace dev;

constexpr int kSmallWaves = 16;
constexpr int kSmallRows = kSmallWaves * 64;  // rows of a row block, one per thread

// Row `row` of the logits: NE floats.  Unconditional loads from clamped
// addresses, so a thread's loads are all in flight at once.
template <int NE, bool VEC>
MOE_DEV void load_row(const float* L, long row, bool ok, float (&x)[NE]) {
    if constexpr (VEC) {
        const f32x4* p = reinterpret_cast<const f32x4*>(L);
#pragma unroll
        for (int q = 0; q < NE / 4; ++q) {
            const f32x4 v = p[ok ? row * (NE / 4) + q : 0];
            x[4 * q] = v.x;
            x[4 * q + 1] = v.y;
            x[4 * q + 2] = v.z;
            x[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < NE; ++e) x[e] = L[ok ? row * NE + e : 0];
    }
}

// Order key of a logit: an order-preserving unsigned integer of the value,
// -0.0 canonicalised to +0.0, and at least 1 (only one NaN pattern maps to
// 0), so that 0 can mark a column already picked.
MOE_DEV uint32_t order_key(float v) {
    const uint32_t u = __float_as_uint(v + 0.0f);
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return o > 1u ? o : 1u;
}

// The k picks of a row, best first: for k = 1 and 2 one scan over the
// values, else k rounds of arg-max over the order keys; every scan goes
// through the experts in ascending order with strict comparisons, so ties go
// to the lower expert, and a picked column's key becomes 0.  pm gets bit e
// for every picked expert and jp the pick index j of expert e in bits
// [4e, 4e+4); pick(j, col) is called in order.
template <int NE, bool BIAS, class Pick>
MOE_DEV void select_row(const float (&x)[NE], const float* bl, int k, uint32_t& pm, uint64_t& jp, Pick pick) {
    if (k == 1) {
        // one pick: the arg-max of the values themselves (a float
        // comparison already takes -0.0 equal to +0.0), lower expert on ties
        float best = BIAS ? x[0] + bl[0] : x[0];
        int col = 0;
#pragma unroll
        for (int e = 1; e < NE; ++e) {
            const float v = BIAS ? x[e] + bl[e] : x[e];
            const bool gt = v > best;
            best = gt ? v : best;
            col = gt ? e : col;
        }
        pm = 1u << col;
        jp = 0;
        pick(0, col);
        return;
    }
    if (NE >= 2 && k == 2) {
        // two picks in one scan: the best two values, the lower expert first
        // among equals; the first two columns seed them, so both picks are
        // always distinct experts (also for NaN values)
        const float v0 = BIAS ? x[0] + bl[0] : x[0];
        const float v1 = BIAS ? x[NE > 1 ? 1 : 0] + bl[NE > 1 ? 1 : 0] : x[NE > 1 ? 1 : 0];
        const bool sw = v1 > v0;
        float b1 = sw ? v1 : v0, b2 = sw ? v0 : v1;
        int c1 = sw ? 1 : 0, c2 = sw ? 0 : 1;
#pragma unroll
        for (int e = 2; e < NE; ++e) {
            const float v = BIAS ? x[e] + bl[e] : x[e];
            const bool g1 = v > b1;
            const bool g2 = !g1 && v > b2;
            b2 = g1 ? b1 : (g2 ? v : b2);
            c2 = g1 ? c1 : (g2 ? e : c2);
            b1 = g1 ? v : b1;
            c1 = g1 ? e : c1;
        }
        pm = (1u << c1) | (1u << c2);
        jp = uint64_t(1) << (4 * c2);
        pick(0, c1);
        pick(1, c2);
        return;
    }
    uint32_t key[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) key[e] = order_key(BIAS ? x[e] + bl[e] : x[e]);
    pm = 0;
    jp = 0;
#pragma unroll
    for (int j = 0; j < NE; ++j) {
        if (j >= k) break;
        uint32_t best = key[0];
        int col = 0;
#pragma unroll
        for (int e = 1; e < NE; ++e) {
            const bool gt = key[e] > best;
            best = gt ? key[e] : best;
            col = gt ? e : col;
        }
        pm |= 1u << col;
        jp |= uint64_t(j) << (4 * col);
#pragma unroll
        for (int e = 0; e < NE; ++e) key[e] = (e == col) ? 0u : key[e];
        pick(j, col);
    }
}

// Softmax statistics of a row: max m and s = sum_e exp(l_e - m) (exp2 of
// the logit scaled by log2 e), with the terms ex.
template <int NE>
MOE_DEV void row_softmax(const float (&x)[NE], float& m, float& ssum, float (&ex)[NE]) {
    m = x[0];
#pragma unroll
    for (int e = 1; e < NE; ++e) m = fmaxf(m, x[e]);
    const float mL = m * kLog2e;
    ssum = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        ex[e] = __builtin_amdgcn_exp2f(fmaf(x[e], kLog2e, -mL));
        ssum += ex[e];
    }
}

template <int NE, bool VEC, bool BIAS>
__global__ void __launch_bounds__(kSmallRows)
route_small_kernel(const SmallArgs a)
{
    const ScatterArgs& o = a.out;
    const int k = o.k, Tm = o.Tm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int mb = blockIdx.y, b = blockIdx.x;
    const bool stats = b == a.nb;  // the microbatch's statistics workgroup
    const long first = long(mb) * Tm;
    const int NI = (Tm + kSmallRows - 1) / kSmallRows;  // row rounds of the microbatch
    constexpr int CH = 16 / NE;                          // rows a thread has in flight per round
    constexpr int NP = (NE + 3) / 4;                     // words of packed counts a thread

    __shared__ float bl[NE];
    __shared__ uint32_t cw[2][NP][kSmallRows];  // packed counts by thread: all rows, rows before the block's
    __shared__ float pa[NE][kSmallRows];        // statistics workgroup: probability sums by thread
    __shared__ int wc[kSmallWaves][NE];
    __shared__ double psum[NE];
    __shared__ int tot[NE + 1], lofs[NE + 1], bef[NE];
    __shared__ double q[4 * NE];
    if (BIAS && tid < NE) bl[tid] = a.bias[tid];
    if (BIAS) __syncthreads();

    // ---- every row of the microbatch: picks (all workgroups) and, in the
    // statistics workgroup, softmax probability sums and the non-finite flag
    // per-thread counts, 8 bits an expert, four experts a word (a thread
    // holds at most kSmallMaxLogits / kSmallRows = 32 rows)
    uint32_t cnt[NP];
    float acc[NE];
#pragma unroll
    for (int u = 0; u < NP; ++u) cnt[u] = 0;
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = 0.f;
    float xo[NE];  // the block's own row, kept from the pass below
    int bad = 0;
    float xr[CH][NE];
    auto load_round = [&](int i0) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const long r = long(i0 + c) * kSmallRows + tid;
            load_row<NE, VEC>(a.logits, first + r, i0 + c < NI && r < Tm, xr[c]);
        }
    };
    load_round(0);
    for (int i0 = 0; i0 < NI; i0 += CH) {
        float x[CH][NE];
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int e = 0; e < NE; ++e) x[c][e] = xr[c][e];
        if (i0 + CH < NI) load_round(i0 + CH);  // next round in flight meanwhile
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int i = i0 + c;  // uniform over the block
            if (i >= NI) break;
            const bool valid = long(i) * kSmallRows + tid < Tm;
            uint32_t pm;
            uint64_t jp;
            select_row<NE, BIAS>(x[c], bl, k, pm, jp, [](int, int) {});
            if (!valid) pm = 0;
            if (i == b) {
#pragma unroll
                for (int u = 0; u < NP; ++u) cw[1][u][tid] = cnt[u];  // the rows before the block's own
#pragma unroll
                for (int e = 0; e < NE; ++e) xo[e] = x[c][e];
            }
            // bits 4u..4u+3 of pm spread to the bytes of word u (the four
            // shifted copies the product adds never overlap)
#pragma unroll
            for (int u = 0; u < NP; ++u) cnt[u] += (((pm >> (4 * u)) & 0xFu) * 0x00204081u) & 0x01010101u;
            if (stats && valid) {
                float m, ssum, ex[NE];
                row_softmax<NE>(x[c], m, ssum, ex);
                const float inv = __builtin_amdgcn_rcpf(ssum);
#pragma unroll
                for (int e = 0; e < NE; ++e)
                    acc[e] = (!o.p_masked || ((pm >> e) & 1u)) ? fmaf(ex[e], inv, acc[e]) : acc[e];
                if (!(ssum > 0.f && ssum <= 3.0e38f)) bad = 1;
            }
        }
    }
    // ---- block sums through LDS, thread t's values in column t: wave e
    // (e < NE) adds byte e of the packed counts, 16 columns a lane, and in the
    // statistics workgroup wave NE + e expert e's probability sums (fp64,
    // columns in order, then the lanes) -- one reduction per expert, not one
    // per expert and wave
#pragma unroll
    for (int u = 0; u < NP; ++u) cw[0][u][tid] = cnt[u];
    if (stats) {
#pragma unroll
        for (int e = 0; e < NE; ++e) pa[e][tid] = acc[e];
    }
    const int any_bad = __syncthreads_or(bad);
    if (wave < NE) {
        const int e = wave, sh = 8 * (e % 4);
        int sa = 0, sb = 0;
#pragma unroll
        for (int j = 0; j < kSmallWaves; ++j) {
            sa += int((cw[0][e / 4][lane + 64 * j] >> sh) & 0xFFu);
            sb += int((cw[1][e / 4][lane + 64 * j] >> sh) & 0xFFu);
        }
        sa = seg_sumi<64>(sa);
        sb = seg_sumi<64>(sb);
        if (lane == 0) {
            tot[e] = sa;
            bef[e] = stats ? 0 : sb;  // (the statistics workgroup has no rows of its own)
        }
    } else if (stats && wave < 2 * NE) {
        const int e = wave - NE;
        double sv = 0.0;
#pragma unroll
        for (int j = 0; j < kSmallWaves; ++j) sv += double(pa[e][lane + 64 * j]);
        sv = wave_sum_f64(sv);
        if (lane == 0) psum[e] = sv;
    }
    __syncthreads();
    // the offsets: exclusive prefix of the counts over the experts
    if (tid == 0) {
        int run = 0;
        for (int e = 0; e < NE; ++e) {
            lofs[e] = run;
            run += tot[e];
        }
        lofs[NE] = run;
    }

    if (stats) {
        double ps[1] = {tid < NE ? psum[tid] : 0.0};
        if (o.status && tid == 0) o.status[0] = any_bad ? MOE_STATUS_NONFINITE : 0;
        __syncthreads();
        microbatch_statistics<kSmallWaves, 1>(o, mb, tot, lofs, ps, q);
        return;
    }

    // ---- this block's own row: its picks in order, gate weights, places
    const long t = long(b) * kSmallRows + tid;  // row inside the microbatch
    const bool own = t < Tm;
    const long row = first + t;
    float m, ssum, ex[NE];
    row_softmax<NE>(xo, m, ssum, ex);
    int pc[NE];
    float pw[NE];
#pragma unroll
    for (int j = 0; j < NE; ++j) {
        pc[j] = 0;
        pw[j] = 0.f;
    }
    uint32_t pm;
    uint64_t jp;
    select_row<NE, BIAS>(xo, bl, k, pm, jp, [&](int j, int col) {
        pc[j] = col;
        float w = 0.f;
#pragma unroll
        for (int e = 0; e < NE; ++e) w = (e == col) ? ex[e] : w;
        pw[j] = w;
    });
    if (!own) pm = 0;
    float esum = 0.f;
#pragma unroll
    for (int j = 0; j < NE; ++j) esum += pw[j];  // (slots past k hold 0)
    const float rden = a.renorm ? __builtin_amdgcn_rcpf(esum) : __builtin_amdgcn_rcpf(ssum);
    if (own) {
#pragma unroll
        for (int j = 0; j < NE; ++j) {
            if (j >= k) break;
            a.topk_idx[row * k + j] = pc[j];
            a.topk_w[row * k + j] = pw[j] * rden;
        }
        if (a.save_stats) {
            a.row_stats[2 * row] = m;
            a.row_stats[2 * row + 1] = ssum;
        }
    }

    // ranks: per expert a ballot over the wave -- the lane's rank is its
    // popcount below the lane, the wave's count its popcount -- then the
    // counts of the earlier waves
    const uint64_t below = (1ull << lane) - 1ull;
    int rk[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const uint64_t bal = __ballot(((pm >> e) & 1u) != 0);
        rk[e] = __popcll(bal & below);
        if (lane == 0) wc[wave][e] = __popcll(bal);
    }
    __syncthreads();
    if (tid < NE) {
        int run = 0;
        for (int w = 0; w < kSmallWaves; ++w) {
            const int c = wc[w][tid];
            wc[w][tid] = run;
            run += c;
        }
    }
    __syncthreads();
    const long segment = long(mb) * Tm * k;
    const long seglen = long(Tm) * k;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        if (!((pm >> e) & 1u)) continue;
        const int j = int((jp >> (4 * e)) & 15u);
        const int rank = bef[e] + wc[wave][e] + rk[e];
        const long pos = long(lofs[e]) + rank;
        const long i = row * k + j;
        if (pos >= 0 && pos < seglen) {
            o.perm[segment + pos] = int32_t(i);
            if (o.inv_perm) o.inv_perm[i] = int32_t(segment + pos);
        }
        o.dropped[i] = (o.capacity >= 0 && rank >= o.capacity) ? 1 : 0;
    }
}

template <int NE, bool VEC, bool BIAS>
hipError_t launch_small_t(const SmallArgs& a, hipStream_t st, const LaunchEvents* ev) {
    const dim3 grid(a.nb + 1, a.out.n_micro), block(kSmallRows);
    auto kern = route_small_kernel<NE, VEC, BIAS>;
    if (ev) {
        hipExtLaunchKernelGGL(kern, grid, block, 0, st, ev->start, ev->stop, 0u, a);
    } else {
        hipLaunchKernelGGL(kern, grid, block, 0, st, a);
    }
    return hipGetLastError();
}

template <int NE>
hipError_t launch_small_ne(const SmallArgs& a, hipStream_t st, const LaunchEvents* ev) {
    const bool bias = a.bias != nullptr;
    if constexpr (NE % 4 == 0) {
        // whole rows of 16-byte vectors when the logits are 16-byte aligned
        if ((reinterpret_cast<uintptr_t>(a.logits) & 15) == 0)
            return bias ? launch_small_t<NE, true, true>(a, st, ev) : launch_small_t<NE, true, false>(a, st, ev);
    }
    return bias ? launch_small_t<NE, false, true>(a, st, ev) : launch_small_t<NE, false, false>(a, st, ev);
}

}  // namespace

bool small_path_fits(int Tm, int E, int k, int n_micro) {
    return E <= kSmallMaxE && (E & (E - 1)) == 0 && k * E <= kSmallMaxPicks && long(Tm) * E <= kSmallMaxLogits &&
           n_micro <= 65535;
}

int small_row_blocks(int Tm) { return (Tm + kSmallRows - 1) / kSmallRows; }

hipError_t launch_route_small(const SmallArgs& a, hipStream_t st, const LaunchEvents* ev) {
    const ScatterArgs& o = a.out;
    if (!small_path_fits(o.Tm, o.E, o.k, o.n_micro) || o.k < 1 || o.k > o.E || a.nb != small_row_blocks(o.Tm))
        return hipErrorInvalidValue;
    switch (o.E) {
        case 1: return launch_small_ne<1>(a, st, ev);
        case 2: return launch_small_ne<2>(a, st, ev);
        case 4: return launch_small_ne<4>(a, st, ev);
        case 8: return launch_small_ne<8>(a, st, ev);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
