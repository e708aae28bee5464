// route_common.hpp -- launch configuration, kernel argument blocks and
// wavefront helpers shared by the gfx950 routing kernels.
//
// Data layout: logits [T,E] fp32 row-major.  A row is handled by a
// "segment" of S lanes of a 64-lane wavefront; lane s of the segment owns the
// G columns c = g*S + s (g < G), so each load instruction of a segment reads
// S consecutive floats of one row and a wave reads 64/S rows at once.
#pragma once

#include <climits>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_route.h"

namespace moe {

// ----------------------------------------------------------------- config
struct RowCfg {
    int S;       // lanes per row (power of two, >= k)
    int G;       // columns per lane
    int VEC;     // floats per load: 4 when E % 4 == 0, else 1
    int PAD;     // 1 when S*G > E (some lane columns fall past the row)
    int NW;      // waves per block
    int R;       // rows of the largest block (blocks differ by at most one row)
    int bpm;     // row blocks per microbatch
    int B;       // row blocks in total (= n_micro * bpm)
    int nsplit;  // block-scan splits per microbatch
};

// Columns per lane that have kernel instantiations.
constexpr int kGTableVec4[] = {4, 8, 16, 24};
constexpr int kGTableVec1[] = {1, 2, 4, 8, 16, 24};
constexpr int kGMax = 24;
constexpr int kScanWaves = 16;     // waves per block-scan block
constexpr int kScanPerWave = 8;    // row blocks per block-scan wave
constexpr int kAssumedCUs = 256;   // MI355X compute units (grid sizing only)

// Waves per row-pass block for S lanes per row and G columns per lane.  As
// many waves per compute unit as the row pass's registers allow: 16 (4 per
// SIMD) when a lane owns up to 16 columns, as two blocks of 8 (blocks of
// half the rows: the combine and the scatter that follow work per row
// block, and the scatter's smaller blocks overlap two per compute unit;
// measured 1.5 us less a step at E=256 top-8 than one block of 16), 12 in
// one block when a lane owns 24.  One or two lanes per row with 16 columns
// hold more per-row state per lane (ranking passes): 12 waves there too, so
// nothing spills; likewise 16 columns of scalar loads (E not a multiple of
// 4), whose kernels spill at the 128-register budget of two blocks of 8
// (E = 250 top-8: 61 -> 55.5 us a call, 140 -> 105 us with masked P; kernels
// of vector loads that spill stay faster as two blocks: E = 60 top-2 with
// masked P 28.2 against 30.2 us as one block of 12).  The
// selection-bias variant reads the bias of its columns
// from the block's LDS copy; it runs the two blocks of 8 as well when it fits
// their register budget (whole rows of vector loads, all-token P: v3 shape
// with a bias 38.7 -> 35.3 us against one block of 12), else one block of 12
// (8 when a lane owns 24).
constexpr int rows_waves(int S, int G, bool bias, bool masked = false, int vec = 4, bool pad = false) {
    if (!bias) return (G > 16 || (S <= 2 && G >= 16) || (vec == 1 && G >= 16)) ? 12 : 8;
    if (G > 16) return 8;
    return (!masked && vec == 4 && !pad && !(S <= 2 && G >= 16)) ? 8 : 12;
}

// Row-pass blocks per compute unit: two for the eight-wave blocks of lanes
// owning up to 16 columns, else one.
constexpr int rows_blocks_per_cu(int NW, int G) { return (NW == 8 && G <= 16) ? 2 : 1; }

inline int next_pow2(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Pick the lane mapping: the narrowest segment (S >= k, power of two) whose
// per-lane column count fits the table; a single lane per row takes at most
// 8 columns (with one lane per row a wave keeps 64 rows' candidate lists and
// row copies in LDS, which at 16 or 24 columns do not fit).  Then the waves
// per block and the rows per block: one or two resident blocks per compute
// unit over the whole batch, so the grid is one wave of blocks and the
// per-block partials stay few.
inline RowCfg choose_rows(int T, int E, int k, int n_micro, bool bias = false, bool masked = false) {
    RowCfg c{};
    c.VEC = (E % 4 == 0) ? 4 : 1;
    int S = next_pow2(k < 1 ? 1 : k);
    while (S < 64 && ((E + S - 1) / S > kGMax || (S == 1 && E > 8))) S <<= 1;
    c.S = S;
    const int g0 = (E + S - 1) / S;
    c.G = -1;
    if (c.VEC == 4) {
        for (int t : kGTableVec4) if (c.G < 0 && g0 <= t) c.G = t;
    } else {
        for (int t : kGTableVec1) if (c.G < 0 && g0 <= t) c.G = t;
    }
    // unaligned rows take the generic (bounds-checked) column path
    c.PAD = (S * c.G != E || c.VEC == 1) ? 1 : 0;
    c.NW = rows_waves(S, c.G, bias, masked, c.VEC, c.PAD != 0);
    const int W = 64 / S;
    const long per_iter = long(c.NW) * W;
    const long Tm = T / n_micro;
    long blocks_per_cu = rows_blocks_per_cu(c.NW, c.G);
    // when two blocks per compute unit would leave each wave one row group,
    // one block with two: the same rows in flight, half the row blocks for
    // the combine and the scatter (65536 tokens, E=64 top-2: step 20.45 ->
    // 20.0 us)
    if (blocks_per_cu == 2 && long(T) <= 2L * kAssumedCUs * per_iter) blocks_per_cu = 1;
    const long target = kAssumedCUs * blocks_per_cu;
    // balanced split: every block of a microbatch gets floor or ceil of
    // Tm / bpm rows, at least one row group per wave iteration
    long bpm = (target + n_micro - 1) / n_micro;
    const long max_bpm = (Tm + per_iter - 1) / per_iter;
    if (bpm > max_bpm) bpm = max_bpm;
    if (bpm < 1) bpm = 1;
    c.bpm = int(bpm);
    c.R = int((Tm + bpm - 1) / bpm);  // rows of the largest block
    c.B = c.bpm * n_micro;
    const int per_split = kScanWaves * kScanPerWave;
    c.nsplit = (c.bpm + per_split - 1) / per_split;
    return c;
}

// Rows [begin, end) of row block b: microbatch b / bpm, balanced split of
// its Tm rows over bpm blocks.
__host__ __device__ inline void block_rows(int b, int bpm, int Tm, long& begin, long& end) {
    const int mb = b / bpm, bi = b - (b / bpm) * bpm;
    begin = long(mb) * Tm + (long(bi) * Tm) / bpm;
    end = long(mb) * Tm + (long(bi + 1) * Tm) / bpm;
}

// Candidate-list capacity per row for the threshold top-k (see route_rows).
__host__ __device__ constexpr int cand_cap(int S, int G) {
    // narrow segments (k <= 4) keep a 16-entry list: fewer ranking passes in
    // registers; a longer candidate list takes the exact fallback
    return (S <= 4) ? ((S * G < 16) ? S * G : 16)
                    : ((S * G < (2 * S > 32 ? 2 * S : 32)) ? S * G : (2 * S > 32 ? 2 * S : 32));
}

// Candidate-list row stride (keys): room for the list padded to a multiple of
// 4 keys (read 4 at a time), plus 2 so that rows start 16-byte aligned on
// different banks.
__host__ __device__ constexpr int cand_stride(int S, int G) { return ((cand_cap(S, G) + 3) & ~3) + 2; }

// LDS row stride (floats) of the row copy: S times an odd number >= G, so
// the segments of a wave start on distinct banks.
__host__ __device__ constexpr int row_stride(int S, int G) { return S * (G | 1); }

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Per-wave capacity of the overflow queue of the row pass: one entry for
// every row the wave can process.
inline int rows_queue_cap(const RowCfg& c) {
    const int W = 64 / c.S;
    const int per_iter = c.NW * W;
    return ((c.R + per_iter - 1) / per_iter) * W;
}

inline size_t rows_lds_bytes(const RowCfg& c, int E, int k, bool bias = false) {
    const int W = 64 / c.S;
    size_t hist = align_up(size_t(E) * 4, 16) * (bias ? 2 : 1);
    size_t rowbuf = size_t(c.NW) * W * row_stride(c.S, c.G) * 4;
    size_t cand = size_t(c.NW) * W * cand_stride(c.S, c.G) * 8;
    size_t sel = size_t(c.NW) * W * k * 8;
    size_t queue = size_t(c.NW) * rows_queue_cap(c) * 4;
    return hist + align_up(rowbuf, 16) + cand + sel + queue;
}

// Workspace carve-up (each piece 256-byte aligned).
struct Workspace {
    int32_t* cnt_part;    // [B,E]        per-block histograms
    float*   P_part;      // [B,E]        per-block probability sums
    int32_t* flag_part;   // [B]          per-block status bits
    int32_t* colprefix;   // [B,E]        exclusive prefix over the blocks of a split
    int32_t* split_tot;   // [m,nsplit,E] counts per split
    double*  split_P;     // [m,nsplit,E] probability sums per split
    uint16_t* Wt;         // gate weights laid out as the MFMA B operand (gate path only)
    size_t   bytes;
};

inline Workspace carve_workspace(void* base, const RowCfg& c, int E, int m, size_t gate_bytes) {
    Workspace w{};
    size_t off = 0;
    auto take = [&](size_t n) {
        size_t o = off;
        off = align_up(off + n, 256);
        return o;
    };
    const size_t B = size_t(c.B), ns = size_t(c.nsplit);
    size_t o_cnt = take(B * E * 4);
    size_t o_P = take(B * E * 4);
    size_t o_flag = take(B * 4);
    size_t o_pre = take(B * E * 4);
    size_t o_tot = take(size_t(m) * ns * E * 4);
    size_t o_ps = take(size_t(m) * ns * E * 8);
    size_t o_wt = take(gate_bytes);
    w.bytes = off;
    char* b = static_cast<char*>(base);
    if (b) {
        w.cnt_part = reinterpret_cast<int32_t*>(b + o_cnt);
        w.P_part = reinterpret_cast<float*>(b + o_P);
        w.flag_part = reinterpret_cast<int32_t*>(b + o_flag);
        w.colprefix = reinterpret_cast<int32_t*>(b + o_pre);
        w.split_tot = reinterpret_cast<int32_t*>(b + o_tot);
        w.split_P = reinterpret_cast<double*>(b + o_ps);
        w.Wt = gate_bytes ? reinterpret_cast<uint16_t*>(b + o_wt) : nullptr;
    }
    return w;
}

// ------------------------------------------------------- kernel arguments
struct RowsArgs {
    const float* logits;
    const float* bias;  // [E] selection bias, or nullptr
    int T, E, k, Tm, R, bpm;
    int renorm, save_stats;
    int p_masked;  // P from the picks only (divided by Tm*k by the scatter)
    int qcap;  // per-wave queue entries: row groups of the largest block times rows per group
    int32_t* topk_idx;
    float* topk_w;
    float* row_stats;
    int32_t* cnt_part;
    float* P_part;
    int32_t* flag_part;
    int32_t* status;  // nullable; zeroed by block 0 (the later kernels OR bits in)
};

struct ScanArgs {
    const int32_t* cnt_part;
    const float* P_part;
    const int32_t* flag_part;
    int E, k, Tm, bpm, n_micro, B, nsplit;
    int32_t* colprefix;
    int32_t* split_tot;
    double* split_P;
    int32_t* status;
};

struct ScatterArgs {
    const int32_t* topk_idx;
    const int32_t* colprefix;   // from the block combine (fold_q == 0)
    const int32_t* split_tot;
    const double* split_P;
    const int32_t* cnt_part;    // the row pass's partials (fold_q > 0)
    const float* P_part;
    const int32_t* flag_part;
    int fold_q;  // > 0: sum the row pass's partials here, in fold_q groups of row blocks
    int stats_sep;  // 1: n_micro extra workgroups form the statistics (B + n_micro fit the chip)
    int n_micro;
    int nw;      // waves per block (scatter_waves)
    int B;       // row blocks in total
    int T, E, k, Tm, bpm, nsplit;
    int rows_per_wave;  // rows a wave ranks per window (<= 64, one mask bit each)
    int capacity;  // < 0: unlimited
    int vec_idx;   // topk_idx 16-byte aligned and k % 4 == 0: vector index loads
    float alpha;
    int p_masked;  // P_e = probability sum / (Tm*k) instead of / Tm
    int32_t* perm;
    int32_t* inv_perm;
    uint8_t* dropped;
    int32_t* status;
    // per-microbatch results, written by the microbatch's statistics
    // workgroup or shared by its first six blocks
    int32_t* counts;
    int32_t* offsets;
    float* f;
    float* P;
    float* aux;
    float* cv;
    float* max_over_mean;
    float* extra;
    // one microbatch only: the selection bias to step from these counts once
    // the statistics are formed (nullptr: none), and the step
    float* upd_bias;
    float upd_gamma;
};

// One-launch path for small microbatches (route_small.hip): E a power of
// two up to kSmallMaxE, k*E up to kSmallMaxPicks and at most kSmallMaxLogits
// logits a microbatch, where every workgroup selects the whole microbatch
// itself (its cost grows with k*E per row and with the microbatch).
constexpr int kSmallMaxE = 8;
constexpr int kSmallMaxPicks = 16;
constexpr long kSmallMaxLogits = 32768;

struct SmallArgs {
    const float* logits;
    const float* bias;  // [E] selection bias, or nullptr
    int nb;             // row blocks per microbatch (small_row_blocks)
    int renorm, save_stats;
    int32_t* topk_idx;
    float* topk_w;
    float* row_stats;
    ScatterArgs out;    // sizes, capacity, alpha, permutation and statistics outputs
};

struct BackArgs {
    const float* logits;
    const float* row_stats;
    const int32_t* counts;
    const float* d_aux;
    const int32_t* topk_idx;  // [T,k]; needed for p_masked and d_topk_w
    const float* d_topk_w;    // [T,k] upstream gradient of the gate weights, or nullptr
    float* dlogits;
    int T, E, k, Tm, R, bpm;
    float alpha;
    int p_masked, renorm;
};

// LDS of the backward's sparse variant: f [E4], then per segment two [E4]
// row buffers.
inline size_t backward_lds_bytes(const RowCfg& c, int E) {
    const size_t E4 = size_t((E + 3) & ~3);
    return (E4 + size_t(c.NW) * (64 / c.S) * 2 * E4) * 4;
}

struct BiasArgs {
    const int32_t* counts;  // [m,E]
    float* bias;            // [E], updated in place
    int E, n_micro;
    int64_t Tk;             // T * k
    float gamma;
};

struct GateBackArgs {
    const uint16_t* X;       // [T,d] bf16 bits
    const uint16_t* Wg;      // [d,E] bf16 bits
    const float* dlogits;    // [T,E]
    uint16_t* dX;            // [T,d] bf16 bits, or nullptr
    float* dWg;              // [d,E], or nullptr
    float* dWg_part;         // [slices,d,E] workspace
    int T, d, E;
};

struct EplbArgs {
    const int32_t* weight;  // [E] loads (e.g. one row of moe_route's counts)
    int32_t* phy2log;       // [P]
    int32_t* phy_rank;      // [P]
    int32_t* logcnt;        // [E]
    int32_t* pack;          // [P]
    int32_t* slot;          // [P]
    double* pack_load;      // [num_packs]
    int E, num_phys, num_packs;
};

struct SinkhornArgs {
    const double* supply;  // [R]
    const double* demand;  // [R]
    const double* C;       // [R,R]
    double* u;             // [R]
    double* v;             // [R]
    double* T;             // [R,R]
    double eps;
    int R, iters;
};

struct GateArgs {
    const uint16_t* X;
    const uint16_t* Wg;
    float* logits;
    int T, d, E;
};

// Optional timing of one launch: the runtime stamps start and stop from the
// kernel's own dispatch (hipExtLaunchKernel), as a kernel trace does.
struct LaunchEvents {
    hipEvent_t start;
    hipEvent_t stop;
};

// Launchers (each defined next to its kernel).  Return a hipError_t.
hipError_t launch_route_rows(const RowCfg& c, const RowsArgs& a, hipStream_t st, const LaunchEvents* ev);
template <int S>
hipError_t launch_rows_s(const RowCfg& c, const RowsArgs& a, hipStream_t st, const LaunchEvents* ev);
template <int S>
hipError_t launch_backward_s(const RowCfg& c, const BackArgs& a, hipStream_t st);
#define MOE_DECLARE_SEGMENT(SV)                                                           \
    template <> hipError_t launch_rows_s<SV>(const RowCfg&, const RowsArgs&, hipStream_t, const LaunchEvents*); \
    template <> hipError_t launch_backward_s<SV>(const RowCfg&, const BackArgs&, hipStream_t);
MOE_DECLARE_SEGMENT(1) MOE_DECLARE_SEGMENT(2) MOE_DECLARE_SEGMENT(4) MOE_DECLARE_SEGMENT(8)
MOE_DECLARE_SEGMENT(16) MOE_DECLARE_SEGMENT(32) MOE_DECLARE_SEGMENT(64)
#undef MOE_DECLARE_SEGMENT
hipError_t launch_route_scan(const RowCfg& c, const ScanArgs& a, hipStream_t st);
hipError_t launch_route_scatter(const RowCfg& c, const ScatterArgs& a, hipStream_t st);
int scatter_waves(int E, int row_nw);
int scatter_rows_per_wave(int E, int k, int NW);
size_t scatter_lds_bytes(int E, int k, int NW);
int scatter_fold_groups(int E, int k, int bpm, int NW);
hipError_t launch_route_backward(const RowCfg& c, const BackArgs& a, hipStream_t st);
bool small_path_fits(int Tm, int E, int k, int n_micro);
int small_row_blocks(int Tm);
hipError_t launch_route_small(const SmallArgs& a, hipStream_t st, const LaunchEvents* ev);
hipError_t launch_bias_update(const BiasArgs& a, hipStream_t st);
hipError_t launch_gate_backward(const GateBackArgs& a, hipStream_t st);
hipError_t launch_eplb(const EplbArgs& a, hipStream_t st);
hipError_t launch_sinkhorn(const SinkhornArgs& a, hipStream_t st);
size_t eplb_lds_bytes(int E, int num_phys);
int gate_backward_slices(int T, int d, int E);
size_t gate_backward_workspace_bytes(int T, int d, int E);
hipError_t launch_gate_gemm(const GateArgs& a, uint16_t* wt, hipStream_t st);
bool gate_supported(int T, int d, int E);
size_t gate_workspace_bytes(int d, int E);

}  // namespace moe

// ------------------------------------------------------- device helpers
#ifdef __HIP_DEVICE_COMPILE__
#define MOE_DEV __device__ __forceinline__
#else
#define MOE_DEV __device__ inline
#endif

namespace moe {
namespace dev {

constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// DPP move with a compile-time control word (row/bank masks full).
// DPP move with a compile-time control word (row/bank masks full; lanes with
// no source read 0), foldable into the instruction that consumes it.
template <int CTRL>
MOE_DEV float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
MOE_DEV int dppi(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

// Partner value for a butterfly step of distance D inside aligned groups of
// 2D lanes.  D = 1, 2 use quad permutes; D = 4, 8 use the half-row / row
// mirrors (partner in the other half of the 8- or 16-lane group, which is
// all an all-reduce needs); D = 16 a swizzle; D = 32 a bpermute.
template <int D>
MOE_DEV float xstep(float v) {
    if constexpr (D == 1) return dpp<0xB1>(v);        // quad_perm [1,0,3,2]
    else if constexpr (D == 2) return dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    else if constexpr (D == 4) return dpp<0x141>(v);  // row_half_mirror
    else if constexpr (D == 8) return dpp<0x140>(v);  // row_mirror
    else if constexpr (D == 16)
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
    else return __shfl_xor(v, 32);
}
// Value of lane (lane XOR D): a true exchange, for per-lane (not
// group-uniform) data.
template <int D>
MOE_DEV float xor_lane(float v) {
    if constexpr (D == 1) return dpp<0xB1>(v);
    else if constexpr (D == 2) return dpp<0x4E>(v);
    else if constexpr (D < 32)
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (D << 10)));
    else return __shfl_xor(v, 32);
}

template <int D>
MOE_DEV int xstepi(int v) {
    return __float_as_int(xstep<D>(__int_as_float(v)));
}

template <int S>
MOE_DEV float seg_max(float v) {
    if constexpr (S >= 2) v = fmaxf(v, xstep<1>(v));
    if constexpr (S >= 4) v = fmaxf(v, xstep<2>(v));
    if constexpr (S >= 8) v = fmaxf(v, xstep<4>(v));
    if constexpr (S >= 16) v = fmaxf(v, xstep<8>(v));
    if constexpr (S >= 32) v = fmaxf(v, xstep<16>(v));
    if constexpr (S >= 64) v = fmaxf(v, xstep<32>(v));
    return v;
}

template <int S>
MOE_DEV float seg_sum(float v) {
    if constexpr (S >= 2) v += xstep<1>(v);
    if constexpr (S >= 4) v += xstep<2>(v);
    if constexpr (S >= 8) v += xstep<4>(v);
    if constexpr (S >= 16) v += xstep<8>(v);
    if constexpr (S >= 32) v += xstep<16>(v);
    if constexpr (S >= 64) v += xstep<32>(v);
    return v;
}

template <int S>
MOE_DEV int seg_sumi(int v) {
    if constexpr (S >= 2) v += xstepi<1>(v);
    if constexpr (S >= 4) v += xstepi<2>(v);
    if constexpr (S >= 8) v += xstepi<4>(v);
    if constexpr (S >= 16) v += xstepi<8>(v);
    if constexpr (S >= 32) v += xstepi<16>(v);
    if constexpr (S >= 64) v += xstepi<32>(v);
    return v;
}

// Maximum over the whole wave of a value that is uniform inside each
// segment of S lanes; the result is wave-uniform.
template <int S>
MOE_DEV int wave_max_over_segments(int v) {
    if constexpr (S <= 1) v = max(v, xstepi<1>(v));
    if constexpr (S <= 2) v = max(v, xstepi<2>(v));
    if constexpr (S <= 4) v = max(v, xstepi<4>(v));
    if constexpr (S <= 8) v = max(v, xstepi<8>(v));
    if constexpr (S <= 16) v = max(v, xstepi<16>(v));
    if constexpr (S <= 32) v = max(v, xstepi<32>(v));
    return __builtin_amdgcn_readfirstlane(v);
}

// Inclusive prefix sum over the lanes of a segment (lane s gets the sum of
// lanes 0..s of its segment): Hillis-Steele shifts inside 16-lane rows, then
// the total of the preceding row(s) for segments wider than a row.
template <int S>
MOE_DEV int seg_incl_scan(int v, int s) {
    if constexpr (S >= 16) {
        // segments are whole rows: lanes shifted in from before the row read 0
        v += dppi<0x111>(v);  // row_shr:1
        v += dppi<0x112>(v);  // row_shr:2
        v += dppi<0x114>(v);  // row_shr:4
        v += dppi<0x118>(v);  // row_shr:8
    } else {
        if constexpr (S >= 2) { int t = dppi<0x111>(v); v += (s >= 1) ? t : 0; }
        if constexpr (S >= 4) { int t = dppi<0x112>(v); v += (s >= 2) ? t : 0; }
        if constexpr (S >= 8) { int t = dppi<0x114>(v); v += (s >= 4) ? t : 0; }
    }
    if constexpr (S >= 32) {
        const int lane = __lane_id();
        int t = __shfl(v, (lane & ~31) | 15);
        v += (s & 16) ? t : 0;
    }
    if constexpr (S >= 64) {
        int t = __shfl(v, 31);
        v += (s & 32) ? t : 0;
    }
    return v;
}

// Value held by another lane of the same segment; over R = 1..S-1 every
// other lane of the segment is visited exactly once.
template <int S, int R>
MOE_DEV float seg_other(float v) {
    static_assert(R >= 1 && R < S, "bad segment offset");
    if constexpr (S == 2 || S == 4) {
        // quad_perm with lane' = lane ^ R
        constexpr int q0 = 0 ^ R, q1 = 1 ^ R, q2 = 2 ^ R, q3 = 3 ^ R;
        return dpp<(q0 | (q1 << 2) | (q2 << 4) | (q3 << 6))>(v);
    } else if constexpr (S == 16) {
        return dpp<0x120 + R>(v);  // row_ror:R
    } else if constexpr (S == 8 || S == 32) {
        // swizzle, bit-mask mode: lane' = lane ^ R inside 32-lane groups
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (R << 10)));
    } else {
        return __shfl_xor(v, R);
    }
}

// Order key of (logit, expert): a larger key means "earlier in the top-k
// order" -- larger logit, or equal logit and lower expert.  The logit is
// canonicalised (-0.0 -> +0.0) and mapped to an order-preserving unsigned
// integer in the high word; the low word is ~expert.
MOE_DEV uint64_t make_key(float v, int col) {
    uint32_t u = __float_as_uint(v + 0.0f);
    uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (uint64_t(ord) << 32) | uint32_t(0xFFFFFFFFu - uint32_t(col));
}
MOE_DEV int key_col(uint64_t key) { return int(0xFFFFFFFFu - uint32_t(key)); }
MOE_DEV float key_val(uint64_t key) {
    uint32_t ord = uint32_t(key >> 32);
    uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
    return __uint_as_float(u);
}

MOE_DEV uint64_t shfl_xor_u64(uint64_t v, int m) {
    int lo = __shfl_xor(int(uint32_t(v)), m);
    int hi = __shfl_xor(int(uint32_t(v >> 32)), m);
    return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
}

template <int S>
MOE_DEV uint64_t seg_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 1; m < S; m <<= 1) {
        uint64_t o = shfl_xor_u64(v, m);
        v = o > v ? o : v;
    }
    return v;
}

MOE_DEV double shfl_xor_f64(double v, int m) {
    uint64_t u = __double_as_longlong(v);
    return __longlong_as_double((long long)shfl_xor_u64(u, m));
}

// Whole-wave reductions without LDS traffic: butterflies inside each 16-lane
// row through DPP (every lane of a row ends with the row's value), then the
// four rows combined in row order from readlanes.  Deterministic; the result
// is wave-uniform.
template <int D>
MOE_DEV double xstep_f64(double v) {
    const int lo = xstepi<D>(__double2loint(v));
    const int hi = xstepi<D>(__double2hiint(v));
    return __hiloint2double(hi, lo);
}
MOE_DEV double readlane_f64(double v, int l) {
    const int lo = __builtin_amdgcn_readlane(__double2loint(v), l);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(v), l);
    return __hiloint2double(hi, lo);
}
MOE_DEV double wave_sum_f64(double v) {
    v += xstep_f64<1>(v);
    v += xstep_f64<2>(v);
    v += xstep_f64<4>(v);
    v += xstep_f64<8>(v);
    return ((readlane_f64(v, 0) + readlane_f64(v, 16)) + readlane_f64(v, 32)) + readlane_f64(v, 48);
}
MOE_DEV int wave_max_i(int v) {
    v = max(v, xstepi<1>(v));
    v = max(v, xstepi<2>(v));
    v = max(v, xstepi<4>(v));
    v = max(v, xstepi<8>(v));
    return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
MOE_DEV int wave_min_i(int v) {
    v = min(v, xstepi<1>(v));
    v = min(v, xstepi<2>(v));
    v = min(v, xstepi<4>(v));
    v = min(v, xstepi<8>(v));
    return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
MOE_DEV double wave_min_f64(double v) {
    v = fmin(v, xstep_f64<1>(v));
    v = fmin(v, xstep_f64<2>(v));
    v = fmin(v, xstep_f64<4>(v));
    v = fmin(v, xstep_f64<8>(v));
    return fmin(fmin(readlane_f64(v, 0), readlane_f64(v, 16)), fmin(readlane_f64(v, 32), readlane_f64(v, 48)));
}
MOE_DEV double wave_max_f64(double v) {
    v = fmax(v, xstep_f64<1>(v));
    v = fmax(v, xstep_f64<2>(v));
    v = fmax(v, xstep_f64<4>(v));
    v = fmax(v, xstep_f64<8>(v));
    return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)), fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}
// Inclusive prefix sum over the 64 lanes of a wave.
MOE_DEV int wave_incl_scan_i(int v) { return seg_incl_scan<64>(v, __lane_id()); }

// Load p[i] when ok, else return dflt -- always from a valid address (index 0
// stands in), so the load is issued unconditionally and independent loads
// overlap instead of each waiting inside its own branch.
template <class T>
MOE_DEV T load_or(const T* p, long i, bool ok, T dflt) {
    const T v = p[ok ? i : 0];
    return ok ? v : dflt;
}

// Counts, offsets and balance statistics of microbatch mb, by one block of
// NW waves, from the counts tot[0..E) and their exclusive prefix lofs[0..E]
// (both in LDS), in fp64 with every sum in a fixed order:
//   f_e = counts_e/(Tm*k) and P_e = probability sum/Tm (or /(Tm*k) for the
//   masked form of mhpq.cn section 4.4, whose sums cover the picks only) with
//   aux = alpha*E*sum_e f_e*P_e (mhpq.cn sections 4.2, 4.4; codechina.net
//   article 413310 section 2.2), CV = population std/mean and balance degree
//   1-(max-mean)/mean (page cnvsn.com/news/335486 sections 3.1, 5.1),
//   max/mean load (mhpq.cn section 5.4), entropy and max/min share of f
//   (codechina.net section 4.2), kept and dropped assignments under C.
// Every thread forms the terms of its experts (psum[it]: the probability sum
// of expert tid + it*NW*64 over the splits) into q, four arrays of E doubles
// in LDS; then waves 0..5 each reduce one quantity (lane-strided sums in
// expert order, then the lanes) and write its results.  q is free LDS
// scratch of the caller; the function ends with a barrier.
// parts selects what this block forms, so that several blocks can share
// the work: bit 0 the per-expert outputs (counts, offsets, f, P) and the aux
// loss -- the only part that reads psum --, bit w (w = 1..5) the quantity
// wave w reduces; kStatsAll is everything.
constexpr int kStatsAll = 0x3F;
template <int NW, int EPT>
__device__ void microbatch_statistics(const ScatterArgs& a, int mb, const int* tot, const int* lofs,
                                      const double* psum, double* q, int parts = kStatsAll) {
    static_assert(NW >= 6, "one wave per reduced quantity");
    const int E = a.E;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const double total = double(a.Tm) * double(a.k);
    const double mean = total / double(E);
    const long cb = long(mb) * E;
    // f and P scale by reciprocals formed once (within an ulp of dividing)
    const double inv_total = 1.0 / total;
    const double inv_pden = a.p_masked ? inv_total : 1.0 / double(a.Tm);
#pragma unroll
    for (int it = 0; it < EPT; ++it) {
        const int e = tid + it * NW * 64;
        if (e >= E) break;
        const int cnt = tot[e];
        const double fe = double(cnt) * inv_total;
        if (parts & 1) {
            const double pe = psum[it] * inv_pden;
            a.counts[cb + e] = cnt;
            a.offsets[long(mb) * (E + 1) + e] = lofs[e];
            if (a.f) a.f[cb + e] = float(fe);
            if (a.P) a.P[cb + e] = float(pe);
            q[e] = fe * pe;
        }
        if (parts & 2) q[E + e] = (double(cnt) - mean) * (double(cnt) - mean);
        // -f ln f with a hardware fp32 log2 (about 1e-7 relative per term;
        // the terms share one sign, so the sum keeps that precision)
        if (parts & 4)
            q[2 * E + e] = fe > 0.0 ? -fe * (double(__builtin_amdgcn_logf(float(fe))) * 0.69314718055994531) : 0.0;
        if (parts & 8) q[3 * E + e] = double((a.capacity >= 0 && cnt > a.capacity) ? a.capacity : cnt);
    }
    __syncthreads();
    if (wave < 6 && !((parts >> wave) & 1)) {
        // not this block's quantity
    } else if (wave < 4) {
        // sum of terms: f.P, squared deviations, entropy terms, kept
        const double* v = q + wave * E;
        double acc = 0.0;
        for (int e = lane; e < E; e += 64) acc += v[e];
        acc = wave_sum_f64(acc);
        if (lane == 0) {
            float* x = a.extra ? a.extra + long(mb) * 8 : nullptr;
            if (wave == 0) {
                a.aux[mb] = float(double(a.alpha) * double(E) * acc);
                a.offsets[long(mb) * (E + 1) + E] = lofs[E];
            } else if (wave == 1) {
                a.cv[mb] = float(sqrt(acc / double(E)) / mean);
            } else if (wave == 2) {
                if (x) x[2] = float(acc);
            } else if (x) {
                x[3] = float(acc);
                x[4] = float(total - acc);
                x[5] = float(a.capacity);
            }
        }
    } else if (wave < 6) {
        // largest (wave 4) and smallest (wave 5) count
        int m = (wave == 4) ? -1 : INT_MAX;
        for (int e = lane; e < E; e += 64) m = (wave == 4) ? max(m, tot[e]) : min(m, tot[e]);
        m = (wave == 4) ? wave_max_i(m) : wave_min_i(m);
        if (lane == 0) {
            float* x = a.extra ? a.extra + long(mb) * 8 : nullptr;
            if (wave == 4) {
                a.max_over_mean[mb] = float(double(m) / mean);
                if (x) {
                    x[1] = float(1.0 - (double(m) - mean) / mean);
                    x[6] = float(double(m) / total);
                }
            } else if (x) {
                x[0] = float(double(m) / mean);
                x[7] = float(double(m) / total);
            }
        }
    }
    __syncthreads();
}

}  // namespace dev
}  // namespace moe
