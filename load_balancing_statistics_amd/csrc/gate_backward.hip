// gate_backward.hip -- backward of the gate GEMM logits = X[T,d] . Wg[d,E]:
//   dX  = dlogits . Wg^T   [T,d]  (bf16, rounded to nearest even)
//   dWg = X^T . dlogits    [d,E]  (fp32)
// The gate (router) network of page codechina.net article 413310 section 1.2;
// dlogits is the routing gradient with respect to the logits.
//
// Both products stream X (or dX) once and are bound by HBM (about 6 flop per
// byte), fused in one pass.  For E <= 8 both run on bf16 matrix cores with
// dlogits split exactly into three bf16 parts (gate_backward_bf16_kernel,
// below); for 8 < E <= 16 on fp32 matrix cores (v_mfma_f32_16x16x4_f32, fp32
// in and out), as follows.  dWg, the reduction over
// tokens: 16 lanes share a row, lane n of a row holds CPL consecutive
// columns, and a step of four rows is, for each of the lane's CPL column
// offsets q, the product of A = dlogits [16 experts x 4 rows] (lane l: row
// l/16, expert l%16) and B_q = X [4 rows x 16 columns] (lane l: row l/16,
// column CPL*(l%16) + q), accumulated in a 16 x 16 tile per q.  dX, per 16
// rows of a wave: see the kernel; its tile goes through LDS so that every
// store writes whole runs of a row.  dX is stored nontemporally: nothing
// here reads it again, and its dirty lines, written back later, would
// otherwise slow the next kernel's reads of X by a third.
//
// For 16 < E <= 64 both products run on the vector ALUs.  A block owns a
// 64-column tile of X over a contiguous slice of the tokens; a lane owns CPL
// consecutive columns of one row per step (CPL = 2, 1 for E <= 32, 64,
// keeping CPL*E <= 64 fp32 accumulators), so a row's 64 columns are 128
// contiguous bytes.  Per row the lane reads its X chunk and the row's E
// gradients, writes its dX chunk (its CPL x E slice of Wg stays in registers)
// and adds X * dlogits into its dWg accumulators.  The accumulators are
// reduced over the lanes and waves of the block in a fixed order into a
// per-slice partial; a second kernel sums the slices in order.
// Deterministic: no atomics.
#include "route_common.hpp"

namespace moe {
namespace {

constexpr int kGbWaves = 4;
constexpr int kGbThreads = kGbWaves * 64;
constexpr int kTile = 64;   // columns per block
constexpr int kRowUnroll = 4;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
    return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <int CPL>
__global__ void __launch_bounds__(kGbThreads)
gate_backward_kernel(const GateBackArgs a)
{
    constexpr int EMAX = 64 / CPL;
    constexpr int LPR = kTile / CPL;       // lanes per row
    constexpr int RPI = 64 / LPR;          // rows per wave step
    const int E = a.E, d = a.d;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cl = lane % LPR, rl = lane / LPR;
    const int col0 = blockIdx.x * kTile + cl * CPL;
    const bool col_ok = col0 < d;              // d % 8 == 0 and CPL <= 8: whole chunk in or out
    const long t0 = (long(blockIdx.y) * a.T) / gridDim.y;
    const long t1 = (long(blockIdx.y + 1) * a.T) / gridDim.y;

    // the lane's CPL x E slice of Wg
    float wg[CPL][EMAX];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
            wg[c][e] = (col_ok && e < E) ? bf16_to_f32(a.Wg[long(col0 + c) * E + e]) : 0.f;
    float acc[CPL][EMAX];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int e = 0; e < EMAX; ++e) acc[c][e] = 0.f;

    const long step = long(kGbWaves) * RPI;
    for (long r0 = t0 + long(wave) * RPI + rl; r0 < t1; r0 += step * kRowUnroll) {
        uint16_t xv[kRowUnroll][CPL];
        float gv[kRowUnroll][EMAX];
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            const long r = r0 + u * step;
            const bool in = r < t1;
            const long rr = in ? r : t0;
            if constexpr (CPL == 8) {
                const uint4 v = (col_ok) ? *reinterpret_cast<const uint4*>(a.X + rr * d + col0)
                                         : make_uint4(0, 0, 0, 0);
                xv[u][0] = uint16_t(v.x); xv[u][1] = uint16_t(v.x >> 16);
                xv[u][2] = uint16_t(v.y); xv[u][3] = uint16_t(v.y >> 16);
                xv[u][4] = uint16_t(v.z); xv[u][5] = uint16_t(v.z >> 16);
                xv[u][6] = uint16_t(v.w); xv[u][7] = uint16_t(v.w >> 16);
            } else {
#pragma unroll
                for (int c = 0; c < CPL; ++c) xv[u][c] = col_ok ? a.X[rr * d + col0 + c] : uint16_t(0);
            }
#pragma unroll
            for (int e = 0; e < EMAX; ++e) gv[u][e] = (e < E) ? a.dlogits[rr * E + e] : 0.f;
            if (!in) {
#pragma unroll
                for (int e = 0; e < EMAX; ++e) gv[u][e] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            const long r = r0 + u * step;
            float xf[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) xf[c] = bf16_to_f32(xv[u][c]);
#pragma unroll
            for (int c = 0; c < CPL; ++c)
#pragma unroll
                for (int e = 0; e < EMAX; ++e) acc[c][e] = fmaf(xf[c], gv[u][e], acc[c][e]);
            if (a.dX && col_ok && r < t1) {
                uint16_t o[CPL];
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    float s = 0.f;
#pragma unroll
                    for (int e = 0; e < EMAX; ++e) s = fmaf(gv[u][e], wg[c][e], s);
                    o[c] = f32_to_bf16(s);
                }
                if constexpr (CPL == 8) {
                    uint4 v;
                    v.x = uint32_t(o[0]) | (uint32_t(o[1]) << 16);
                    v.y = uint32_t(o[2]) | (uint32_t(o[3]) << 16);
                    v.z = uint32_t(o[4]) | (uint32_t(o[5]) << 16);
                    v.w = uint32_t(o[6]) | (uint32_t(o[7]) << 16);
                    *reinterpret_cast<uint4*>(a.dX + r * d + col0) = v;
                } else {
#pragma unroll
                    for (int c = 0; c < CPL; ++c) a.dX[r * d + col0 + c] = o[c];
                }
            }
        }
    }

    if (!a.dWg_part) return;
    // reduce over the lanes that share columns (rows rl of the step): xor
    // steps LPR, 2*LPR, ... below 64, in a fixed order
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int e = 0; e < EMAX; ++e) {
            float v = acc[c][e];
#pragma unroll
            for (int m = LPR; m < 64; m <<= 1) v += __shfl_xor(v, m);
            acc[c][e] = v;
        }
    // then over the waves, in wave order, through one LDS tile
    __shared__ float wred[kTile][EMAX];
    for (int w = 0; w < kGbWaves; ++w) {
        if (wave == w && rl == 0) {
#pragma unroll
            for (int c = 0; c < CPL; ++c)
#pragma unroll
                for (int e = 0; e < EMAX; ++e) {
                    float& slot = wred[cl * CPL + c][e];
                    slot = (w == 0) ? acc[c][e] : slot + acc[c][e];
                }
        }
        __syncthreads();
    }
    float* part = a.dWg_part + long(blockIdx.y) * d * E;
    for (int i = threadIdx.x; i < kTile * E; i += kGbThreads) {
        const int cc = i / E, e = i - (i / E) * E;
        const int col = blockIdx.x * kTile + cc;
        if (col < d) part[long(col) * E + e] = wred[cc][e];
    }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kMfWaves = 4;
constexpr int kMfRowSteps = 8;  // 4-row steps whose loads are issued together
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

template <int CTRL>
__device__ __forceinline__ float row_bcast(float v) {  // lane CTRL - 0x150 of the 16-lane row
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// EM: experts padded (8 or 16); CPL: columns per lane (tile = 16 * CPL).
//
// dWg: as described at the top.  dX on the matrix cores too: for each group
// of 16 rows of the wave (four 4-row steps) and each 16-column tile t of the
// block, D_t[i][j] = sum_e Wg[col(t,i)][e] * dlogits[row(j)][e] in EM/4
// products of K = 4 (v_mfma_f32_16x16x4_f32: lane l gives A = Wg[col(t,l%16)]
// [4h + l/16] and B = dlogits[row(l%16)][4h + l/16] and receives D[4(l/16)+m]
// [l%16]).  With col(t, i) = 4*CPL*(i/4) + 4t + i%4, lane l ends up with
// 4*CPL consecutive columns of row l%16; the tile is packed to bf16 and
// passed through LDS, so that each store writes a row's columns of the X
// layout (16 lanes per row, contiguous).
template <int EM, int CPL>
__global__ void __launch_bounds__(kMfWaves * 64)
gate_backward_mfma_kernel(const GateBackArgs a)
{
    constexpr int kTileM = 16 * CPL;
    constexpr int KH = EM / 4;
    constexpr int kPitch = kTileM * 2 + 16;   // bytes per staged dX row
    __shared__ __attribute__((aligned(16))) unsigned char dxs[kMfWaves][16 * kPitch];
    const int E = a.E, d = a.d;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, r = lane >> 4;  // column group, row of the 4-row step
    const int col0 = blockIdx.x * kTileM + CPL * n;
    const bool col_ok = col0 < d;            // d % 8 == 0: a lane's columns are all in or all out
    const long t0 = (long(blockIdx.y) * a.T) / gridDim.y;
    const long t1 = (long(blockIdx.y + 1) * a.T) / gridDim.y;
    unsigned char* stage = dxs[wave];

    // dX A operands: Wg[col(t, n)][4h + r]
    float wa[CPL][KH];
#pragma unroll
    for (int t = 0; t < CPL; ++t)
#pragma unroll
        for (int h = 0; h < KH; ++h) {
            const int c = blockIdx.x * kTileM + 4 * CPL * (n >> 2) + 4 * t + (n & 3);
            const int e = 4 * h + r;
            wa[t][h] = (a.dX && c < d && e < E) ? bf16_to_f32(a.Wg[long(c) * E + e]) : 0.f;
        }
    f32x4 acc[CPL];
#pragma unroll
    for (int q = 0; q < CPL; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};

    const long step = 4L * kMfWaves;
    for (long s0 = t0 + 4L * wave; s0 < t1; s0 += step * kMfRowSteps) {
        uint32_t xv[kMfRowSteps][CPL / 2];
        float dv[kMfRowSteps];
        float gb[kMfRowSteps / 4][KH];
#pragma unroll
        for (int u = 0; u < kMfRowSteps; ++u) {
            const long row = s0 + u * step + r;
            const bool in = row < t1;
            const long rr = in ? row : t0;
            if constexpr (CPL == 8) {
                const uint4 v = col_ok ? *reinterpret_cast<const uint4*>(a.X + rr * d + col0) : make_uint4(0, 0, 0, 0);
                xv[u][0] = v.x; xv[u][1] = v.y; xv[u][2] = v.z; xv[u][3] = v.w;
            } else {
                const uint2 v = col_ok ? *reinterpret_cast<const uint2*>(a.X + rr * d + col0) : make_uint2(0, 0);
                xv[u][0] = v.x; xv[u][1] = v.y;
            }
            const float g = (n < E) ? a.dlogits[rr * E + n] : 0.f;
            dv[u] = in ? g : 0.f;  // rows past the slice add nothing to dWg
        }
        if (a.dX) {
            // B operands of the two 16-row groups: row(G, j) = s0 + (4G + j/4)*step + j%4, j = n
#pragma unroll
            for (int G = 0; G < kMfRowSteps / 4; ++G) {
                const long row = s0 + (4 * G + (n >> 2)) * step + (n & 3);
#pragma unroll
                for (int h = 0; h < KH; ++h) {
                    const int e = 4 * h + r;
                    gb[G][h] = (row < t1 && e < E) ? a.dlogits[row * E + e] : 0.f;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kMfRowSteps; ++u) {
            float x[CPL];
#pragma unroll
            for (int h = 0; h < CPL / 2; ++h) {
                x[2 * h] = bf16_to_f32(uint16_t(xv[u][h]));
                x[2 * h + 1] = bf16_to_f32(uint16_t(xv[u][h] >> 16));
            }
#pragma unroll
            for (int q = 0; q < CPL; ++q) acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(dv[u], x[q], acc[q], 0, 0, 0);
        }
        if (a.dX) {
#pragma unroll
            for (int G = 0; G < kMfRowSteps / 4; ++G) {
                // all tiles' products first (independent accumulators), then the packing
                f32x4 o[CPL];
#pragma unroll
                for (int t = 0; t < CPL; ++t)
                    o[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[t][0], gb[G][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                for (int h = 1; h < KH; ++h)
#pragma unroll
                    for (int t = 0; t < CPL; ++t) o[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[t][h], gb[G][h], o[t], 0, 0, 0);
                uint32_t pk[2 * CPL];
#pragma unroll
                for (int t = 0; t < CPL; ++t) {
                    pk[2 * t] = pack_bf16x2(o[t][0], o[t][1]);
                    pk[2 * t + 1] = pack_bf16x2(o[t][2], o[t][3]);
                }
                // row n of the tile, columns 4*CPL*r .. +4*CPL
#pragma unroll
                for (int w = 0; w < CPL / 2; ++w)
                    *reinterpret_cast<uint4*>(stage + n * kPitch + 8 * CPL * r + 16 * w) =
                        make_uint4(pk[4 * w], pk[4 * w + 1], pk[4 * w + 2], pk[4 * w + 3]);
                wave_lds_sync();
#pragma unroll
                for (int sidx = 0; sidx < 4; ++sidx) {
                    const long row = s0 + (4 * G + sidx) * step + r;
                    const unsigned char* src = stage + (4 * sidx + r) * kPitch + 2 * CPL * n;
                    if (col_ok && row < t1) {
                        // nontemporal: dX is not read again here, and written-back
                        // lines would otherwise stall the next kernel's reads
                        if constexpr (CPL == 8) {
                            const u32x4 v = *reinterpret_cast<const u32x4*>(src);
                            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(a.dX + row * d + col0));
                        } else {
                            const u32x2 v = *reinterpret_cast<const u32x2*>(src);
                            __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(a.dX + row * d + col0));
                        }
                    }
                }
                wave_lds_sync();
            }
        }
    }

    if (!a.dWg_part) return;
    // tile q, element i of lane l: column CPL*(l%16) + q of the block, expert
    // 4*(l/16) + i; waves combined in order through LDS
    __shared__ float wred[kTileM][16];
    for (int w = 0; w < kMfWaves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int q = 0; q < CPL; ++q)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float& slot = wred[CPL * n + q][4 * r + i];
                    slot = (w == 0) ? acc[q][i] : slot + acc[q][i];
                }
        }
        __syncthreads();
    }
    float* part = a.dWg_part + long(blockIdx.y) * d * E;
    for (int i = threadIdx.x; i < kTileM * E; i += kMfWaves * 64) {
        const int cc = i / E, e = i - (i / E) * E;
        const int col = blockIdx.x * kTileM + cc;
        if (col < d) part[long(col) * E + e] = wred[cc][e];
    }
}

// ---- E <= 8: both products on bf16 matrix cores.
//
// v_mfma_f32_16x16x32_bf16: lane l gives A[l%16][8(l/16) .. +8) and
// B[8(l/16) .. +8)[l%16] and receives D[4(l/16) + i][l%16] in element i.
// dlogits is fp32; each value v is split into three bf16 parts,
// v = hi + mid + lo (hi: v rounded to bf16; mid: the remainder rounded; lo:
// what is left, which a bf16 significand holds exactly), so each product of
// a part with a bf16 operand is exact and both results are fp32 sums of the
// exact products, as with fp32 operands.
//   dX, per 16 rows and 16-column tile t: K = 32 holds (part, expert) pairs,
//   8 per part (24 used).  A = Wg[col(t, m)][e] (the same for every part),
//   B = part p of dlogits[row n][e]; with col(t, m) = 32(m/4) + 4t + m%4 lane
//   l receives 32 consecutive columns of row l%16, staged through LDS so that
//   each store writes whole runs of a row.
//   dWg, per 32 rows of the wave and 16-column tile c: K = the rows.  A =
//   X[row k][column m] from an LDS copy of the wave's X tile (row pitch 260
//   bytes: the 64 lanes' 8-row column reads fall in distinct banks); B =
//   parts of dlogits[row k][n%8] in the 16 columns n, hi for n < 8 and mid
//   for n >= 8, then lo for n < 8 into the same accumulator; columns n and
//   n + 8 are added at the end.
constexpr int kB8Waves = 4;
constexpr int kB8Cols = 128;               // columns per block
constexpr int kB8Steps = 8;                // 4-row steps per wave iteration (32 rows)
constexpr int kXPitch = kB8Cols * 2 + 4;   // bytes per staged X row
constexpr int kDPitch = kB8Cols * 2 + 16;  // bytes per staged dX row
constexpr int kB8Stage = 32 * kXPitch;     // the dX stage (16 rows) reuses the X tile's space
static_assert(16 * kDPitch <= kB8Stage, "dX stage fits the X tile's space");
constexpr int kDlPitch = 9;                // floats per staged dlogits row (distinct banks)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Exact three-way split of two values into bf16 pairs (element 0 = a).  A
// non-finite value keeps itself as hi and zero parts below.
__device__ __forceinline__ void split3(float a, float b, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    const uint32_t h = pack_bf16x2(a, b);
    const float ra = __builtin_isfinite(a) ? a - __uint_as_float(h << 16) : 0.f;
    const float rb = __builtin_isfinite(b) ? b - __uint_as_float(h & 0xFFFF0000u) : 0.f;
    const uint32_t m = pack_bf16x2(ra, rb);
    hi = h;
    mid = m;
    lo = pack_bf16x2(ra - __uint_as_float(m << 16), rb - __uint_as_float(m & 0xFFFF0000u));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
    return __builtin_bit_cast(bf16x8, make_uint4(w0, w1, w2, w3));
}

__global__ void __launch_bounds__(kB8Waves * 64) __attribute__((amdgpu_waves_per_eu(2)))
gate_backward_bf16_kernel(const GateBackArgs a)
{
    __shared__ __attribute__((aligned(16))) unsigned char lds[kB8Waves * kB8Stage];
    __shared__ float dlt_all[kB8Waves][32 * kDlPitch];
    __shared__ float wred[kB8Cols][8];
    const int E = a.E, d = a.d;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, r = lane >> 4;
    const int cb = blockIdx.x * kB8Cols;  // the block's first column
    const int colx = cb + 8 * n;          // the lane's 8 columns of an X row
    const bool col_ok = colx < d;         // d % 8 == 0: all 8 in or all out
    // Row slices from the last: the forward's gate GEMM read X from the first
    // row to the last, so its last rows are the likeliest still to be in the
    // Infinity Cache, and walking the slices backwards meets them first
    // (gate workload: 66.5 -> 65.5 us a call).  Slice sy keeps its own dWg
    // partial, so the sums do not change.
    const int sy = gridDim.y - 1 - blockIdx.y;
    const long t0 = (long(sy) * a.T) / gridDim.y;
    const long t1 = (long(sy + 1) * a.T) / gridDim.y;
    unsigned char* stage = lds + wave * kB8Stage;
    float* dlt = dlt_all[wave];  // dlogits of the wave's 32 rows: [k][e], pitch kDlPitch

    // dX A operands: Wg[col(t, n)][0..8) for the parts r < 3, zero for r = 3
    bf16x8 wa[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int c = cb + 32 * (n >> 2) + 4 * t + (n & 3);
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (a.dX && r < 3 && c < d) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t lo = (2 * h < E) ? a.Wg[long(c) * E + 2 * h] : 0u;
                const uint32_t hi = (2 * h + 1 < E) ? a.Wg[long(c) * E + 2 * h + 1] : 0u;
                w[h] = lo | (hi << 16);
            }
        }
        wa[t] = as_bf16x8(w[0], w[1], w[2], w[3]);
    }
    f32x4 acc[8];  // dWg: tile c, column 16c + 4r + i, slot n
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // A wave's rows in one iteration: k = 4u + q is row s0 + u*step + q.
    // Loads of the next iteration are in flight while this one computes.
    const long step = 4L * kB8Waves;
    const long S = step * kB8Steps;
    uint4 xv[kB8Steps];
    float dv[4];
    auto load_iter = [&](long sb) {
#pragma unroll
        for (int u = 0; u < kB8Steps; ++u) {
            const long row = sb + u * step + r;
            const long rr = row < t1 ? row : t0;
            xv[u] = col_ok ? *reinterpret_cast<const uint4*>(a.X + rr * d + colx) : make_uint4(0, 0, 0, 0);
        }
        // dlogits (k, e) for idx = lane + 64j: k = idx/8, e = idx%8; rows past
        // the slice and padding experts are zero
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = lane + 64 * j, k = idx >> 3, e = idx & 7;
            const long row = sb + (k >> 2) * step + (k & 3);
            dv[j] = (row < t1 && e < E) ? a.dlogits[row * E + e] : 0.f;
        }
    };
    long s0 = t0 + 4L * wave;
    if (s0 < t1) load_iter(s0);
    for (; s0 < t1; s0 += S) {
        if (a.dWg_part) {
#pragma unroll
            for (int u = 0; u < kB8Steps; ++u) {
                uint32_t* dst = reinterpret_cast<uint32_t*>(stage + (4 * u + r) * kXPitch + 16 * n);
                dst[0] = xv[u].x;
                dst[1] = xv[u].y;
                dst[2] = xv[u].z;
                dst[3] = xv[u].w;
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = lane + 64 * j;
            dlt[(idx >> 3) * kDlPitch + (idx & 7)] = dv[j];
        }
        wave_lds_sync();
        if (s0 + S < t1) load_iter(s0 + S);

        if (a.dWg_part) {
            // B: rows k = 8r + i, expert n%8: hi|mid, then lo
            uint32_t bh[4], bl[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                uint32_t hi, mid, lo;
                split3(dlt[(8 * r + 2 * h) * kDlPitch + (n & 7)], dlt[(8 * r + 2 * h + 1) * kDlPitch + (n & 7)],
                       hi, mid, lo);
                bh[h] = (n < 8) ? hi : mid;
                bl[h] = (n < 8) ? lo : 0u;
            }
            const bf16x8 Bhm = as_bf16x8(bh[0], bh[1], bh[2], bh[3]);
            const bf16x8 Blo = as_bf16x8(bl[0], bl[1], bl[2], bl[3]);
            // A: X[8r + i][16c + n], i < 8; half the tiles' reads at a time,
            // all issued before the first is used
#pragma unroll
            for (int c0 = 0; c0 < 8; c0 += 4) {
                uint16_t xe[4][8];
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        xe[c][i] = *reinterpret_cast<const uint16_t*>(stage + (8 * r + i) * kXPitch +
                                                                      2 * (16 * (c0 + c) + n));
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const bf16x8 A = as_bf16x8(uint32_t(xe[c][0]) | (uint32_t(xe[c][1]) << 16),
                                               uint32_t(xe[c][2]) | (uint32_t(xe[c][3]) << 16),
                                               uint32_t(xe[c][4]) | (uint32_t(xe[c][5]) << 16),
                                               uint32_t(xe[c][6]) | (uint32_t(xe[c][7]) << 16));
                    acc[c0 + c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bhm, acc[c0 + c], 0, 0, 0);
                    acc[c0 + c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Blo, acc[c0 + c], 0, 0, 0);
                }
            }
        }
        wave_lds_sync();  // the dX stage reuses the X tile's space
        if (a.dX) {
#pragma unroll
            for (int G = 0; G < 2; ++G) {
                // B: part r of dlogits[row 16G + n][0..8), zero for r = 3
                const float* g = dlt + (16 * G + n) * kDlPitch;
                uint32_t b[4];
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    uint32_t hi, mid, lo;
                    split3(g[2 * h], g[2 * h + 1], hi, mid, lo);
                    b[h] = (r == 0) ? hi : (r == 1) ? mid : (r == 2) ? lo : 0u;
                }
                const bf16x8 B = as_bf16x8(b[0], b[1], b[2], b[3]);
                f32x4 o[8];
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[t], B, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                uint32_t pk[16];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    pk[2 * t] = pack_bf16x2(o[t][0], o[t][1]);
                    pk[2 * t + 1] = pack_bf16x2(o[t][2], o[t][3]);
                }
                // row n of the group, block columns 32r .. 32r + 32
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    *reinterpret_cast<uint4*>(stage + n * kDPitch + 64 * r + 16 * w) =
                        make_uint4(pk[4 * w], pk[4 * w + 1], pk[4 * w + 2], pk[4 * w + 3]);
                wave_lds_sync();
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const long row = s0 + (4 * G + q) * step + r;
                    if (col_ok && row < t1) {
                        // nontemporal: dX is not read again here, and written-back
                        // lines would otherwise stall the next kernel's reads
                        const u32x4 v = *reinterpret_cast<const u32x4*>(stage + (4 * q + r) * kDPitch + 16 * n);
                        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(a.dX + row * d + colx));
                    }
                }
                wave_lds_sync();
            }
        }
    }

    if (!a.dWg_part) return;
    // slots n and n + 8 hold parts of the same expert; then the waves in
    // order through LDS
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[c][i] += __shfl_xor(acc[c][i], 8);
    for (int w = 0; w < kB8Waves; ++w) {
        if (wave == w && n < 8) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float& slot = wred[16 * c + 4 * r + i][n];
                    slot = (w == 0) ? acc[c][i] : slot + acc[c][i];
                }
        }
        __syncthreads();
    }
    float* part = a.dWg_part + long(sy) * d * E;
    for (int i = threadIdx.x; i < kB8Cols * E; i += kB8Waves * 64) {
        const int cc = i / E, e = i - (i / E) * E;
        const int col = cb + cc;
        if (col < d) part[long(col) * E + e] = wred[cc][e];
    }
}

// dWg[i] = sum over the token slices of part[slice][i], slices in order
// (eight loads in flight at a time, the additions still in slice order).
__global__ void __launch_bounds__(256)
gate_backward_reduce_kernel(const float* __restrict__ part, float* __restrict__ dWg, long n, int slices)
{
    for (long i = long(blockIdx.x) * 256 + threadIdx.x; i < n; i += long(gridDim.x) * 256) {
        float s = 0.f;
        int sl = 0;
        for (; sl + 8 <= slices; sl += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = part[long(sl + u) * n + i];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += v[u];
        }
        for (; sl < slices; ++sl) s += part[long(sl) * n + i];
        dWg[i] = s;
    }
}

}  // namespace

// Columns per block of the kernel that serves E.
static int gate_backward_tile(int E) { return E <= 8 ? 128 : kTile; }

// Token slices: enough blocks for two per compute unit, at least 64 rows each.
int gate_backward_slices(int T, int d, int E) {
    const int tile = gate_backward_tile(E);
    const long tiles = (d + tile - 1) / tile;
    long sl = (2L * kAssumedCUs + tiles - 1) / tiles;
    const long max_sl = (T + 63) / 64;
    if (sl > max_sl) sl = max_sl;
    if (sl < 1) sl = 1;
    return int(sl);
}

size_t gate_backward_workspace_bytes(int T, int d, int E) {
    return align_up(size_t(gate_backward_slices(T, d, E)) * d * E * 4, 256);
}

hipError_t launch_gate_backward(const GateBackArgs& a, hipStream_t st) {
    const int slices = gate_backward_slices(a.T, a.d, a.E);
    const int tile = gate_backward_tile(a.E);
    const dim3 grid((a.d + tile - 1) / tile, slices);
    GateBackArgs b = a;
    if (!a.dWg) b.dWg_part = nullptr;
    if (a.E <= 8) hipLaunchKernelGGL(gate_backward_bf16_kernel, grid, dim3(kB8Waves * 64), 0, st, b);
    else if (a.E <= 16) hipLaunchKernelGGL((gate_backward_mfma_kernel<16, 4>), grid, dim3(kMfWaves * 64), 0, st, b);
    else if (a.E <= 32) hipLaunchKernelGGL(gate_backward_kernel<2>, grid, dim3(kGbThreads), 0, st, b);
    else if (a.E <= 64) hipLaunchKernelGGL(gate_backward_kernel<1>, grid, dim3(kGbThreads), 0, st, b);
    else return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.dWg) return e;
    const long n = long(a.d) * a.E;
    const int blocks = int(std::min<long>((n + 255) / 256, 1024));
    hipLaunchKernelGGL(gate_backward_reduce_kernel, dim3(blocks), dim3(256), 0, st, b.dWg_part, a.dWg, n,
                       slices);
    return hipGetLastError();
}

}  // namespace moe
