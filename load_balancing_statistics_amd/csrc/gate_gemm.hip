// gate_gemm.hip -- router logits = X[T,d] . Wg[d,E] on gfx950 matrix cores.
//
// The gate (router) network of page codechina.net article 413310 section 1.2
// scores every token against every expert; with a linear gate that is one
// bf16 GEMM with fp32 accumulation.  E is small (8 for the gate workload), so
// the product is bound by streaming X from HBM (about 8 flop per byte), not
// by the matrix cores.
//
// MFMA v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 k, B = 32 k x 16 experts.
// Lane l holds A[l%16][8*(l/16) .. +8) and B[8*(l/16) .. +8)[l%16]; the
// result D[i][j] sits in lane j + 16*(i/4), element i%4.
//
// Operand A is 16 bytes of one X row per lane, 16 different rows across
// consecutive lanes: loaded like that, every quad of lanes touches four cache
// lines and the address unit, not HBM, limits the kernel.  So a wave loads
// its tile of X coalesced (16 lanes cover 256 contiguous bytes of a row),
// stores it in LDS (row pitch 272 bytes: the 16 rows an MFMA operand read
// touches fall in distinct banks) and reads the operands back from there.
// Operand B: when E % 8 == 0 each wave loads its chunk's slice of Wg (a
// contiguous run) beside X and writes it transposed into LDS, from where the
// operands are 16-byte reads; otherwise a tiny kernel lays B out once per
// call, Wb[step][tile][lane] (16 bytes each, zero past d and E), so that its
// loads are contiguous per wave.
//
// A block computes 32 tokens (two 16-token tiles); its 4 waves split the k
// range into four contiguous quarters, staging 128 k (256 bytes per row) at a
// time, and the partial tiles are summed in a fixed order in LDS
// (deterministic).
#include "route_common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGateWaves = 4;
constexpr int kMaxTilesN = 4;              // E <= 64
constexpr int kMT = 2;                     // 16-token tiles per block
constexpr int kRows = 16 * kMT;            // tokens per block
constexpr int kChunkK = 128;               // k staged at a time
constexpr int kSteps = kChunkK / 32;       // MFMA steps per chunk
constexpr int kRowPitch = kChunkK * 2 + 16;
constexpr int kLanesPerRow = kChunkK / 8;  // 16 bytes per lane
constexpr int kRowsPerLoad = 64 / kLanesPerRow;
constexpr int kLoads = kRows / kRowsPerLoad;

// Wb[(s*NT + t)*64 + l] = bf16 Wg[32s + 8(l/16) + j][16t + l%16], j = 0..7
__global__ void __launch_bounds__(256)
swizzle_wg_kernel(const uint16_t* __restrict__ Wg, uint4* __restrict__ Wb, int d, int E, int NT, long n)
{
    for (long i = long(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += long(gridDim.x) * blockDim.x) {
        const int l = int(i % 64);
        const long st = i / 64;
        const int t = int(st % NT);
        const long s = st / NT;
        const int e = t * 16 + (l & 15);
        const long k0 = 32 * s + 8 * (l >> 4);
        uint32_t w[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const long ka = k0 + 2 * h, kb = ka + 1;
            const uint32_t lo = (e < E && ka < d) ? Wg[ka * E + e] : 0u;
            const uint32_t hi = (e < E && kb < d) ? Wg[kb * E + e] : 0u;
            w[h] = lo | (hi << 16);
        }
        Wb[i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// LDS writes by some lanes, then reads of them by others, within one wave
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// RAW (E % 8 == 0): a wave reads its chunk's slice of Wg itself -- rows
// 128c .. 128c + 127 of [d, E], one contiguous run of 128E values -- with
// 16-byte loads issued beside its X loads, and writes it transposed into LDS
// (expert rows, pitch kRowPitch, the padding experts zero), from which it
// reads the B operands as 16-byte runs of 8 k.  Otherwise the B operands
// come pre-laid-out from Wb (swizzle_wg_kernel).
template <int NT, bool RAW>
__global__ void __launch_bounds__(kGateWaves * 64)
gate_gemm_kernel(const uint16_t* __restrict__ X, const uint4* __restrict__ Wb, const uint16_t* __restrict__ Wg,
                 float* __restrict__ logits, int T, int d, int E)
{
    constexpr int kStage = kRows * kRowPitch;
    constexpr int kWbT = RAW ? 16 * NT * kRowPitch : 0;
    constexpr int kWave = kStage + kWbT;
    constexpr int kRed = kGateWaves * kMT * NT * 64 * 16;
    constexpr int kLds = kGateWaves * kWave > kRed ? kGateWaves * kWave : kRed;
    constexpr int kPieces = 4 * NT;  // 16-byte pieces of the Wg slice a lane loads (E/4 used)
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, kq = lane >> 4;
    const long row0 = long(blockIdx.x) * kRows;
    const int nchunks = (d + kChunkK - 1) / kChunkK;
    const int per = (nchunks + kGateWaves - 1) / kGateWaves;
    const int c0 = min(wave * per, nchunks), c1 = min(c0 + per, nchunks);
    unsigned char* stage = lds + wave * kWave;
    unsigned char* wbt = stage + kStage;

    f32x4 acc[kMT][NT];
#pragma unroll
    for (int m = 0; m < kMT; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    if constexpr (RAW) {
        // the padding experts' rows stay zero
        for (int e = E; e < 16 * NT; ++e)
            for (int q = lane; q < kChunkK / 2; q += 64)
                reinterpret_cast<uint32_t*>(wbt + e * kRowPitch)[q] = 0u;
    }

    // coalesced loads: load j covers rows kRowsPerLoad*j + lr, lane's 8 k at lc
    const int lr = lane / kLanesPerRow, lc = (lane % kLanesPerRow) * 8;
    uint4 xr[kLoads];
    uint4 wr[kPieces];
    auto load_chunk = [&](int c) {
        const int k = c * kChunkK + lc;  // d % 8 == 0: the lane's 8 k are all in or all out
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const long row = row0 + kRowsPerLoad * j + lr;
            xr[j] = (row < T && k < d) ? *reinterpret_cast<const uint4*>(X + row * d + k)
                                       : make_uint4(0, 0, 0, 0);
        }
        if constexpr (RAW) {
            // lane covers values [2E*lane, 2E*lane + 2E) of the slice: E/4 pieces
            // of 8 values, each 8 experts of one k row (E % 8 == 0)
#pragma unroll
            for (int j = 0; j < kPieces; ++j) {
                const int i = 2 * E * lane + 8 * j;  // value index within the slice
                const int kk = c * kChunkK + i / E;
                wr[j] = (4 * j < E && kk < d) ? *reinterpret_cast<const uint4*>(Wg + long(c) * kChunkK * E + i)
                                              : make_uint4(0, 0, 0, 0);
            }
        }
    };
    if (c0 < c1) load_chunk(c0);
    for (int c = c0; c < c1; ++c) {
        uint4 bv[kSteps][NT];
        if constexpr (!RAW) {
#pragma unroll
            for (int s = 0; s < kSteps; ++s)
#pragma unroll
                for (int t = 0; t < NT; ++t) bv[s][t] = Wb[(long(c * kSteps + s) * NT + t) * 64 + lane];
        }
#pragma unroll
        for (int j = 0; j < kLoads; ++j)
            *reinterpret_cast<uint4*>(stage + (kRowsPerLoad * j + lr) * kRowPitch + (lane % kLanesPerRow) * 16) = xr[j];
        if constexpr (RAW) {
            // transpose: value (k, e) to row e, column k
#pragma unroll
            for (int j = 0; j < kPieces; ++j) {
                if (4 * j < E) {
                    const int i = 2 * E * lane + 8 * j;
                    const int kr = i / E, e0 = i - kr * E;
                    uint16_t* col = reinterpret_cast<uint16_t*>(wbt + e0 * kRowPitch) + kr;
                    const uint32_t w4[4] = {wr[j].x, wr[j].y, wr[j].z, wr[j].w};
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        col[(2 * h) * (kRowPitch / 2)] = uint16_t(w4[h]);
                        col[(2 * h + 1) * (kRowPitch / 2)] = uint16_t(w4[h] >> 16);
                    }
                }
            }
        }
        wave_lds_sync();
        if (c + 1 < c1) load_chunk(c + 1);  // in flight while this chunk is multiplied
        if constexpr (RAW) {
#pragma unroll
            for (int s = 0; s < kSteps; ++s)
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    bv[s][t] = *reinterpret_cast<const uint4*>(wbt + (16 * t + r16) * kRowPitch + 64 * s + 16 * kq);
        }
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
#pragma unroll
            for (int m = 0; m < kMT; ++m) {
                const uint4 av = *reinterpret_cast<const uint4*>(stage + (m * 16 + r16) * kRowPitch + s * 64 + kq * 16);
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                                       __builtin_bit_cast(bf16x8, bv[s][t]),
                                                                       acc[m][t], 0, 0, 0);
            }
        wave_lds_sync();  // the next chunk overwrites the stage
    }

    __syncthreads();
    f32x4* red = reinterpret_cast<f32x4*>(lds);
#pragma unroll
    for (int m = 0; m < kMT; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) red[((wave * kMT + m) * NT + t) * 64 + lane] = acc[m][t];
    __syncthreads();
    for (int q = wave; q < kMT * NT; q += kGateWaves) {
        const int m = q / NT, t = q % NT;
        f32x4 sum = red[(m * NT + t) * 64 + lane];
#pragma unroll
        for (int w = 1; w < kGateWaves; ++w) sum += red[((w * kMT + m) * NT + t) * 64 + lane];
        const int col = t * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const long r = row0 + m * 16 + kq * 4 + i;
            if (r < T && col < E) logits[r * E + col] = sum[i];
        }
    }
}

int gate_tiles_n(int E) { return (E + 15) / 16; }

// 16-byte units of the laid-out B operand: every MFMA step of every chunk
long gate_wb_units(int d, int E) {
    const long nchunks = (d + kChunkK - 1) / kChunkK;
    return nchunks * kSteps * gate_tiles_n(E) * 64;
}

}  // namespace

bool gate_supported(int T, int d, int E) {
    return T >= 1 && d >= 8 && d % 8 == 0 && E >= 1 && E <= 16 * kMaxTilesN;
}

size_t gate_workspace_bytes(int d, int E) { return align_up(size_t(gate_wb_units(d, E)) * 16, 256); }

hipError_t launch_gate_gemm(const GateArgs& a, uint16_t* wt, hipStream_t st) {
    const int nt = gate_tiles_n(a.E);
    const dim3 grid((a.T + kRows - 1) / kRows);
    uint4* wb = reinterpret_cast<uint4*>(wt);
    const bool raw = a.E % 8 == 0;
    if (!raw) {
        const long n = gate_wb_units(a.d, a.E);
        const int tb = int(std::min<long>((n + 255) / 256, 1024));
        hipLaunchKernelGGL(swizzle_wg_kernel, dim3(tb), dim3(256), 0, st, a.Wg, wb, a.d, a.E, nt, n);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
#define MOE_GEMM(NTV)                                                                                  \
    if (raw) hipLaunchKernelGGL((gate_gemm_kernel<NTV, true>), grid, dim3(256), 0, st, a.X, wb, a.Wg, a.logits, a.T, a.d, a.E); \
    else hipLaunchKernelGGL((gate_gemm_kernel<NTV, false>), grid, dim3(256), 0, st, a.X, wb, a.Wg, a.logits, a.T, a.d, a.E);
    switch (nt) {
        case 1: MOE_GEMM(1) break;
        case 2: MOE_GEMM(2) break;
        case 3: MOE_GEMM(3) break;
        case 4: MOE_GEMM(4) break;
        default: return hipErrorInvalidValue;
    }
#undef MOE_GEMM
    return hipGetLastError();
}

}  // namespace moe
