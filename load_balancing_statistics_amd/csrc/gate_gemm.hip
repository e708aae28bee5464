// gate_gemm.hip -- router logits = X[T,d] . Wg[d,E] on gfx950 matrix cores.
//
// The gate (router) network of page codechina.net article 413310 section 1.2
// scores every token against every expert; with a linear gate that is one
// bf16 GEMM with fp32 accumulation.  E is small (8 for the gate workload), so
// the product is bound by streaming X from HBM (about 8 flop per byte), not
// by the matrix cores.
//
// MFMA v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 k, B = 32 k x 16 experts.
// Lane l holds A[l%16][8*(l/16) .. +8) (16 contiguous bytes of one X row) and
// B[8*(l/16) .. +8)[l%16]; the result D[i][j] sits in lane j + 16*(i/4),
// element i%4.  B wants 8 consecutive k of one expert, which Wg [d,E]
// (expert-minor) does not store contiguously, so a first tiny kernel writes
// Wg transposed, Wt [E,d], into the workspace; the GEMM then reads 16 bytes
// per lane for A (HBM) and for B (L2-resident Wt).
//
// A block computes a 16-token tile; its 4 waves split the k range into four
// contiguous quarters and the partial tiles are summed in a fixed order in
// LDS (deterministic).
#include "route_common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGateWaves = 4;
constexpr int kUnroll = 8;
constexpr int kMaxTilesN = 4;  // E <= 64

__global__ void __launch_bounds__(256)
transpose_wg_kernel(const uint16_t* __restrict__ Wg, uint16_t* __restrict__ Wt, int d, int E)
{
    const long n = long(d) * E;
    for (long i = long(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += long(gridDim.x) * blockDim.x) {
        const long kk = i / E, e = i % E;  // Wg[kk][e]
        Wt[e * d + kk] = Wg[i];
    }
}

__device__ __forceinline__ bf16x8 load8(const uint16_t* p) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 zero8() {
    return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
}

template <int NT>
__global__ void __launch_bounds__(kGateWaves * 64)
gate_gemm_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wt,
                 float* __restrict__ logits, int T, int d, int E)
{
    __shared__ f32x4 red[kGateWaves][NT][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, kq = lane >> 4;
    const long row = long(blockIdx.x) * 16 + r16;
    const bool row_ok = row < T;
    const int nsteps = (d + 31) / 32;
    const int per = (nsteps + kGateWaves - 1) / kGateWaves;
    const int st0 = min(wave * per, nsteps), st1 = min(st0 + per, nsteps);

    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint16_t* xrow = X + row * d;
    for (int s0 = st0; s0 < st1; s0 += kUnroll) {
        bf16x8 av[kUnroll];
        bf16x8 bv[kUnroll][NT];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int kk = (s0 + u) * 32 + kq * 8;
            const bool kin = (s0 + u < st1) && (kk < d);
            av[u] = (row_ok && kin) ? load8(xrow + kk) : zero8();
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int e = t * 16 + r16;
                bv[u][t] = (kin && e < E) ? load8(Wt + long(e) * d + kk) : zero8();
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bv[u][t], acc[t], 0, 0, 0);
    }

#pragma unroll
    for (int t = 0; t < NT; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            f32x4 sum = red[0][t][lane];
#pragma unroll
            for (int w = 1; w < kGateWaves; ++w) sum += red[w][t][lane];
            const int col = t * 16 + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const long r = long(blockIdx.x) * 16 + kq * 4 + i;
                if (r < T && col < E) logits[r * E + col] = sum[i];
            }
        }
    }
}

}  // namespace

bool gate_supported(int T, int d, int E) {
    return T >= 1 && d >= 8 && d % 8 == 0 && E >= 1 && E <= 16 * kMaxTilesN;
}

size_t gate_workspace_bytes(int d, int E) { return align_up(size_t(d) * E * 2, 256); }

hipError_t launch_gate_gemm(const GateArgs& a, uint16_t* wt, hipStream_t st) {
    const long n = long(a.d) * a.E;
    const int tb = int(std::min<long>((n + 255) / 256, 1024));
    hipLaunchKernelGGL(transpose_wg_kernel, dim3(tb), dim3(256), 0, st, a.Wg, wt, a.d, a.E);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((a.T + 15) / 16);
    const int nt = (a.E + 15) / 16;
    switch (nt) {
        case 1: hipLaunchKernelGGL(gate_gemm_kernel<1>, grid, dim3(256), 0, st, a.X, wt, a.logits, a.T, a.d, a.E); break;
        case 2: hipLaunchKernelGGL(gate_gemm_kernel<2>, grid, dim3(256), 0, st, a.X, wt, a.logits, a.T, a.d, a.E); break;
        case 3: hipLaunchKernelGGL(gate_gemm_kernel<3>, grid, dim3(256), 0, st, a.X, wt, a.logits, a.T, a.d, a.E); break;
        case 4: hipLaunchKernelGGL(gate_gemm_kernel<4>, grid, dim3(256), 0, st, a.X, wt, a.logits, a.T, a.d, a.E); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace moe
