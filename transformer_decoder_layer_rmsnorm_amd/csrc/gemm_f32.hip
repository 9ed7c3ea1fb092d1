// fp32 projections, C[M, N] = A[M, K] * B[N, K]^T with the layer's epilogues, any shape.
//
// The fp32 storage configuration (a small model checked at 1e-4) has no fp32 matrix-core
// budget worth tiling for: plain FMA with a 64x64 LDS tile per 256-thread workgroup, 4x4
// outputs per thread, bounds-checked in M, N and K.  Same epilogues as the bf16 path
// (see kernels.hpp); the residual stream x1 is fp32 here as everywhere.
#include "common.hpp"
#include "kernels.hpp"

namespace q3 {

namespace {

constexpr int T64 = 64, TK = 16;

struct DevGemmF32 {
    const float* a;
    const float* b[3];
    int seg_start[3];
    float* out;
    const float* resid;
    int M, N, K;
};

__device__ __forceinline__ const float* seg_row_f32(const DevGemmF32& p, int n) {
    if (n >= p.seg_start[2]) return p.b[2] + (int64_t)(n - p.seg_start[2]) * p.K;
    if (n >= p.seg_start[1]) return p.b[1] + (int64_t)(n - p.seg_start[1]) * p.K;
    return p.b[0] + (int64_t)n * p.K;
}

template <Epilogue EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(DevGemmF32 p) {
    constexpr bool DUAL = (EPI == Epilogue::SwiGLU);
    constexpr int NB = DUAL ? 2 : 1;
    __shared__ float sA[TK][T64 + 1];
    __shared__ float sB[NB][TK][T64 + 1];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.y * T64, n0 = blockIdx.x * T64;
    float acc[NB][4][4] = {};
    for (int k0 = 0; k0 < p.K; k0 += TK) {
        for (int e = tid; e < T64 * TK; e += 256) {
            const int r = e / TK, kk = e % TK;
            const int m = m0 + r, n = n0 + r, k = k0 + kk;
            sA[kk][r] = (m < p.M && k < p.K) ? p.a[(int64_t)m * p.K + k] : 0.f;
            if constexpr (DUAL) {
                sB[0][kk][r] = (n < p.N && k < p.K) ? p.b[0][(int64_t)n * p.K + k] : 0.f;
                sB[NB - 1][kk][r] = (n < p.N && k < p.K) ? p.b[1][(int64_t)n * p.K + k] : 0.f;
            } else {
                sB[0][kk][r] = (n < p.N && k < p.K) ? seg_row_f32(p, n)[k] : 0.f;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            float av[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) av[i] = sA[kk][ty * 4 + i];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float bv = sB[nb][kk][tx * 4 + j];
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[nb][i][j] = fmaf(av[i], bv, acc[nb][i][j]);
                }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty * 4 + i;
        if (m >= p.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= p.N) continue;
            const int64_t o = (int64_t)m * p.N + n;
            if constexpr (EPI == Epilogue::Store) p.out[o] = acc[0][i][j];
            else if constexpr (EPI == Epilogue::SwiGLU) p.out[o] = silu_mul(acc[0][i][j], acc[NB - 1][i][j]);
            else p.out[o] = p.resid[o] + acc[0][i][j];   // both residual forms are fp32 here
        }
    }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s) {
    if (g.M <= 0) return hipSuccess;
    DevGemmF32 p{};
    p.a = static_cast<const float*>(g.a);
    int start = 0;
    for (int i = 0; i < 3; ++i) {
        const int src = i < g.nseg ? i : g.nseg - 1;
        p.b[i] = static_cast<const float*>(g.b[src]);
        p.seg_start[i] = i < g.nseg ? start : 0x7fffffff;
        if (i < g.nseg) start += g.b_rows[i];
    }
    p.out = static_cast<float*>(g.out);
    p.resid = static_cast<const float*>(g.resid);
    p.M = g.M;
    p.N = g.N;
    p.K = g.K;
    const dim3 grid((unsigned)((g.N + T64 - 1) / T64), (unsigned)((g.M + T64 - 1) / T64));
    switch (g.epi) {
        case Epilogue::Store: gemm_f32_kernel<Epilogue::Store><<<grid, 256, 0, s>>>(p); break;
        case Epilogue::ResidToF32: gemm_f32_kernel<Epilogue::ResidToF32><<<grid, 256, 0, s>>>(p); break;
        case Epilogue::SwiGLU: gemm_f32_kernel<Epilogue::SwiGLU><<<grid, 256, 0, s>>>(p); break;
        case Epilogue::ResidF32In: gemm_f32_kernel<Epilogue::ResidF32In><<<grid, 256, 0, s>>>(p); break;
    }
    return hipGetLastError();
}

}  // namespace q3
