// bf16 projections of the layer on gfx950 matrix cores: C[M, N] = A[M, K] * B[N, K]^T, fp32
// accumulation, with the layer's element-wise work fused into the epilogue.
//
// The projections are the nn.Linear layers of "17. A modern architecture: Qwen3" (sections
// Attention with grouped KV heads and Q/K normalization, SwiGLU): q/k/v/o and gate/up/down,
// weights [out, in], no bias.  Both operands are therefore K-contiguous, which is exactly the
// per-lane operand layout of v_mfma_f32_32x32x16_bf16 (each lane feeds 8 consecutive k).
//
// Large-M kernel: 128x128 output tile per 256-thread workgroup, 4 waves in a 2x2 grid each
// owning a 64x64 sub-tile (2x2 MFMA 32x32 blocks), BK = 64, two LDS stages; the next k-slab is
// fetched into registers while the current one feeds the MFMAs.  LDS rows are 128 bytes; the
// 16-byte chunk index is XOR-swizzled with the row so that the 8 lanes served per LDS cycle hit
// distinct banks both when storing and when reading operand fragments.
// Tiles are remapped so that each XCD works on a contiguous band of tiles, grouped 8 M-tiles
// at a time for L2 reuse of the weight tiles.
//
// Skinny kernel (decode, M <= 64): v_mfma_f32_16x16x32_bf16 with the weight rows streamed
// straight from HBM into B fragments; each workgroup owns 16 output columns and splits K
// across its waves, reducing through LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace q3 {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kGroupM = 8;

struct DevGemm {
    const bf16* a;
    const bf16* b[3];
    int seg_start[3];     // first N row of each segment
    void* out;
    const void* resid;
    int M, N, K;
    int tiles_m, tiles_n;
};

__device__ __forceinline__ const bf16* seg_row(const DevGemm& p, int n) {
    // the segment holding B row n (segments are stacked along N)
    if (n >= p.seg_start[2]) return p.b[2] + (int64_t)(n - p.seg_start[2]) * p.K;
    if (n >= p.seg_start[1]) return p.b[1] + (int64_t)(n - p.seg_start[1]) * p.K;
    return p.b[0] + (int64_t)n * p.K;
}

template <Epilogue EPI>
__device__ __forceinline__ void epilogue_store(const DevGemm& p, int row, int col, float v) {
    if constexpr (EPI == Epilogue::Store) {
        static_cast<bf16*>(p.out)[(int64_t)row * p.N + col] = (bf16)v;
    } else if constexpr (EPI == Epilogue::ResidToF32) {
        const float r = (float)static_cast<const bf16*>(p.resid)[(int64_t)row * p.N + col];
        static_cast<float*>(p.out)[(int64_t)row * p.N + col] = r + v;
    } else if constexpr (EPI == Epilogue::ResidF32In) {
        const float r = static_cast<const float*>(p.resid)[(int64_t)row * p.N + col];
        static_cast<bf16*>(p.out)[(int64_t)row * p.N + col] = (bf16)(r + v);
    }
}

__device__ __forceinline__ int swz(int row, int chunk) { return ((chunk ^ (row & 7)) << 3); }

template <Epilogue EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(DevGemm p) {
    constexpr bool DUAL = (EPI == Epilogue::SwiGLU);
    __shared__ __attribute__((aligned(16))) bf16 sA[2][BM * BK];
    __shared__ __attribute__((aligned(16))) bf16 sB[2][BN * BK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- tile index: contiguous band per XCD, then grouped along M
    const int total = p.tiles_m * p.tiles_n;
    int t = blockIdx.x;
    if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
    const int per_group = kGroupM * p.tiles_n;
    const int group = t / per_group;
    const int first_m = group * kGroupM;
    const int gsize = min(p.tiles_m - first_m, kGroupM);
    const int tm = first_m + (t % per_group) % gsize;
    const int tn = (t % per_group) / gsize;
    const int m0 = tm * BM;

    // ---- global -> register loaders: each thread moves 4 16-byte chunks of A and of B per slab
    const bf16* ga[4];
    const bf16* gb[4];
    int la[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = tid + 256 * j;
        const int row = c >> 3, ch = c & 7;
        la[j] = row * BK + swz(row, ch);
        ga[j] = p.a + (int64_t)min(m0 + row, p.M - 1) * p.K + ch * 8;
        if constexpr (DUAL) {
            // tile rows in blocks of 32: gate, up, gate, up for output columns tn*64 + [0,32), [32,64)
            const int n = tn * 64 + (j >> 1) * 32 + (row & 31);
            gb[j] = p.b[j & 1] + (int64_t)n * p.K + ch * 8;
        } else {
            gb[j] = seg_row(p, tn * BN + row) + ch * 8;
        }
    }

    bf16x8 ra[4], rb[4];
    auto gload = [&](int kt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ra[j] = *reinterpret_cast<const bf16x8*>(ga[j] + kt * BK);
            rb[j] = *reinterpret_cast<const bf16x8*>(gb[j] + kt * BK);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<bf16x8*>(&sA[buf][la[j]]) = ra[j];
            *reinterpret_cast<bf16x8*>(&sB[buf][la[j]]) = rb[j];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = p.K / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int ch = 2 * kk + (lane >> 5);
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = wm * 64 + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const bf16x8*>(&sA[buf][r * BK + swz(r, ch)]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = wn * 64 + j * 32 + (lane & 31);
                bfr[j] = *reinterpret_cast<const bf16x8*>(&sB[buf][r * BK + swz(r, ch)]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue.  32x32 accumulator layout: lane l, register r holds
    //      row 8*(r/4) + 4*(l/32) + r%4, column l%32 of its block.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row >= p.M) continue;
            if constexpr (DUAL) {
                const int col = tn * 64 + wn * 32 + (lane & 31);
                static_cast<bf16*>(p.out)[(int64_t)row * p.N + col] = (bf16)silu_mul(acc[i][0][r], acc[i][1][r]);
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = tn * BN + wn * 64 + j * 32 + (lane & 31);
                    epilogue_store<EPI>(p, row, col, acc[i][j][r]);
                }
            }
        }
    }
}

// ------------------------------------------------------------------ skinny (M <= 64)
template <Epilogue EPI, int MG, int NW>
__global__ __launch_bounds__(NW * 64) void gemv_bf16_kernel(DevGemm p) {
    constexpr bool DUAL = (EPI == Epilogue::SwiGLU);
    constexpr int NB = DUAL ? 2 : 1;
    __shared__ float red[NB][NW][MG][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 16;
    const int kper = p.K / NW;
    const int k0 = wave * kper + 8 * (lane >> 4);

    const bf16* brow[NB];
    if constexpr (DUAL) {
        brow[0] = p.b[0] + (int64_t)(n0 + (lane & 15)) * p.K;
        brow[NB - 1] = p.b[1] + (int64_t)(n0 + (lane & 15)) * p.K;
    } else {
        brow[0] = seg_row(p, n0 + (lane & 15));
    }
    const bf16* arow[MG];
    bool avalid[MG];
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
        const int r = mg * 16 + (lane & 15);
        avalid[mg] = r < p.M;
        arow[mg] = p.a + (int64_t)min(r, p.M - 1) * p.K;
    }

    f32x4 acc[NB][MG];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) acc[nb][mg] = f32x4{0.f, 0.f, 0.f, 0.f};

    const bf16x8 zero = {};
#pragma unroll 4
    for (int k = k0; k < wave * kper + kper; k += 32) {
        bf16x8 bv[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bv[nb] = *reinterpret_cast<const bf16x8*>(brow[nb] + k);
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) {
            bf16x8 av = *reinterpret_cast<const bf16x8*>(arow[mg] + k);
            if (!avalid[mg]) av = zero;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc[nb][mg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[nb], acc[nb][mg], 0, 0, 0);
        }
    }
    // 16x16 accumulator layout: lane l, register i holds row 4*(l/16) + i, column l%16.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mg = 0; mg < MG; ++mg)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[nb][wave][mg][(4 * (lane >> 4) + i) * 16 + (lane & 15)] = acc[nb][mg][i];
    __syncthreads();
    for (int idx = threadIdx.x; idx < MG * 256; idx += NW * 64) {
        const int mg = idx >> 8, e = idx & 255;
        const int row = mg * 16 + (e >> 4);
        const int col = n0 + (e & 15);
        if (row >= p.M) continue;
        float s[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            s[nb] = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) s[nb] += red[nb][w][mg][e];
        }
        if constexpr (DUAL) {
            static_cast<bf16*>(p.out)[(int64_t)row * p.N + col] = (bf16)silu_mul(s[0], s[NB - 1]);
        } else {
            epilogue_store<EPI>(p, row, col, s[0]);
        }
    }
}

DevGemm make_dev(const GemmArgs& g) {
    DevGemm p{};
    p.a = static_cast<const bf16*>(g.a);
    int start = 0;
    for (int s = 0; s < 3; ++s) {
        const int src = s < g.nseg ? s : g.nseg - 1;
        p.b[s] = static_cast<const bf16*>(g.b[src]);
        p.seg_start[s] = s < g.nseg ? start : 0x7fffffff;
        if (s < g.nseg) start += g.b_rows[s];
    }
    p.out = g.out;
    p.resid = g.resid;
    p.M = g.M;
    p.N = g.N;
    p.K = g.K;
    return p;
}

template <Epilogue EPI, int MG>
hipError_t launch_gemv_mg(const DevGemm& p, hipStream_t s) {
    const unsigned grid = (unsigned)(p.N / 16);
    if (p.K % (32 * 8) == 0)
        gemv_bf16_kernel<EPI, MG, 8><<<grid, 512, 0, s>>>(p);
    else if (p.K % (32 * 4) == 0)
        gemv_bf16_kernel<EPI, MG, 4><<<grid, 256, 0, s>>>(p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <Epilogue EPI>
hipError_t launch_gemv_epi(const DevGemm& p, hipStream_t s) {
    if (p.M <= 16) return launch_gemv_mg<EPI, 1>(p, s);
    if (p.M <= 32) return launch_gemv_mg<EPI, 2>(p, s);
    if (p.M <= 64) return launch_gemv_mg<EPI, 4>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace

bool gemm_bf16_supported(int n_rows, int K) { return n_rows % 128 == 0 && K % 128 == 0; }

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s) {
    if (g.M <= 0) return hipSuccess;
    DevGemm p = make_dev(g);
    if (p.K % BK) return hipErrorInvalidValue;
    p.tiles_m = (p.M + BM - 1) / BM;
    p.tiles_n = (g.epi == Epilogue::SwiGLU) ? p.N / 64 : p.N / BN;
    const unsigned grid = (unsigned)(p.tiles_m * p.tiles_n);
    switch (g.epi) {
        case Epilogue::Store: gemm_bf16_kernel<Epilogue::Store><<<grid, 256, 0, s>>>(p); break;
        case Epilogue::ResidToF32: gemm_bf16_kernel<Epilogue::ResidToF32><<<grid, 256, 0, s>>>(p); break;
        case Epilogue::SwiGLU: gemm_bf16_kernel<Epilogue::SwiGLU><<<grid, 256, 0, s>>>(p); break;
        case Epilogue::ResidF32In: gemm_bf16_kernel<Epilogue::ResidF32In><<<grid, 256, 0, s>>>(p); break;
    }
    return hipGetLastError();
}

hipError_t launch_gemv_bf16(const GemmArgs& g, hipStream_t s) {
    if (g.M <= 0) return hipSuccess;
    DevGemm p = make_dev(g);
    switch (g.epi) {
        case Epilogue::Store: return launch_gemv_epi<Epilogue::Store>(p, s);
        case Epilogue::ResidToF32: return launch_gemv_epi<Epilogue::ResidToF32>(p, s);
        case Epilogue::SwiGLU: return launch_gemv_epi<Epilogue::SwiGLU>(p, s);
        case Epilogue::ResidF32In: return launch_gemv_epi<Epilogue::ResidF32In>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace q3
