// bf16 projections of the layer on gfx950 matrix cores: C[M, N] = A[M, K] * B[N, K]^T, fp32
// accumulation, with the layer's element-wise work fused into the epilogue.
//
// The projections are the nn.Linear layers of "17. A modern architecture: Qwen3" (sections
// Attention with grouped KV heads and Q/K normalization, SwiGLU): q/k/v/o and gate/up/down,
// weights [out, in], no bias.  Both operands are therefore K-contiguous, which is exactly the
// per-lane operand layout of v_mfma_f32_32x32x16_bf16 (each lane feeds 8 consecutive k).
//
// Large-M kernel, templated on the workgroup tile BM x BN and its WM x WN wave grid (each wave
// owns (BM/WM) x (BN/WN), i.e. FM x FN blocks of 32x32); BK = 64, two LDS stages, the next
// k-slab fetched into registers while the current one feeds the MFMAs.  LDS rows are padded to
// 144 bytes: the 16 lanes served per cycle by the 64-bank LDS then read 16 rows of the same
// 16-byte chunk from 16 disjoint bank groups, and every fragment address is a per-lane base
// plus an immediate.  Large problems use 256x256 tiles on 8 waves (one workgroup per CU, two
// waves per SIMD, half the L2 traffic per FLOP of 128x128); smaller ones 128x128 on 4 waves,
// and problems with fewer than 256 such tiles 64x64 (64x128 for SwiGLU) so every CU has work.
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

constexpr int BK = 64;
constexpr int LP = BK + 8;   // LDS row pitch in elements (144 bytes)
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

template <Epilogue EPI, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_kernel(DevGemm p) {
    constexpr bool DUAL = (EPI == Epilogue::SwiGLU);
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;        // wave tile
    constexpr int FM = TM / 32, FN = TN / 32;        // 32x32 blocks per wave
    constexpr int CA = BM * 8 / NT, CB = BN * 8 / NT;  // 16-byte chunks staged per thread per slab
    static_assert(CA >= 1 && CB >= 1 && (BM * 8) % NT == 0 && (BN * 8) % NT == 0, "tile vs threads");
    static_assert(!DUAL || TN % 64 == 0, "SwiGLU tiles need whole gate/up block pairs per wave");
    __shared__ __attribute__((aligned(16))) bf16 sA[2 * BM * LP];
    __shared__ __attribute__((aligned(16))) bf16 sB[2 * BN * LP];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

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

    // ---- global -> register loaders (chunk c = tid + NT j: row c / 8, 16-byte chunk c % 8)
    const bf16* ga[CA];
    const bf16* gb[CB];
    int la[CA], lb[CB];
#pragma unroll
    for (int j = 0; j < CA; ++j) {
        const int c = tid + NT * j;
        const int row = c >> 3, ch = c & 7;
        la[j] = row * LP + ch * 8;
        ga[j] = p.a + (int64_t)min(m0 + row, p.M - 1) * p.K + ch * 8;
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
        const int c = tid + NT * j;
        const int row = c >> 3, ch = c & 7;
        lb[j] = row * LP + ch * 8;
        if constexpr (DUAL) {
            // B tile rows in blocks of 32: gate, up, gate, up, ... of output columns
            // tn*BN/2 + 32*(row/64) + row%32
            const int n = tn * (BN / 2) + (row >> 6) * 32 + (row & 31);
            gb[j] = p.b[(row >> 5) & 1] + (int64_t)n * p.K + ch * 8;
        } else {
            gb[j] = seg_row(p, tn * BN + row) + ch * 8;
        }
    }
    bf16x8 ra[CA], rb[CB];
    auto gload = [&](int kt) {
#pragma unroll
        for (int j = 0; j < CA; ++j) ra[j] = *reinterpret_cast<const bf16x8*>(ga[j] + kt * BK);
#pragma unroll
        for (int j = 0; j < CB; ++j) rb[j] = *reinterpret_cast<const bf16x8*>(gb[j] + kt * BK);
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < CA; ++j) *reinterpret_cast<bf16x8*>(&sA[buf * BM * LP + la[j]]) = ra[j];
#pragma unroll
        for (int j = 0; j < CB; ++j) *reinterpret_cast<bf16x8*>(&sB[buf * BN * LP + lb[j]]) = rb[j];
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // fragment reads: row (wave's first row) + 32 i + lane%32, chunk 2 kk + lane/32
    const int a_rd = (wm * TM + (lane & 31)) * LP + (lane >> 5) * 8;
    const int b_rd = (wn * TN + (lane & 31)) * LP + (lane >> 5) * 8;
    const int nk = p.K / BK;
    gload(0);
    lstore(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const bf16* pa = sA + buf * BM * LP + a_rd;
        const bf16* pb = sB + buf * BN * LP + b_rd;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8*>(pa + i * 32 * LP + kk * 16);
#pragma unroll
            for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(pb + j * 32 * LP + kk * 16);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue.  32x32 accumulator layout: lane l, register r holds
    //      row 8*(r/4) + 4*(l/32) + r%4, column l%32 of its block.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * TM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row >= p.M) continue;
            if constexpr (DUAL) {
#pragma unroll
                for (int j = 0; j < FN; j += 2) {   // blocks j (gate) and j+1 (up) share columns
                    const int col = tn * (BN / 2) + (wn * TN + j * 32) / 2 + (lane & 31);
                    static_cast<bf16*>(p.out)[(int64_t)row * p.N + col] =
                        (bf16)silu_mul(acc[i][j][r], acc[i][j + 1][r]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int col = tn * BN + wn * TN + j * 32 + (lane & 31);
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

template <Epilogue EPI, int BM, int BN, int WM, int WN>
static hipError_t run_tile(DevGemm p, hipStream_t s) {
    const int bn_out = (EPI == Epilogue::SwiGLU) ? BN / 2 : BN;
    if (p.N % bn_out || p.K % BK) return hipErrorInvalidValue;
    p.tiles_m = (p.M + BM - 1) / BM;
    p.tiles_n = p.N / bn_out;
    gemm_bf16_kernel<EPI, BM, BN, WM, WN><<<(unsigned)(p.tiles_m * p.tiles_n), WM * WN * 64, 0, s>>>(p);
    return hipGetLastError();
}

template <Epilogue EPI>
static hipError_t run_epi(const DevGemm& p, hipStream_t s) {
    // The largest tile that still gives at least one workgroup per CU (256 CUs).
    constexpr bool DUAL = (EPI == Epilogue::SwiGLU);
    const int bn256 = DUAL ? 128 : 256, bn128 = DUAL ? 64 : 128;
    const long tiles256 = (long)((p.M + 255) / 256) * (p.N / bn256);
    const long tiles128 = (long)((p.M + 127) / 128) * (p.N / bn128);
    if (tiles256 >= 256 && p.N % bn256 == 0) return run_tile<EPI, 256, 256, 4, 2>(p, s);
    if (tiles128 >= 256) return run_tile<EPI, 128, 128, 2, 2>(p, s);
    if constexpr (DUAL)
        return run_tile<EPI, 64, 128, 2, 2>(p, s);
    else
        return run_tile<EPI, 64, 64, 2, 2>(p, s);
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s) {
    if (g.M <= 0) return hipSuccess;
    const DevGemm p = make_dev(g);
    switch (g.epi) {
        case Epilogue::Store: return run_epi<Epilogue::Store>(p, s);
        case Epilogue::ResidToF32: return run_epi<Epilogue::ResidToF32>(p, s);
        case Epilogue::SwiGLU: return run_epi<Epilogue::SwiGLU>(p, s);
        case Epilogue::ResidF32In: return run_epi<Epilogue::ResidF32In>(p, s);
    }
    return hipErrorInvalidValue;
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
