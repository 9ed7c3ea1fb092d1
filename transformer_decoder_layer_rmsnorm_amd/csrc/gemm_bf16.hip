// bf16 projections of the layer on gfx950 matrix cores: C[M, N] = A[M, K] * B[N, K]^T, fp32
// accumulation, with the layer's element-wise work fused into the epilogue.
//
// The projections are the nn.Linear layers of "17. A modern architecture: Qwen3" (sections
// Attention with grouped KV heads and Q/K normalization, SwiGLU): q/k/v/o and gate/up/down,
// weights [out, in], no bias.  Both operands are therefore K-contiguous, which is exactly the
// per-lane operand layout of v_mfma_f32_32x32x16_bf16 (each lane feeds 8 consecutive k).
//
// Large tiles (256 x 256 on 8 waves, one workgroup per CU, two waves per SIMD) stage operands
// with direct global->LDS loads (buffer_load_dwordx4 ... lds: lane l's 16 bytes land at the
// wave's LDS base + 16 l, without passing through VGPRs) in 64-k stages of 128-byte LDS rows, so
// every load moves whole cache lines, and the two wave groups of each SIMD alternate between
// memory and matrix phases ("ping-pong", see gemm_bf16_pp_kernel).  The validated layer shapes
// make every K a multiple of 128, so no other large-tile form is needed.  The ping-pong kernel
// also has a 256 x 128 form, used by the fused QKV projection when 256 x 256 tiles would leave
// too many CUs idle.  Its epilogues that read a residual stage the tile through LDS and move 16
// bytes per lane (see pp_store_tile).
//
// Smaller tiles (128 x 128 on 4 waves; 64 x 64, or 64 x 128 for SwiGLU, when fewer than 256
// tiles would remain; 64 x 128 for split-K partial slabs) keep a register prefetch: BK = 64, two LDS stages, the next k-slab fetched
// into registers while the current one feeds the MFMAs, two or more workgroups per CU.  Their LDS
// rows are padded to 144 bytes: the 16 lanes served per cycle by the 64-bank LDS then read 16 rows
// of the same 16-byte chunk from 16 disjoint bank groups.
//
// Every tile is a grid of 32x32 MFMA blocks per wave (FM x FN blocks of the wave's share).
// Tiles are remapped so that each XCD works on a contiguous band of tiles, grouped 8 M-tiles
// at a time for L2 reuse of the weight tiles.
//
// Skinny kernel (decode, M <= 64): v_mfma_f32_16x16x32_bf16 with the weight rows streamed
// straight from HBM into B fragments; each workgroup owns 16 output columns and deals K out to
// its waves in interleaved 32-k chunks, reducing through LDS.
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
    int splits;           // PartialF32: number of K ranges (one fp32 slab [M, N] each)
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
    } else if constexpr (EPI == Epilogue::PartialF32) {
        static_cast<float*>(p.out)[(int64_t)row * p.N + col] = v;   // p.out already at this split's slab
    }
}

// Tile of workgroup `bid`: contiguous band of tiles per XCD (bid % 8), grouped along M.
__device__ __forceinline__ void tile_of(const DevGemm& p, int bid, int& tm, int& tn) {
    const int total = p.tiles_m * p.tiles_n;
    int t = bid;
    if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
    const int per_group = kGroupM * p.tiles_n;
    const int group = t / per_group;
    const int first_m = group * kGroupM;
    const int gsize = min(p.tiles_m - first_m, kGroupM);
    tm = first_m + (t % per_group) % gsize;
    tn = (t % per_group) / gsize;
}

// Epilogue of one wave's FM x FN blocks.  32x32 accumulator layout: lane l, register r holds
// row 8*(r/4) + 4*(l/32) + r%4, column l%32 of its block.
template <Epilogue EPI, int BN, int TM, int TN, int FM, int FN>
__device__ __forceinline__ void write_tile(const DevGemm& p, const f32x16 (&acc)[FM][FN], int m0, int tn, int wm,
                                           int wn, int lane) {
    constexpr bool DUAL = (EPI == Epilogue::SwiGLU);
    if constexpr (DUAL) {
        // Every row of the wave in range (all but a ragged last tile): no per-row branch, so the
        // exponentials and reciprocals of all the wave's outputs are one straight-line block the
        // compiler interleaves, instead of short dependent chains behind an exec-mask branch each.
        if (m0 + wm * TM + TM <= p.M) {
            // the wave's rows from one uniform base: each store address is that base plus a 32-bit
            // lane offset plus a uniform row offset (no 64-bit arithmetic per row); TM rows of N
            // bf16 stay far below 4 GiB
            char* base = reinterpret_cast<char*>(static_cast<bf16*>(p.out) + (int64_t)(m0 + wm * TM) * p.N +
                                                 tn * (BN / 2) + (wn * TN) / 2);
            const unsigned lane_off = (unsigned)(4 * (lane >> 5) * p.N + (lane & 31) + ((lane & 1) ? 31 : 0)) * 2u;
            // bytes of {partner's word, own word}: even lanes (own low, partner low), odd lanes
            // (partner high, own high)
            const unsigned pair_sel = (lane & 1) ? 0x03020706u : 0x05040100u;
            constexpr int NJ = FN / 2;   // outputs per row and lane
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    // four rows at a time: their 4 NJ exponentials, then the reciprocals, then the
                    // products and stores (silu(g) u = g u / (1 + e^-g))
                    float e[4][NJ];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                        for (int jj = 0; jj < NJ; ++jj) e[rr][jj] = __expf(-acc[i][2 * jj][4 * rq + rr]);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                        for (int jj = 0; jj < NJ; ++jj) e[rr][jj] = __builtin_amdgcn_rcpf(1.0f + e[rr][jj]);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int r = 4 * rq + rr;
                        const unsigned row_off = (unsigned)((i * 32 + 8 * rq + rr) * p.N) * 2u;
                        if constexpr (NJ == 2) {
                            // lanes 2k and 2k + 1 hold adjacent columns of the row: each packs its
                            // two outputs (columns c and c + 32), the pair swaps the packed words,
                            // and a byte permute keeps two adjacent outputs per lane for one 4-byte
                            // store (the even lane its column and the next, the odd lane columns
                            // 31 + its own)
                            const bf16x2 own = {(bf16)(acc[i][0][r] * acc[i][1][r] * e[rr][0]),
                                                (bf16)(acc[i][2][r] * acc[i][3][r] * e[rr][1])};
                            const unsigned pw = __builtin_bit_cast(unsigned, own);
                            const unsigned qw = (unsigned)__builtin_amdgcn_mov_dpp((int)pw, 0xB1, 0xf, 0xf, false);
                            *reinterpret_cast<unsigned*>(base + (lane_off + row_off)) = __builtin_amdgcn_perm(qw, pw, pair_sel);
                        } else {
                            const unsigned own = lane_off - ((lane & 1) ? 62u : 0u);   // this lane's column
#pragma unroll
                            for (int jj = 0; jj < NJ; ++jj)
                                *reinterpret_cast<bf16*>(base + (own + row_off + jj * 64)) =
                                    (bf16)(acc[i][2 * jj][r] * acc[i][2 * jj + 1][r] * e[rr][jj]);
                        }
                    }
                }
            return;
        }
    }
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

// Main loop of the register-prefetch kernel: accumulates the workgroup's tile (and K range, for
// split-K) into acc and hands acc to `epi` with the tile's coordinates; smem is the kernel's LDS,
// free for the epilogue once the loop has ended.
template <Epilogue EPI, int BM, int BN, int WM, int WN, typename Epi>
__device__ __forceinline__ void gemm_bf16_body(const DevGemm& p, bf16* smem, Epi&& epi) {
    constexpr bool DUAL = (EPI == Epilogue::SwiGLU);
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;        // wave tile
    constexpr int FM = TM / 32, FN = TN / 32;        // 32x32 blocks per wave
    constexpr int CA = BM * 8 / NT, CB = BN * 8 / NT;  // 16-byte chunks staged per thread per slab
    static_assert(CA >= 1 && CB >= 1 && (BM * 8) % NT == 0 && (BN * 8) % NT == 0, "tile vs threads");
    static_assert(!DUAL || TN % 64 == 0, "SwiGLU tiles need whole gate/up block pairs per wave");
    bf16* sA = smem;
    bf16* sB = smem + 2 * BM * LP;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // split-K: workgroup blockIdx.x covers tile blockIdx.x % tiles over K range blockIdx.x / tiles
    const int tiles = p.tiles_m * p.tiles_n;
    const int split = (int)blockIdx.x / tiles;
    int tm, tn;
    tile_of(p, (int)blockIdx.x - split * tiles, tm, tn);
    const int m0 = tm * BM;
    const int nk = p.K / BK / p.splits;
    const int k_base = split * nk * BK;

    // ---- global -> register loaders (chunk c = tid + NT j: row c / 8, 16-byte chunk c % 8)
    const bf16* ga[CA];
    const bf16* gb[CB];
    int la[CA], lb[CB];
#pragma unroll
    for (int j = 0; j < CA; ++j) {
        const int c = tid + NT * j;
        const int row = c >> 3, ch = c & 7;
        la[j] = row * LP + ch * 8;
        ga[j] = p.a + (int64_t)min(m0 + row, p.M - 1) * p.K + k_base + ch * 8;
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
            gb[j] = p.b[(row >> 5) & 1] + (int64_t)n * p.K + k_base + ch * 8;
        } else {
            gb[j] = seg_row(p, tn * BN + row) + k_base + ch * 8;
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
    gload(0);
    lstore(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        const bf16* pa = sA + buf * BM * LP + a_rd;
        const bf16* pb = sB + buf * BN * LP + b_rd;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            // With several MFMA blocks per wave the next slab is requested once the first MFMAs
            // of this one are queued, so a wave that stalls on a full address queue still has
            // matrix work in flight; with one block per wave it is requested up front.
            if (kk == (FM * FN >= 4 ? 1 : 0) && kt + 1 < nk) gload(kt + 1);
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

    epi(acc, m0, tn, wm, wn, lane, split);
}

template <Epilogue EPI, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_kernel(DevGemm p) {
    constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * BM * LP + 2 * BN * LP];
    gemm_bf16_body<EPI, BM, BN, WM, WN>(p, smem, [&](const f32x16 (&acc)[FM][FN], int m0, int tn, int wm, int wn,
                                                     int lane, int split) {
        DevGemm q = p;
        if constexpr (EPI == Epilogue::PartialF32) q.out = static_cast<float*>(p.out) + (int64_t)split * p.M * p.N;
        write_tile<EPI, BN, TM, TN, FM, FN>(q, acc, m0, tn, wm, wn, lane);
    });
}

// ------------------------------------------------------------------ QKV projection + QK-norm + RoPE
// Each 128-column block of the q | k | v product is exactly one head (head_dim 128), so the
// epilogue can finish step 3 of the layer in place ("17. A modern architecture: Qwen3", section
// Attention with grouped KV heads and Q/K normalization: per-head RMSNorm of q and k over
// head_dim with one gain per projection, then rotate-half RoPE at the token's position; v copied
// to the cache): the fp32 tile goes to LDS, then 16 lanes per token row normalise, rotate and
// store it as qhat [B, Hq, T, D] or into the K / V cache slots.  The q / k vectors are normalised
// from the fp32 accumulators (no bf16 rounding before the norm); each row's (cos, sin) and cache
// slot come from the table the input RMSNorm wrote (RopeTable).  128 x 128 register tiles hold
// one head per tile, 256 x 256 ping-pong tiles two (see gemm_qkv_qkrope_pp_kernel).
__device__ __forceinline__ float dpp_row_f32(float x, int ctrl_sel) {
    switch (ctrl_sel) {
        case 0: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xf, 0xf, false));
        case 1: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xf, 0xf, false));
        case 2: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xf, 0xf, false));
        default: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xf, 0xf, false));
    }
}
// sum over each 16-lane row of the wave (DPP: quad permutes, half-row and row mirrors)
__device__ __forceinline__ float sum16(float v) {
    v += dpp_row_f32(v, 0);
    v += dpp_row_f32(v, 1);
    v += dpp_row_f32(v, 2);
    v += dpp_row_f32(v, 3);
    return v;
}

// Gains of head hs for the features lane jl handles (4jl..4jl+3 and 64+4jl..64+4jl+3).
template <typename Args>
__device__ __forceinline__ void qkrope_gains(const Args& a, int hs, int jl, float (&g)[8]) {
    const bool is_v = hs >= a.Hq + a.Hkv, is_q = hs < a.Hq;
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = 0.f;
    if (is_v) return;
    const void* qn = a.q_norm;
    const void* kn = a.k_norm;
    asm("" : "+s"(qn), "+s"(kn));   // select the loaded pointers, not the argument fields
    const bf16* gain = static_cast<const bf16*>(is_q ? qn : kn);
    const bf16x4 g0 = *reinterpret_cast<const bf16x4*>(gain + 4 * jl);
    const bf16x4 g1 = *reinterpret_cast<const bf16x4*>(gain + 64 + 4 * jl);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        g[e] = a.goff + (float)g0[e];
        g[4 + e] = a.goff + (float)g1[e];
    }
}

// Arguments of the ping-pong variant: pointers and sizes only.  Its main loop is written with
// memory-clobbering inline assembly, after which the compiler no longer reads a by-value kernel
// argument in place but copies it to scratch memory when an array inside it is indexed at run
// time; the arrays of QkRopeArgs are not needed here (angles and slots come from the table).
struct QkPpArgs {
    const void* q_norm;
    const void* k_norm;
    void* qhat;
    void* k_cache;
    void* v_cache;
    const float* rope_cs;
    const int32_t* rope_slot;
    int T, Hq, Hkv, cap;
    float eps, goff;
};

// A token row's entries of the RoPE table for lane jl: (cos, sin) of frequencies 4jl..4jl+3
// and the row's cache slot.  The epilogues fetch them for all their rows before the tile goes
// through LDS, so the table's latency overlaps that step instead of every row's processing.
struct RopeRow {
    f32x4 c01, c23;
    int lin;
};
template <typename Args>
__device__ __forceinline__ RopeRow rope_row_load(int m, int jl, bool need_cs, bool need_slot, const DevGemm& p,
                                                 const Args& a) {
    const int mc = m < p.M ? m : p.M - 1;
    RopeRow r{};
    if (need_cs) {
        const float* csr = a.rope_cs + (int64_t)mc * 128 + 8 * jl;
        r.c01 = *reinterpret_cast<const f32x4*>(csr);
        r.c23 = *reinterpret_cast<const f32x4*>(csr + 4);
    }
    if (need_slot) r.lin = a.rope_slot[mc];
    return r;
}

// Token row m of head hs (q, k or v column block of the QKV product), fp32 values at `tr`:
// q and k are RMS-normalised over the head, scaled by their gains and rotated with the row's
// (cos, sin) from the RoPE table, then stored to qhat or the K cache slot; v is rounded and
// stored to the V cache slot.  The 16 lanes of a DPP row share the token; lane jl owns features
// 4jl..4jl+3 and their rotation partners 64+4jl..64+4jl+3.  Every lane of the row takes part in
// the reduction even when m >= M (its loads are clamped and its store is skipped).
template <typename Args>
__device__ __forceinline__ void qkrope_row(const float* tr, int jl, int m, int hs, const float (&g)[8],
                                           const DevGemm& p, const Args& a, const RopeRow& rr) {
    constexpr int D = 128;
    // the argument's fields as values (selecting between fields would index the argument)
    void* qhat = a.qhat;
    void* kc = a.k_cache;
    void* vc = a.v_cache;
    int Hq = a.Hq, Hkv = a.Hkv;
    asm("" : "+s"(qhat), "+s"(kc), "+s"(vc), "+s"(Hq), "+s"(Hkv));
    const bool is_v = hs >= Hq + Hkv, is_q = hs < Hq;
    const bool valid = m < p.M;
    const int mc = valid ? m : p.M - 1;
    const int b = mc / a.T, t = mc - b * a.T;
    const int lin = rr.lin;
    const f32x4 lo = *reinterpret_cast<const f32x4*>(tr + 4 * jl);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(tr + 64 + 4 * jl);
    bf16x4 olo, ohi;
    bf16* dst;
    if (is_v) {
#pragma unroll
        for (int e = 0; e < 4; ++e) { olo[e] = (bf16)lo[e]; ohi[e] = (bf16)hi[e]; }
        dst = static_cast<bf16*>(vc) + (((int64_t)b * Hkv + (hs - Hq - Hkv)) * a.cap + lin) * D;
    } else {
        const f32x4 c01 = rr.c01, c23 = rr.c23;   // (cos, sin) of 4jl..4jl+3
        const float cs[4] = {c01[0], c01[2], c23[0], c23[2]}, sn[4] = {c01[1], c01[3], c23[1], c23[3]};
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) ss = fmaf(lo[e], lo[e], fmaf(hi[e], hi[e], ss));
        const float rstd = rsqrtf(sum16(ss) * (1.0f / D) + a.eps);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float n0 = g[e] * (lo[e] * rstd), n1 = g[4 + e] * (hi[e] * rstd);
            olo[e] = (bf16)(n0 * cs[e] - n1 * sn[e]);
            ohi[e] = (bf16)(n1 * cs[e] + n0 * sn[e]);
        }
        dst = is_q ? static_cast<bf16*>(qhat) + (((int64_t)b * Hq + hs) * a.T + t) * D
                   : static_cast<bf16*>(kc) + (((int64_t)b * Hkv + (hs - Hq)) * a.cap + lin) * D;
    }
    if (valid) {
        *reinterpret_cast<bf16x4*>(dst + 4 * jl) = olo;
        *reinterpret_cast<bf16x4*>(dst + 64 + 4 * jl) = ohi;
    }
}

__global__ __launch_bounds__(256) void gemm_qkv_qkrope_kernel(DevGemm p, QkRopeArgs a) {
    constexpr int BM = 128, BN = 128, WM = 2, WN = 2, TM = 64, TN = 64, FM = 2, FN = 2, D = 128;
    constexpr int TP = D + 8;   // fp32 tile pitch: rows r and r+4 of a store land 32 banks apart
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * BM * LP + 2 * BN * LP];
    static_assert(BM * TP * 4 <= (int)sizeof(smem), "fp32 tile fits the main loop's LDS");
    gemm_bf16_body<Epilogue::Store, BM, BN, WM, WN>(p, smem, [&](const f32x16 (&acc)[FM][FN], int m0, int tn,
                                                                 int wm, int wn, int lane, int) {
        float* tile = reinterpret_cast<float*>(smem);
        const int jl = threadIdx.x & 15, r0 = threadIdx.x >> 4;
        constexpr int NR = BM / 16;   // token rows per thread
        const bool need_cs = tn < a.Hq + a.Hkv, need_slot = tn >= a.Hq;   // q/k rotate, k/v go to the cache
        RopeRow rr[NR];
#pragma unroll
        for (int k = 0; k < NR; ++k) rr[k] = rope_row_load(m0 + r0 + 16 * k, jl, need_cs, need_slot, p, a);
        // the main loop ended with a barrier: every wave is done reading its last k-slab
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wm * TM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    tile[row * TP + wn * TN + j * 32 + (lane & 31)] = acc[i][j][r];
                }
        __syncthreads();
        float g[8];
        qkrope_gains(a, tn, jl, g);   // the column block is head tn of the q | k | v layout
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const int row = r0 + 16 * k;
            qkrope_row(tile + row * TP, jl, m0 + row, tn, g, p, a, rr[k]);
        }
    });
}


// ------------------------------------------------------------------ direct global->LDS loads
typedef int int4v __attribute__((ext_vector_type(4)));

// Buffer descriptor held in SGPRs: base, stride 0, num_records bytes (reads past them return 0).
__device__ __forceinline__ int4v sgpr_desc(const void* base, int nbytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    int4v d;
    d[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    d[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffff));
    d[2] = __builtin_amdgcn_readfirstlane(nbytes);
    d[3] = 0x00020000;
    return d;
}
// One 16-byte global->LDS load per lane.  Issued as inline assembly so that the compiler does
// not treat it as an LDS write of unknown extent (it would then wait for every such load before
// any LDS read, which defeats the multi-stage pipeline); completion is tracked explicitly with
// vmcnt below.
__device__ __forceinline__ void dma16(int4v rsrc, int voff, int soff, unsigned lds_addr) {
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_addr) : "memory");
}

// ------------------------------------------------------------------ large tiles: ping-pong
// 256 x 256 tiles on 8 waves (4 x 2, each wave 64 x 128), BK = 64 per stage in two LDS stages of
// 128-byte rows (8 chunks of 16 bytes, XOR-swizzled by (row >> 1) & 7), so that every DMA
// instruction moves 8 rows x 128 contiguous bytes: whole cache lines, which measurably lowers the
// traffic and power of the operand stream compared with 64-byte row segments.
//
// Waves 0-3 and 4-7 (one of each per SIMD) alternate, offset by one phase through an extra
// barrier: while one group issues its LDS fragment reads and DMA requests, the other runs 16
// MFMAs, so each SIMD's matrix core is fed by one wave at a time without either waiting on LDS.
// A phase covers one 32-row half i of the wave's A rows over the whole 64-k stage; the B
// fragments of the stage are read in phase 0 and held in registers for phase 1.  So B and the
// i = 0 rows of A are free one phase early and are refilled two stages ahead (requested in phase
// (t, 1) for stage t + 2); the i = 1 rows of A are requested in phase (t, 0) for stage t + 1.
// Every request is waited for four phases after it was issued.
__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }
template <int N> __device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }
__device__ __forceinline__ void lgkm_wait0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }
// at most n loads of this wave in flight; n is one of the counts the schedule below produces
__device__ __forceinline__ void vm_wait_at_most(int n) {
    if (n >= 8) vm_wait<8>();
    else if (n >= 6) vm_wait<6>();
    else if (n >= 2) vm_wait<2>();
    else vm_wait<0>();
}

// Tiles are 256 x BN (BN = 256 or 128) over 4 x 2 waves: a wave owns 64 rows and BN / 2 columns.
constexpr int kPpBM = 256, kPpK = 64;
constexpr int kPpTM = 64, kPpFM = 2;
constexpr int kPpStage = kPpBM * kPpK;   // A elements per stage
template <int BN> struct PpTile {
    static constexpr int TN = BN / 2, FN = TN / 32;
    static constexpr int NB = BN / 64;        // B DMA instructions per wave and stage (8 rows each)
    static constexpr int B_ST = BN * kPpK;    // B elements per stage
};

// Main loop of the ping-pong kernel: accumulates the workgroup's 256 x BN tile and hands acc to
// `epi` with the tile's coordinates.  sA and sB are the kernel's LDS (2 stages each, 1 KB-aligned),
// free for the epilogue once the loop has ended.
template <Epilogue EPI, int BN, typename Epi>
__device__ __forceinline__ void gemm_pp_body(const DevGemm& p, bf16* sA, bf16* sB, Epi&& epi) {
    constexpr int BM = kPpBM, WN = 2, PK = kPpK;
    constexpr int TM = kPpTM, FM = kPpFM, TN = PpTile<BN>::TN, FN = PpTile<BN>::FN, NB = PpTile<BN>::NB;
    constexpr bool DUAL = (EPI == Epilogue::SwiGLU);
    constexpr int A_ST = kPpStage, B_ST = PpTile<BN>::B_ST;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int grp = wave >> 2;
    int tm, tn;
    tile_of(p, blockIdx.x, tm, tn);
    const int m0 = tm * BM;
    const int rowbytes = p.K * 2;

    // DMA instructions of this wave, 8 tile rows each.  A: two per half h (h = 0: rows
    // 64 w + 0..31 of every wave row w, h = 1: rows 64 w + 32..63); B: BN / 64.  A rows past M
    // read as zeros (the descriptor covers only the valid rows).
    int4v ra[2][2], rb[NB];
    int ra_row[2][2], rb_row[NB];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = wave * 2 + i;
            const int tr = (q >> 2) * 64 + 32 * h + (q & 3) * 8;
            ra_row[h][i] = tr;
            const int r0 = m0 + tr;
            const int nrows = max(0, min(8, p.M - r0));
            ra[h][i] = sgpr_desc(p.a + (int64_t)min(r0, p.M - 1) * p.K, nrows * rowbytes);
        }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int lr = (wave * NB + i) * 8;
        rb_row[i] = lr;
        const bf16* base;
        if constexpr (DUAL) {
            // B tile rows in blocks of 32: gate, up, gate, up, ... of output columns
            // tn*BN/2 + 32*(row/64) + row%32
            const int n = tn * (BN / 2) + (lr >> 6) * 32 + (lr & 31);
            base = p.b[(lr >> 5) & 1] + (int64_t)n * p.K;
        } else {
            base = seg_row(p, tn * BN + lr);   // 8 rows never straddle a segment
        }
        rb[i] = sgpr_desc(base, 8 * rowbytes);
    }
    // lane l moves row 8g + l/8 of its instruction's rows, into physical chunk l % 8, which holds
    // logical chunk (l % 8) ^ swz8(row); swz8 depends on the parity of g
    const int r8 = lane >> 3;
    const int voff_even = r8 * rowbytes + (((lane & 7) ^ swz8(r8)) << 4);
    const int voff_odd = r8 * rowbytes + (((lane & 7) ^ swz8(8 + r8)) << 4);
    const unsigned sA_lds = (unsigned)(uintptr_t)(__attribute__((address_space(3))) bf16*)sA;
    const unsigned sB_lds = (unsigned)(uintptr_t)(__attribute__((address_space(3))) bf16*)sB;
    auto issue_b_a0 = [&](int st) {   // NB + 2 loads
        const int slot = st & 1;
        const int soff = st * (PK * 2);
#pragma unroll
        for (int i = 0; i < NB; ++i)
            dma16(rb[i], ((rb_row[i] >> 3) & 1) ? voff_odd : voff_even, soff,
                  __builtin_amdgcn_readfirstlane(sB_lds + (slot * B_ST + rb_row[i] * PK) * 2));
#pragma unroll
        for (int i = 0; i < 2; ++i)
            dma16(ra[0][i], ((ra_row[0][i] >> 3) & 1) ? voff_odd : voff_even, soff,
                  __builtin_amdgcn_readfirstlane(sA_lds + (slot * A_ST + ra_row[0][i] * PK) * 2));
    };
    auto issue_a1 = [&](int st) {     // 2 loads
        const int slot = st & 1;
        const int soff = st * (PK * 2);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            dma16(ra[1][i], ((ra_row[1][i] >> 3) & 1) ? voff_odd : voff_even, soff,
                  __builtin_amdgcn_readfirstlane(sA_lds + (slot * A_ST + ra_row[1][i] * PK) * 2));
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // fragment reads for k step q (k 16q .. 16q+15): row (wave base) + 32 i + lane % 32,
    // logical chunk 2q + lane / 32
    const int fr = lane & 31;
    int a_rd[4], b_rd[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        a_rd[q] = (wm * TM + fr) * PK + (((2 * q + (lane >> 5)) ^ swz8(fr)) << 3);
        b_rd[q] = (wn * TN + fr) * PK + (((2 * q + (lane >> 5)) ^ swz8(fr)) << 3);
    }
    const int nst = p.K / PK;

    // Request order: B,A0(0) A1(0) B,A0(1), then per stage t: A1(t+1) in phase (t,0) and
    // B,A0(t+2) in phase (t,1).  Before a phase's closing barrier each wave waits for the data
    // the next phase reads: A1(t) at the end of (t,0), B,A0(t+1) at the end of (t,1).
    issue_b_a0(0);
    issue_a1(0);
    if (nst > 1) issue_b_a0(1);
    vm_wait_at_most(nst > 1 ? NB + 4 : 2);
    barrier_only();
    if (grp == 1) barrier_only();
    bf16x8 af[4], bfr[4][FN];
    for (int t = 0; t < nst; ++t) {
        const bf16* pa = sA + (t & 1) * A_ST;
        const bf16* pb = sB + (t & 1) * B_ST;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            // ---- memory phase
            __builtin_amdgcn_sched_barrier(0);
            if (i == 0) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int j = 0; j < FN; ++j) bfr[q][j] = *reinterpret_cast<const bf16x8*>(pb + b_rd[q] + j * 32 * PK);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) af[q] = *reinterpret_cast<const bf16x8*>(pa + a_rd[q] + i * 32 * PK);
            if (i == 0) {
                if (t + 1 < nst) issue_a1(t + 1);
                vm_wait_at_most(t + 1 < nst ? NB + 4 : 0);
            } else {
                if (t + 2 < nst) issue_b_a0(t + 2);
                vm_wait_at_most((t + 1 < nst ? 2 : 0) + (t + 2 < nst ? NB + 2 : 0));
            }
            lgkm_wait0();
            barrier_only();
            __builtin_amdgcn_sched_barrier(0);
            // ---- compute phase
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[q], bfr[q][j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            barrier_only();
        }
    }
    if (grp == 0) barrier_only();
    epi(acc, m0, tn, wm, wn, lane);
}

// Epilogue of the ping-pong kernel through LDS, for the epilogues that read a residual.  Storing
// straight from the accumulators moves 2 or 4 bytes per lane and instruction and loads the
// residual the same way: over two thousand memory instructions per workgroup, issued by every
// workgroup of a round at once while the matrix cores idle.  Instead each half of the tile (128
// rows: the waves of rows 0-1, then 2-3) goes to LDS as fp32 (row pitch BNo + 8 floats so the
// two row groups of a store hit different banks), then every thread finishes 8 consecutive
// output columns of a row with 16-byte loads and stores.  A half's residual chunks are all
// requested before any of them is used (the first half's before the accumulators go to LDS, the
// second half's as soon as the first half's registers are free): the compiler cannot move a
// residual load above the output stores before it (it cannot tell that out and resid never
// overlap), and loading chunk by chunk made every chunk a full memory round trip.  The plain and
// SwiGLU epilogues, which read nothing, store from the accumulators.
template <Epilogue EPI, int BN>
struct PpEpi {
    static_assert(EPI != Epilogue::SwiGLU, "SwiGLU stores from the accumulators");
    static constexpr int BNo = BN;         // output columns
    static constexpr int P = BNo + 8;      // LDS row pitch (floats)
    static constexpr int BYTES = 128 * P * 4;
};
// Residual chunk of 8 columns: bf16 x for o_proj, fp32 x1 for down (none for split-K slabs).
template <Epilogue EPI> struct ResidChunk { f32x4 lo, hi; };
template <> struct ResidChunk<Epilogue::ResidToF32> { bf16x8 v; };
template <Epilogue EPI>
__device__ __forceinline__ void load_resid_chunk(const DevGemm& p, int64_t o, ResidChunk<EPI>& r) {
    if constexpr (EPI == Epilogue::ResidToF32) {
        r.v = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(p.resid) + o);
    } else if constexpr (EPI == Epilogue::ResidF32In) {
        r.lo = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.resid) + o);
        r.hi = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.resid) + o + 4);
    }
}
template <Epilogue EPI, int BN>
__device__ __forceinline__ void pp_store_tile(const DevGemm& p, const f32x16 (&acc)[kPpFM][PpTile<BN>::FN], int m0,
                                              int tn, int wm, int wn, int lane, float* tile) {
    using T = PpTile<BN>;
    using E = PpEpi<EPI, BN>;
    constexpr int CPR = E::BNo / 8;             // 8-column chunks per row
    constexpr int PER = 128 * CPR / 512;        // chunks per thread and half
    constexpr bool RESID = (EPI == Epilogue::ResidToF32 || EPI == Epilogue::ResidF32In);
    // chunk k of this thread in half h: tile row 128 h + lr, columns c0 .. c0 + 7
    auto chunk_at = [&](int h, int k, int& lr, int& c0, int& m, int64_t& o) {
        const int c = (int)threadIdx.x + 512 * k;
        lr = c / CPR;
        c0 = (c % CPR) * 8;
        m = m0 + 128 * h + lr;
        o = (int64_t)m * p.N + tn * E::BNo + c0;
    };
    ResidChunk<EPI> rv[RESID ? PER : 1];
    auto load_half = [&](int h) {
        if constexpr (RESID) {
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                int lr, c0, m;
                int64_t o;
                chunk_at(h, k, lr, c0, m, o);
                if (m < p.M) load_resid_chunk<EPI>(p, o, rv[k]);
            }
        }
    };
    load_half(0);
    __syncthreads();   // every wave is past its last LDS fragment read
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if ((wm >> 1) == h) {
#pragma unroll
            for (int i = 0; i < kPpFM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = (wm & 1) * kPpTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
#pragma unroll
                    for (int j = 0; j < T::FN; ++j) tile[row * E::P + wn * T::TN + j * 32 + (lane & 31)] = acc[i][j][r];
                }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            int lr, c0, m;
            int64_t o;
            chunk_at(h, k, lr, c0, m, o);
            if (m < p.M) {
                const f32x4 v0 = *reinterpret_cast<const f32x4*>(tile + lr * E::P + c0);
                const f32x4 v1 = *reinterpret_cast<const f32x4*>(tile + lr * E::P + c0 + 4);
                float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                if constexpr (EPI == Epilogue::ResidToF32) {
                    f32x4 w0, w1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        w0[e] = (float)rv[k].v[e] + v[e];
                        w1[e] = (float)rv[k].v[4 + e] + v[4 + e];
                    }
                    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + o) = w0;
                    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + o + 4) = w1;
                } else if constexpr (EPI == Epilogue::PartialF32) {
                    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + o) = v0;
                    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + o + 4) = v1;
                } else {
                    if constexpr (EPI == Epilogue::ResidF32In) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            v[e] += rv[k].lo[e];
                            v[4 + e] += rv[k].hi[e];
                        }
                    }
                    bf16x8 b;
#pragma unroll
                    for (int e = 0; e < 8; ++e) b[e] = (bf16)v[e];
                    *reinterpret_cast<bf16x8*>(static_cast<bf16*>(p.out) + o) = b;
                }
            }
        }
        if (h == 0) {
            load_half(1);
            __syncthreads();   // the second half overwrites the LDS tile
        }
    }
}

template <Epilogue EPI, int BN>
__global__ __launch_bounds__(512) void gemm_bf16_pp_kernel(DevGemm p) {
    using T = PpTile<BN>;
    constexpr bool VIA_LDS = (EPI == Epilogue::ResidToF32 || EPI == Epilogue::ResidF32In || EPI == Epilogue::PartialF32);
    constexpr int LOOP = 2 * (kPpStage + T::B_ST) * 2;
    constexpr int EPIB = VIA_LDS ? 128 * (BN + 8) * 4 : 0;   // PpEpi<EPI, BN>::BYTES
    __shared__ __attribute__((aligned(1024))) char smem[LOOP > EPIB ? LOOP : EPIB];
    bf16* sA = reinterpret_cast<bf16*>(smem);
    bf16* sB = sA + 2 * kPpStage;
    gemm_pp_body<EPI, BN>(p, sA, sB, [&](const f32x16 (&acc)[kPpFM][T::FN], int m0, int tn, int wm, int wn, int lane) {
        if constexpr (VIA_LDS)
            pp_store_tile<EPI, BN>(p, acc, m0, tn, wm, wn, lane, reinterpret_cast<float*>(smem));
        else
            write_tile<EPI, BN, kPpTM, T::TN, kPpFM, T::FN>(p, acc, m0, tn, wm, wn, lane);
    });
}

// QKV projection on 256 x BN ping-pong tiles with the QK-norm + RoPE + cache write epilogue
// (same per-row work as gemm_qkv_qkrope_kernel).  A tile spans BN / 128 heads; per head, the
// waves whose columns lie in it put their fp32 accumulators into LDS (256 rows x 136 floats,
// over the stage buffers), then all 512 threads finish its 256 token rows.  With BN = 256 each
// wave column is one head (two passes), with BN = 128 the two wave columns are its halves.
constexpr int kPpQkTP = 128 + 8;
template <int BN>
__global__ __launch_bounds__(512) void gemm_qkv_qkrope_pp_kernel(DevGemm p, QkPpArgs a) {
    using T = PpTile<BN>;
    constexpr int TP = kPpQkTP, HPT = BN / 128;
    constexpr int LOOP = 2 * (kPpStage + T::B_ST) * 2;
    constexpr int SMEM = (kPpBM * TP * 4 > LOOP) ? kPpBM * TP * 4 : LOOP;
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];
    bf16* sA = reinterpret_cast<bf16*>(smem);
    bf16* sB = sA + 2 * kPpStage;
    gemm_pp_body<Epilogue::Store, BN>(p, sA, sB, [&](const f32x16 (&acc)[kPpFM][T::FN], int m0, int tn, int wm,
                                                     int wn, int lane) {
        float* tile = reinterpret_cast<float*>(smem);
        const int jl = threadIdx.x & 15, r0 = threadIdx.x >> 4;
        const int wh = (wn * T::TN) / 128, wc = (wn * T::TN) % 128;   // the wave's head and column in it
        constexpr int NR = kPpBM / 32;   // token rows per thread
        // the table entries serve every head of the tile: q and k heads rotate, k and v heads
        // go to the cache
        int Hq = a.Hq, Hkv = a.Hkv;
        asm("" : "+s"(Hq), "+s"(Hkv));
        const int h0 = HPT * tn, h1 = HPT * tn + HPT - 1;
        const bool need_cs = h0 < Hq + Hkv, need_slot = h1 >= Hq;
        RopeRow rr[NR];
#pragma unroll
        for (int k = 0; k < NR; ++k) rr[k] = rope_row_load(m0 + r0 + 32 * k, jl, need_cs, need_slot, p, a);
        __syncthreads();   // every wave is past its last LDS fragment read
#pragma unroll
        for (int hh = 0; hh < HPT; ++hh) {
            if (wh == hh) {
#pragma unroll
                for (int i = 0; i < kPpFM; ++i)
#pragma unroll
                    for (int j = 0; j < T::FN; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int row = wm * kPpTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                            tile[row * TP + wc + j * 32 + (lane & 31)] = acc[i][j][r];
                        }
            }
            __syncthreads();
            const int hs = HPT * tn + hh;
            float g[8];
            qkrope_gains(a, hs, jl, g);
#pragma unroll
            for (int k = 0; k < NR; ++k) {
                const int row = r0 + 32 * k;
                qkrope_row(tile + row * TP, jl, m0 + row, hs, g, p, a, rr[k]);
            }
            __syncthreads();   // the tile is rewritten by the next head's waves
        }
    });
}

// ------------------------------------------------------------------ thin products: deep ring
// Products with few output tiles (M x N of one to four million: the 0.6B-shaped o_proj and down at
// 2048 tokens) give each tile little matrix work per k stage.  Here 64 x 128 tiles (four waves of
// 32 x 64, one per SIMD) stream K through a ring of three 128-k stages loaded straight into LDS
// two stages ahead (96 KB in flight per CU), and the residual is added from the accumulators: K
// is not split, so there are no partial sums and no extra pass over them.  A stage is two 64-k
// halves of 128-byte rows, XOR-swizzled by (row >> 1) & 7 as in the ping-pong kernel; A rows past
// M read as zeros (one descriptor per 8-row group, covering its valid rows).  The first touch of
// each operand line on an XCD misses L2, so a stage still waits on memory: a deeper ring of
// 64-k stages (five in flight) was no faster, its extra barriers costing what the depth gained.
constexpr int kRgBM = 64, kRgBN = 128;
constexpr int kRgS = 3, kRgH = 2;                // ring slots; 64-k halves per stage
constexpr int kRgHalf = (kRgBM + kRgBN) * 64;   // elements of one 64-k half
constexpr int kRgSlot = kRgH * kRgHalf;          // elements of one stage

static bool ring_fits(int M, int N, int K) {
    if (M <= 64 || N % kRgBN || K % (64 * kRgH) || (int64_t)K * 2 * 8 >= ((int64_t)1 << 31)) return false;
    const long tiles = (long)((M + kRgBM - 1) / kRgBM) * (N / kRgBN);
    const long tiles128 = (long)((M + 127) / 128) * (N / 128);
    return tiles >= 128 && tiles128 < 256;
}

template <Epilogue EPI>
__global__ __launch_bounds__(256) void gemm_bf16_ring_kernel(DevGemm p) {
    static_assert(EPI == Epilogue::Store || EPI == Epilogue::ResidToF32 || EPI == Epilogue::ResidF32In,
                  "plain and residual epilogues");
    __shared__ __attribute__((aligned(1024))) bf16 smem[kRgS * kRgSlot];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    tile_of(p, blockIdx.x, tm, tn);
    const int m0 = tm * kRgBM;
    const int rowbytes = p.K * 2;

    // this wave's loads of each 64-k half: A groups 2w, 2w + 1 and B groups 4w .. 4w + 3 (8 rows each)
    int4v da[2], db[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r0 = m0 + 8 * (2 * wave + i);
        da[i] = sgpr_desc(p.a + (int64_t)min(r0, p.M - 1) * p.K, max(0, min(8, p.M - r0)) * rowbytes);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) db[j] = sgpr_desc(seg_row(p, tn * kRgBN + 8 * (4 * wave + j)), 8 * rowbytes);
    // lane l moves row l / 8 of its group into physical chunk l % 8 (logical chunk (l % 8) ^
    // swz8(row)); the swizzle depends on the parity of the group
    const int r8 = lane >> 3;
    const int voff_even = r8 * rowbytes + (((lane & 7) ^ swz8(r8)) << 4);
    const int voff_odd = r8 * rowbytes + (((lane & 7) ^ swz8(8 + r8)) << 4);
    const unsigned s_lds = (unsigned)(uintptr_t)(__attribute__((address_space(3))) bf16*)smem;
    // the 12 loads of stage st into ring slot `slot`; with live false the descriptors hold no
    // records (zeros, nothing fetched), so every stage issues the same count
    auto issue = [&](int st, int slot, bool live) {
#pragma unroll
        for (int hf = 0; hf < kRgH; ++hf) {
            const int soff = st * (128 * kRgH) + hf * 128;
            const unsigned base = s_lds + (unsigned)(slot * kRgSlot + hf * kRgHalf) * 2;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                int4v d = da[i];
                d[2] = live ? d[2] : 0;
                dma16(d, (i & 1) ? voff_odd : voff_even, soff,
                      __builtin_amdgcn_readfirstlane(base + (unsigned)(8 * (2 * wave + i) * 64) * 2));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int4v d = db[j];
                d[2] = live ? d[2] : 0;
                dma16(d, (j & 1) ? voff_odd : voff_even, soff,
                      __builtin_amdgcn_readfirstlane(base + (unsigned)((kRgBM + 8 * (4 * wave + j)) * 64) * 2));
            }
        }
    };

    // fragment of a 32-row block for 16-k step q of a half: row lane % 32, logical chunk
    // 2 q + lane / 32 (the block's base row is a multiple of 32, so the swizzle is swz8(lane % 32))
    const int fr = lane & 31;
    int rd[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) rd[q] = fr * 64 + (((2 * q + (lane >> 5)) ^ swz8(fr)) << 3);
    const int a_off = wm * 32 * 64, b_off = (kRgBM + wn * 64) * 64;

    f32x16 acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

    const int nst = p.K / (64 * kRgH);
#pragma unroll
    for (int i = 0; i < kRgS - 1; ++i) issue(i, i, i < nst);
    int slot = 0, slot_next = kRgS - 1;
    for (int t = 0; t < nst; ++t) {
        vm_wait<6 * kRgH * (kRgS - 2)>();   // this wave's loads of stage t have landed
        barrier_only();   // ... every wave's; and every wave is past its reads of stage t - 1
        const bf16* st = smem + slot * kRgSlot;
        // a half's 12 fragments are read together, the next half's over this half's MFMAs, so a
        // stage waits out one LDS round trip rather than one per 16-k step
        bf16x8 fa[kRgH][4], fb[kRgH][4][2];
        auto read_half = [&](int hf) {
            const bf16* h = st + hf * kRgHalf;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                fa[hf][q] = *reinterpret_cast<const bf16x8*>(h + a_off + rd[q]);
#pragma unroll
                for (int j = 0; j < 2; ++j) fb[hf][q][j] = *reinterpret_cast<const bf16x8*>(h + b_off + j * 32 * 64 + rd[q]);
            }
        };
        read_half(0);
        issue(t + kRgS - 1, slot_next, t + kRgS - 1 < nst);   // into the slot stage t - 1 used
#pragma unroll
        for (int hf = 0; hf < kRgH; ++hf) {
            __builtin_amdgcn_sched_barrier(0);
            if (hf + 1 < kRgH) read_half(hf + 1);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[hf][q], fb[hf][q][j], acc[j], 0, 0, 0);
            if (hf + 1 < kRgH) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (k < 6) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        slot = slot == kRgS - 1 ? 0 : slot + 1;
        slot_next = slot_next == kRgS - 1 ? 0 : slot_next + 1;
    }
    vm_wait<0>();   // the empty requests past the last stage

    // 32x32 accumulator layout: lane l, register r holds row 8 (r / 4) + 4 (l / 32) + r % 4, column
    // l % 32 of its block.  Every residual value is loaded before any output is stored, so the
    // loads share one memory round trip.
    const bool full = m0 + kRgBM <= p.M;
    const int row0 = m0 + wm * 32 + 4 * (lane >> 5);
    const int col0 = tn * kRgBN + wn * 64 + (lane & 31);
    if constexpr (EPI == Epilogue::Store) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = row0 + 8 * (r >> 2) + (r & 3);
            if (full || row < p.M) {
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    static_cast<bf16*>(p.out)[(int64_t)row * p.N + col0 + 32 * j] = (bf16)acc[j][r];
            }
        }
    } else {
        float rv[2][16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = min(row0 + 8 * (r >> 2) + (r & 3), p.M - 1);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t o = (int64_t)row * p.N + col0 + 32 * j;
                if constexpr (EPI == Epilogue::ResidToF32)
                    rv[j][r] = (float)static_cast<const bf16*>(p.resid)[o];
                else
                    rv[j][r] = static_cast<const float*>(p.resid)[o];
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = row0 + 8 * (r >> 2) + (r & 3);
            if (full || row < p.M) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int64_t o = (int64_t)row * p.N + col0 + 32 * j;
                    if constexpr (EPI == Epilogue::ResidToF32)
                        static_cast<float*>(p.out)[o] = rv[j][r] + acc[j][r];
                    else
                        static_cast<bf16*>(p.out)[o] = (bf16)(rv[j][r] + acc[j][r]);
                }
            }
        }
    }
}

// ------------------------------------------------------------------ skinny (M <= 64)
// Weight streaming for decode-sized M: a workgroup owns 16 output columns (16 weight rows, or 16
// gate and 16 up rows) over the whole K; its NW waves take interleaved 32-k chunks, so the
// workgroup reads its rows as runs of NW * 64 contiguous bytes.  The loop is software-pipelined
// D chunks deep: chunk i's loads are issued when chunk i - D is consumed, so a wave always has
// D chunks (D KB of weights per matrix) in flight instead of emptying its queue every few chunks;
// with one workgroup per CU that is what keeps HBM busy.
template <Epilogue EPI, int MG, int NW, int D>
__global__ __launch_bounds__(NW * 64) void gemv_bf16_kernel(DevGemm p) {
    constexpr bool DUAL = (EPI == Epilogue::SwiGLU);
    constexpr int NB = DUAL ? 2 : 1;
    __shared__ float red[NB][NW][MG][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 16;
    const int k0 = wave * 32 + 8 * (lane >> 4);
    const int niter = p.K / (32 * NW);   // the launcher checks that 32 NW divides K

    const bf16* brow[NB];
    if constexpr (DUAL) {
        brow[0] = p.b[0] + (int64_t)(n0 + (lane & 15)) * p.K + k0;
        brow[NB - 1] = p.b[1] + (int64_t)(n0 + (lane & 15)) * p.K + k0;
    } else {
        brow[0] = seg_row(p, n0 + (lane & 15)) + k0;
    }
    const bf16* arow[MG];
    bool avalid[MG];
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
        const int r = mg * 16 + (lane & 15);
        avalid[mg] = r < p.M;
        arow[mg] = p.a + (int64_t)min(r, p.M - 1) * p.K + k0;
    }

    f32x4 acc[NB][MG];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) acc[nb][mg] = f32x4{0.f, 0.f, 0.f, 0.f};

    bf16x8 bq[D][NB], aq[D][MG];
    auto issue = [&](int slot, int it) {
        const int64_t k = (int64_t)it * (32 * NW);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bq[slot][nb] = *reinterpret_cast<const bf16x8*>(brow[nb] + k);
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) aq[slot][mg] = *reinterpret_cast<const bf16x8*>(arow[mg] + k);
    };
    const bf16x8 zero = {};
    auto consume = [&](int slot) {
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) {
            const bf16x8 av = avalid[mg] ? aq[slot][mg] : zero;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc[nb][mg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bq[slot][nb], acc[nb][mg], 0, 0, 0);
        }
    };
    // niter is a multiple of D (the launcher picks D so): the steady loop has no tail tests, so
    // the compiler's wait before each chunk counts only the loads issued after that chunk's
    // instead of draining the queue at the loop head
#pragma unroll
    for (int i = 0; i < D; ++i) issue(i, i);
    for (int base = 0; base + D < niter; base += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            consume(i);
            issue(i, base + D + i);
            __builtin_amdgcn_sched_barrier(0);   // keep each refill right after its chunk's product
        }
    }
#pragma unroll
    for (int i = 0; i < D; ++i) consume(i);
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

// Skinny product for M <= 16 with whole-line weight loads.  In the MFMA operand layout a
// 16-column fragment is 16 rows x 64 bytes, so a load instruction that feeds the matrix core
// directly reads half of each of 16 cache lines, and the other halves come with another wave's
// instruction: every weight line crosses from L2 twice.  Here a wave reads its 16 (SwiGLU: 16
// gate and 16 up) weight rows over a 256-k stage as instructions of two rows x 512 contiguous
// bytes, puts them in its own LDS buffer (row pitch 528 bytes: the 16 rows of a fragment read
// fall on distinct banks) and reads the fragments back from there; no barrier is needed since
// a wave's LDS operations complete in order.  Waves take interleaved stages, D of them in
// flight per wave; the activations (16 rows) are read in the operand layout as before.
template <Epilogue EPI, int D>
__global__ __launch_bounds__(512) void gemv_lds_kernel(DevGemm p) {
    constexpr int NW = 8;
    constexpr bool DUAL = (EPI == Epilogue::SwiGLU);
    constexpr int NB = DUAL ? 2 : 1;
    constexpr int R = 16 * NB;            // weight rows of the workgroup
    constexpr int NI = R / 2;             // weight loads per stage
    constexpr int KS = 256;               // k per stage
    constexpr int PITCH = KS * 2 + 16;    // LDS row pitch, bytes
    __shared__ __attribute__((aligned(16))) char rows[NW][R * PITCH];
    __shared__ float red[NB][NW][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 16;
    const int niter = p.K / (KS * NW);   // a multiple of D (the launcher checks)

    // weight load i of a stage: tile rows 2i (lanes 0-31) and 2i+1 (lanes 32-63), 16 bytes a lane
    const bf16* wsrc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int r = 2 * i + (lane >> 5);
        const int n = n0 + (r & 15);
        const bf16* base;
        if constexpr (DUAL) base = p.b[r >> 4] + (int64_t)n * p.K;
        else base = seg_row(p, n);
        wsrc[i] = base + wave * KS + (lane & 31) * 8;
    }
    const bool avalid = (lane & 15) < p.M;
    const bf16* asrc = p.a + (int64_t)min(lane & 15, p.M - 1) * p.K + wave * KS + 8 * (lane >> 4);
    char* my = rows[wave];

    int4v wq[D][NI];
    bf16x8 aq[D][KS / 32];
    auto issue = [&](int slot, int it) {
        const int64_t k = (int64_t)it * (KS * NW);
#pragma unroll
        for (int i = 0; i < NI; ++i) wq[slot][i] = *reinterpret_cast<const int4v*>(wsrc[i] + k);
#pragma unroll
        for (int q = 0; q < KS / 32; ++q) aq[slot][q] = *reinterpret_cast<const bf16x8*>(asrc + k + 32 * q);
    };
    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16x8 zero = {};
    auto consume = [&](int slot) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
            *reinterpret_cast<int4v*>(my + (2 * i + (lane >> 5)) * PITCH + (lane & 31) * 16) = wq[slot][i];
#pragma unroll
        for (int q = 0; q < KS / 32; ++q) {
            const bf16x8 av = avalid ? aq[slot][q] : zero;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const bf16x8 bv =
                    *reinterpret_cast<const bf16x8*>(my + ((lane & 15) + 16 * nb) * PITCH + 64 * q + 16 * (lane >> 4));
                acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[nb], 0, 0, 0);
            }
        }
    };
#pragma unroll
    for (int i = 0; i < D; ++i) issue(i, i);
    for (int base = 0; base + D < niter; base += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            consume(i);
            issue(i, base + D + i);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int i = 0; i < D; ++i) consume(i);

    // 16x16 accumulator layout: lane l, register i holds row 4*(l/16) + i, column l%16
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[nb][wave][(4 * (lane >> 4) + i) * 16 + (lane & 15)] = acc[nb][i];
    __syncthreads();
    if (threadIdx.x < 256) {
        const int e = threadIdx.x;
        const int row = e >> 4, col = n0 + (e & 15);
        if (row < p.M) {
            float sum[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                sum[nb] = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) sum[nb] += red[nb][w][e];
            }
            if constexpr (DUAL) {
                static_cast<bf16*>(p.out)[(int64_t)row * p.N + col] = (bf16)silu_mul(sum[0], sum[NB - 1]);
            } else {
                epilogue_store<EPI>(p, row, col, sum[0]);
            }
        }
    }
}

// Split-K skinny product for M <= 16.  With 16 columns per workgroup every workgroup reads all of
// the activations, as many bytes as its weights, and those L2-resident loads take half of the
// vector-memory slots that should be keeping weight bytes in flight.  Here a unit is a column
// group of 16 CG outputs (16 CG weight rows) over one k slice of 32 NW NIT: each activation
// fragment feeds CG weight fragments, every load of the slice is issued before the first
// product, and the units still number several per CU.  Unit (group, slice) writes its fp32
// partial sums into slab `slice` of p.out ([kslices][M][N]); the kernel that consumes the
// projection adds the slabs in slice order (the split-K form of the prefill GEMMs, reduced the
// same way).
template <int CG, int NW, int NIT>
__global__ __launch_bounds__(NW * 64) void gemv_splitk_kernel(DevGemm p, int kslices) {
    constexpr int NT = NW * 64;
    constexpr int KL = 32 * NW * NIT;                // k slice
    constexpr int OUT = (CG * 256 + NT - 1) / NT;    // tile values per thread (the last may be idle)
    constexpr bool FULL = CG * 256 % NT == 0;
    __shared__ float red[NW][CG][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int group = (int)blockIdx.x / kslices, ks = (int)blockIdx.x % kslices;
    const int n0 = group * 16 * CG;
    const int kb = ks * KL + wave * 32 + 8 * (lane >> 4);

    const bf16* brow[CG];
#pragma unroll
    for (int c = 0; c < CG; ++c) brow[c] = seg_row(p, n0 + 16 * c + (lane & 15)) + kb;
    const bool avalid = (lane & 15) < p.M;
    const bf16* arow = p.a + (int64_t)min(lane & 15, p.M - 1) * p.K + kb;

    bf16x8 aq[NIT], bq[NIT][CG];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        aq[it] = *reinterpret_cast<const bf16x8*>(arow + it * 32 * NW);
#pragma unroll
        for (int c = 0; c < CG; ++c) bq[it][c] = *reinterpret_cast<const bf16x8*>(brow[c] + it * 32 * NW);
    }
    f32x4 acc[CG];
#pragma unroll
    for (int c = 0; c < CG; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16x8 zero = {};
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const bf16x8 av = avalid ? aq[it] : zero;
#pragma unroll
        for (int c = 0; c < CG; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bq[it][c], acc[c], 0, 0, 0);
    }
    // 16x16 accumulator layout: lane l, register i holds row 4*(l/16) + i, column l%16
#pragma unroll
    for (int c = 0; c < CG; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][c][(4 * (lane >> 4) + i) * 16 + (lane & 15)] = acc[c][i];
    __syncthreads();
    // thread t finishes values t + NT j of the tile: block (value / 256), row (value % 256) / 16,
    // column value % 16
    float* slab = static_cast<float*>(p.out) + (int64_t)ks * p.M * p.N;
#pragma unroll
    for (int j = 0; j < OUT; ++j) {
        const int idx = threadIdx.x + NT * j;
        if (!FULL && idx >= CG * 256) break;
        const int c = idx >> 8, e = idx & 255;
        const int row = e >> 4;
        if (row >= p.M) continue;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) v += red[w][c][e];
        slab[(int64_t)row * p.N + n0 + 16 * c + (e & 15)] = v;
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
    p.splits = g.splits > 1 ? g.splits : 1;
    return p;
}

template <Epilogue EPI, int MG, int NW>
void launch_gemv_depth(const DevGemm& p, unsigned grid, hipStream_t s) {
    const int niter = p.K / (32 * NW);
    if (niter % 8 == 0)
        gemv_bf16_kernel<EPI, MG, NW, 8><<<grid, NW * 64, 0, s>>>(p);
    else if (niter % 4 == 0)
        gemv_bf16_kernel<EPI, MG, NW, 4><<<grid, NW * 64, 0, s>>>(p);
    else if (niter % 2 == 0)
        gemv_bf16_kernel<EPI, MG, NW, 2><<<grid, NW * 64, 0, s>>>(p);
    else
        gemv_bf16_kernel<EPI, MG, NW, 1><<<grid, NW * 64, 0, s>>>(p);
}

template <Epilogue EPI, int MG>
hipError_t launch_gemv_mg(const DevGemm& p, hipStream_t s) {
    const unsigned grid = (unsigned)(p.N / 16);
    if (p.K <= 0 || p.N % 16) return hipErrorInvalidValue;
    if (p.K % (32 * 8) == 0)
        launch_gemv_depth<EPI, MG, 8>(p, grid, s);
    else if (p.K % (32 * 4) == 0)
        launch_gemv_depth<EPI, MG, 4>(p, grid, s);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <Epilogue EPI>
hipError_t launch_gemv_epi(const DevGemm& p, hipStream_t s) {
    if (p.M <= 16 && p.K > 0 && p.K % 2048 == 0 && p.N % 16 == 0) {   // whole-line weight loads
        const unsigned grid = (unsigned)(p.N / 16);
        // two stages in flight per wave; SwiGLU's 32 rows a stage leave registers for one
        if (EPI != Epilogue::SwiGLU && (p.K / 2048) % 2 == 0) gemv_lds_kernel<EPI, 2><<<grid, 512, 0, s>>>(p);
        else gemv_lds_kernel<EPI, 1><<<grid, 512, 0, s>>>(p);
        return hipGetLastError();
    }
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
    if (EPI != Epilogue::PartialF32) p.splits = 1;
    if (p.splits < 1 || p.N % bn_out || p.K % (BK * p.splits)) return hipErrorInvalidValue;
    p.tiles_m = (p.M + BM - 1) / BM;
    p.tiles_n = p.N / bn_out;
    gemm_bf16_kernel<EPI, BM, BN, WM, WN><<<(unsigned)(p.tiles_m * p.tiles_n * p.splits), WM * WN * 64, 0, s>>>(p);
    return hipGetLastError();
}

template <Epilogue EPI, int BN = 256>
static hipError_t run_pp_tile(DevGemm p, hipStream_t s) {
    const int bn_out = (EPI == Epilogue::SwiGLU) ? BN / 2 : BN;
    if (p.N % bn_out || p.K % 64 || (int64_t)p.K * 2 * 8 >= (int64_t)1 << 31) return hipErrorInvalidValue;
    p.tiles_m = (p.M + 255) / 256;
    p.tiles_n = p.N / bn_out;
    gemm_bf16_pp_kernel<EPI, BN><<<(unsigned)(p.tiles_m * p.tiles_n), 512, 0, s>>>(p);
    return hipGetLastError();
}

template <Epilogue EPI>
static hipError_t run_ring(DevGemm p, hipStream_t s) {
    if (!ring_fits(p.M, p.N, p.K)) return hipErrorInvalidValue;
    p.tiles_m = (p.M + kRgBM - 1) / kRgBM;
    p.tiles_n = p.N / kRgBN;
    gemm_bf16_ring_kernel<EPI><<<(unsigned)(p.tiles_m * p.tiles_n), 256, 0, s>>>(p);
    return hipGetLastError();
}

template <Epilogue EPI>
static hipError_t run_epi(const DevGemm& p, hipStream_t s) {
    // split-K partials, one fp32 slab per K range: 64 x 128 tiles, so the thin products that are
    // split (fewer than 256 tiles of 128 x 128) run two workgroups per CU (0.6B-shaped o_proj and
    // down: 1.9-4.4 us less per layer than on 128 x 128 tiles, one per CU; 64 x 64 was slower)
    if constexpr (EPI == Epilogue::PartialF32) return run_tile<EPI, 64, 128, 2, 2>(p, s);
    // The largest tile that still gives at least one workgroup per CU (256 CUs).
    constexpr bool DUAL = (EPI == Epilogue::SwiGLU);
    const int bn256 = DUAL ? 128 : 256, bn128 = DUAL ? 64 : 128;
    const long tiles256 = (long)((p.M + 255) / 256) * (p.N / bn256);
    const long tiles128 = (long)((p.M + 127) / 128) * (p.N / bn128);
    // 256 x 256 tiles: the ping-pong kernel (whole-line DMA, two 64-k stages), also taken with one
    // tile for only three CUs in four: its per-tile rate outweighs the idle quarter (2048 x 6144 x 1024 SwiGLU
    // product: 31.5 us against 38-40 us on 768 tiles of 128 x 128).
    if (tiles256 >= 192 && p.N % bn256 == 0 && p.K % 64 == 0) return run_pp_tile<EPI>(p, s);
    if (tiles128 >= 256) return run_tile<EPI, 128, 128, 2, 2>(p, s);
    // thin products (64 x 128 tiles, deep ring): the residual in the epilogue, K not split
    if constexpr (!DUAL && EPI != Epilogue::PartialF32)
        if (ring_fits(p.M, p.N, p.K)) return run_ring<EPI>(p, s);
    if constexpr (DUAL)
        return run_tile<EPI, 64, 128, 2, 2>(p, s);
    else
        return run_tile<EPI, 64, 64, 2, 2>(p, s);
}

// Which fused QKV kernel serves the projection g (0: none): 256 x 256 ping-pong tiles (2) when the
// generic launcher would take them, else 256 x 128 ping-pong tiles (3) when those give a
// workgroup per CU, else 128 x 128 register tiles (1); provided each head is a whole 128-column
// block and the RoPE is the plain rotate-half over the full head.
static int qkv_fused_kind(const GemmArgs& g, const QkRopeArgs& a) {
    if (g.epi != Epilogue::Store || g.M <= 64 || a.D != 128 || a.rotary_dim != 128 || a.adjacent || a.local.rolling)
        return 0;
    if (!a.rope_cs || !a.rope_slot || g.M != a.B * a.T) return 0;
    if (g.N != (a.Hq + 2 * a.Hkv) * 128 || g.K % BK || g.K % kPpK) return 0;
    const long tiles256 = (long)((g.M + 255) / 256) * (g.N / 256);
    const long tiles_pp128 = (long)((g.M + 255) / 256) * (g.N / 128);
    const long tiles128 = (long)((g.M + 127) / 128) * (g.N / 128);
    const bool dma_ok = (int64_t)g.K * 2 * 8 < ((int64_t)1 << 31);
    if (tiles256 >= 192 && g.N % 256 == 0) return dma_ok ? 2 : 0;
    if (tiles_pp128 >= 256 && dma_ok) return 3;
    return tiles128 >= 256 ? 1 : 0;
}

bool gemm_qkv_fusable(const GemmArgs& g, const QkRopeArgs& a) { return qkv_fused_kind(g, a) != 0; }

hipError_t launch_gemm_qkv_qkrope(const GemmArgs& g, const QkRopeArgs& a, hipStream_t s) {
    const int kind = qkv_fused_kind(g, a);
    if (kind == 0) return hipErrorInvalidValue;
    DevGemm p = make_dev(g);
    p.splits = 1;
    if (kind == 2) {
        p.tiles_m = (p.M + kPpBM - 1) / kPpBM;
        p.tiles_n = p.N / 256;
        const QkPpArgs pa{a.q_norm, a.k_norm, a.qhat, a.k_cache, a.v_cache, a.rope_cs, a.rope_slot,
                          a.T, a.Hq, a.Hkv, a.cap, a.eps, a.goff};
        gemm_qkv_qkrope_pp_kernel<256><<<(unsigned)(p.tiles_m * p.tiles_n), 512, 0, s>>>(p, pa);
    } else if (kind == 3) {
        p.tiles_m = (p.M + kPpBM - 1) / kPpBM;
        p.tiles_n = p.N / 128;
        const QkPpArgs pa{a.q_norm, a.k_norm, a.qhat, a.k_cache, a.v_cache, a.rope_cs, a.rope_slot,
                          a.T, a.Hq, a.Hkv, a.cap, a.eps, a.goff};
        gemm_qkv_qkrope_pp_kernel<128><<<(unsigned)(p.tiles_m * p.tiles_n), 512, 0, s>>>(p, pa);
    } else {
        p.tiles_m = (p.M + 127) / 128;
        p.tiles_n = p.N / 128;
        gemm_qkv_qkrope_kernel<<<(unsigned)(p.tiles_m * p.tiles_n), 256, 0, s>>>(p, a);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s) {
    if (g.M <= 0) return hipSuccess;
    const DevGemm p = make_dev(g);
    switch (g.epi) {
        case Epilogue::Store: return run_epi<Epilogue::Store>(p, s);
        case Epilogue::ResidToF32: return run_epi<Epilogue::ResidToF32>(p, s);
        case Epilogue::SwiGLU: return run_epi<Epilogue::SwiGLU>(p, s);
        case Epilogue::ResidF32In: return run_epi<Epilogue::ResidF32In>(p, s);
        case Epilogue::PartialF32: return run_epi<Epilogue::PartialF32>(p, s);
    }
    return hipErrorInvalidValue;
}

int gemm_bf16_splits(int M, int N, int K) {
    if (M <= 64 || N % 128 || K % (2 * BK) || K < 512 || ring_fits(M, N, K)) return 1;
    const long tiles128 = (long)((M + 127) / 128) * (N / 128);
    return tiles128 < 256 ? 2 : 1;
}

// Geometry of the split-K skinny product: column groups of 64 outputs and k slices of 1024 while
// that leaves at least kSkinnyUnits units, otherwise shorter slices, then narrower groups; no
// split (kslices 0) when no geometry divides the shape or one slice would cover K.
constexpr int kSkinnyUnits = 512;
SkinnyPlan skinny_plan(int M, int N, int K) {
    SkinnyPlan pl{};
    if (M <= 0 || M > 16 || K <= 0 || N <= 0) return pl;
    // candidates in order of preference: the first with kSkinnyUnits units, else the one with
    // the most
    int best_cg = 0, best_nit = 0;
    long best = 0;
    bool enough = false;
    for (int cg = 4; cg >= 1 && !enough; cg /= 2)
        for (int nit = 4; nit >= 1 && !enough; nit /= 2) {
            if (N % (16 * cg) || K % (256 * nit)) continue;
            const long units = (long)(N / (16 * cg)) * (K / (256 * nit));
            enough = units >= kSkinnyUnits;
            if (enough || units > best) {
                best = units;
                best_cg = cg;
                best_nit = nit;
            }
        }
    if (best == 0 || K / (256 * best_nit) < 2) return pl;
    pl.cg = best_cg;
    pl.nit = best_nit;
    pl.kslices = K / (256 * best_nit);
    pl.groups = N / (16 * best_cg);
    return pl;
}

template <int CG>
void launch_splitk_cg(const DevGemm& p, const SkinnyPlan& pl, hipStream_t s) {
    const unsigned grid = (unsigned)(pl.groups * pl.kslices);
    if (pl.nit == 4) gemv_splitk_kernel<CG, 8, 4><<<grid, 512, 0, s>>>(p, pl.kslices);
    else if (pl.nit == 2) gemv_splitk_kernel<CG, 8, 2><<<grid, 512, 0, s>>>(p, pl.kslices);
    else gemv_splitk_kernel<CG, 8, 1><<<grid, 512, 0, s>>>(p, pl.kslices);
}

hipError_t launch_gemv_bf16(const GemmArgs& g, hipStream_t s) {
    if (g.M <= 0) return hipSuccess;
    DevGemm p = make_dev(g);
    if (g.epi == Epilogue::PartialF32) {   // split-K slabs (M <= 16, skinny_plan's geometry)
        const SkinnyPlan pl = skinny_plan(g.M, g.N, g.K);
        if (pl.kslices < 2 || pl.kslices != g.splits) return hipErrorInvalidValue;
        if (pl.cg == 4) launch_splitk_cg<4>(p, pl, s);
        else if (pl.cg == 2) launch_splitk_cg<2>(p, pl, s);
        else launch_splitk_cg<1>(p, pl, s);
        return hipGetLastError();
    }
    switch (g.epi) {
        case Epilogue::Store: return launch_gemv_epi<Epilogue::Store>(p, s);
        case Epilogue::ResidToF32: return launch_gemv_epi<Epilogue::ResidToF32>(p, s);
        case Epilogue::SwiGLU: return launch_gemv_epi<Epilogue::SwiGLU>(p, s);
        case Epilogue::ResidF32In: return launch_gemv_epi<Epilogue::ResidF32In>(p, s);
        case Epilogue::PartialF32: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace q3
