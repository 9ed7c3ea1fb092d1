// Causal grouped-query attention for prefill, head_dim 128, bf16 operands on gfx950 matrix
// cores with an fp32 online softmax.
//
// What it computes ("Transformer architectures: from BERT to diffusion, lesson 6", section 3;
// "17. A modern architecture: Qwen3", section Attention with grouped KV heads and Q/K
// normalization): for query head h and KV head floor(h / g), g = Hq / Hkv,
//   o_i = sum_{j : pos_j <= pos_i} softmax_j(q_i . k_j / sqrt(D)) v_j.
// The score matrix is never written out: keys and values stream through LDS in tiles of 64 and
// the softmax is accumulated online (running max and sum per query, rescaling the output).
//
// Layout choices for CDNA4:
//  * A workgroup (4 waves) serves several query heads of ONE KV head (up to 4), so each K/V
//    tile staged in LDS is read by every head of its group (the fused-kernel point of the GQA
//    section: one read of a shared KV head serves g query heads).  Each wave owns 32 queries of
//    one head.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: in the 32x32
//    accumulator a lane holds 16 keys of ONE query (column = lane % 32), so the row max and
//    sum of the softmax are per-lane reductions plus one exchange with lane ^ 32.
//  * The probabilities stay in registers and feed O^T += V^T P^T directly as the B operand.
//    V^T is produced while staging V into LDS (4 keys x 8 dims per thread, packed into 8-byte
//    cells), with a cell swizzle that keeps both the transposed stores and the fragment reads
//    free of bank conflicts.
//  * K rows in LDS are 256 bytes with the 16-byte chunk index XOR-swizzled by the key.
//  * Tiles above the diagonal are never visited; per wave, 32-key blocks that lie entirely
//    above its queries skip their MFMAs.  The heaviest query tiles are dispatched first.
#include "common.hpp"
#include "kernels.hpp"

namespace q3 {

namespace {

constexpr int HD = 128;  // head_dim
constexpr int KT = 64;   // keys per tile

__device__ __forceinline__ int k_off(int key, int chunk) { return key * HD + ((chunk ^ (key & 7)) << 3); }
__device__ __forceinline__ int vt_off(int d, int cell) {
    return d * KT + ((cell ^ ((d & 15) ^ ((d >> 3) & 15))) << 2);
}

template <int HPW>
__global__ __launch_bounds__(256) void flash_prefill_kernel(AttnArgs a, float scale_log2) {
    constexpr int WPH = 4 / HPW;       // waves per head
    constexpr int QB = 32 * WPH;       // queries per workgroup
    __shared__ __attribute__((aligned(16))) bf16 sK[2][KT * HD];
    __shared__ __attribute__((aligned(16))) bf16 sV[2][HD * KT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = a.Hq / a.Hkv;
    const int subs = g / HPW;
    const int kvh = blockIdx.y / subs;
    const int h = kvh * g + (blockIdx.y % subs) * HPW + wave / WPH;
    const int b = blockIdx.z;
    const int nqt = (a.T + QB - 1) / QB;
    const int q0 = (nqt - 1 - (int)blockIdx.x) * QB;
    const int qw = q0 + (wave % WPH) * 32;          // first query index of this wave
    const int pos0 = seq_pos(a.pos, b);
    const int kv_len = pos0 + min(q0 + QB, a.T);    // keys 0 .. last query position of the group
    const int ntiles = (kv_len + KT - 1) / KT;
    const int my_pos = pos0 + qw + (lane & 31);
    const int wave_first = pos0 + qw;
    const int wave_last = pos0 + min(qw + 31, a.T - 1);

    // Q^T fragments (B operand): query qw + lane%32, d chunk 2s + lane/32.
    bf16x8 qf[8];
    {
        const bf16* qrow = static_cast<const bf16*>(a.qhat) +
                           (((int64_t)b * a.Hq + h) * a.T + min(qw + (lane & 31), a.T - 1)) * HD;
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + (2 * s + (lane >> 5)) * 8);
    }

    const int64_t kv_base = ((int64_t)b * a.Hkv + kvh) * a.cap * HD;
    const bf16* kg = static_cast<const bf16*>(a.k_cache) + kv_base;
    const bf16* vg = static_cast<const bf16*>(a.v_cache) + kv_base;

    bf16x8 rk[4], rv[4];
    auto gload = [&](int kt) {
        const int k0 = kt * KT;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = tid + 256 * j;
            const int key = min(k0 + (c >> 4), kv_len - 1);
            rk[j] = *reinterpret_cast<const bf16x8*>(kg + (int64_t)key * HD + (c & 15) * 8);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = min(k0 + (tid >> 4) * 4 + i, kv_len - 1);
            rv[i] = *reinterpret_cast<const bf16x8*>(vg + (int64_t)key * HD + (tid & 15) * 8);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = tid + 256 * j;
            *reinterpret_cast<bf16x8*>(&sK[buf][k_off(c >> 4, c & 15)]) = rk[j];
        }
        const int cell = tid >> 4, dc = tid & 15;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16x4 v4 = {rv[0][e], rv[1][e], rv[2][e], rv[3][e]};
            *reinterpret_cast<bf16x4*>(&sV[buf][vt_off(dc * 8 + e, cell)]) = v4;
        }
    };

    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    float m_run = -1e30f, l_run = 0.f;

    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < ntiles) gload(kt + 1);
        const int k0 = kt * KT;

        // ---- S^T for the two 32-key blocks of the tile
        f32x16 sacc[2];
        bool live[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            live[kb] = (k0 + kb * 32) <= wave_last;
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
            if (live[kb]) {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
                        &sK[buf][k_off(kb * 32 + (lane & 31), 2 * s + (lane >> 5))]);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[kb], 0, 0, 0);
                }
            }
        }
        // ---- causal mask (only tiles reaching past the wave's first query)
        if (k0 + KT - 1 > wave_first) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (!live[kb] || key > my_pos) sacc[kb][r] = -INFINITY;
                }
        }
        // ---- online softmax in base 2
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_run, mt * scale_log2);
        const float corr = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= corr;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= corr;

        bf16x8 pf[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float pv = fast_exp2(fmaf(sacc[kb][8 * hf + j], scale_log2, -m_new));
                    l_run += pv;
                    pf[kb][hf][j] = (bf16)pv;
                }

        // ---- O^T += V^T P^T ; key of element j of lane group q: 16hf + 8(j/4) + 4q + j%4
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (!live[kb]) continue;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int cell0 = kb * 8 + hf * 4 + (lane >> 5);
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const int d = db * 32 + (lane & 31);
                    const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(&sV[buf][vt_off(d, cell0)]);
                    const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(&sV[buf][vt_off(d, cell0 + 2)]);
                    const bf16x8 vf = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][hf], o[db], 0, 0, 0);
                }
            }
        }
        if (kt + 1 < ntiles) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- normalise and store: lane holds d = db*32 + 8(r/4) + 4(lane/32) + r%4 of its query
    const float inv = 1.0f / (l_run + __shfl_xor(l_run, 32, 64));
    const int q = qw + (lane & 31);
    if (q < a.T) {
        bf16* orow = static_cast<bf16*>(a.out) + ((int64_t)b * a.T + q) * a.Hq * HD + (int64_t)h * HD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                bf16x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = (bf16)(o[db][4 * rq + e] * inv);
                *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * rq + 4 * (lane >> 5)) = v4;
            }
    }
}

}  // namespace

hipError_t launch_attention_prefill_bf16(const AttnArgs& a, hipStream_t stream) {
    if (a.D != HD || a.Hkv <= 0 || a.Hq % a.Hkv) return hipErrorInvalidValue;
    if (a.B <= 0 || a.T <= 0) return hipSuccess;
    const int g = a.Hq / a.Hkv;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const int hpw = (g % 4 == 0) ? 4 : (g % 2 == 0) ? 2 : 1;
    const int qb = 32 * (4 / hpw);
    const dim3 grid((unsigned)((a.T + qb - 1) / qb), (unsigned)(a.Hkv * (g / hpw)), (unsigned)a.B);
    if (hpw == 4)
        flash_prefill_kernel<4><<<grid, 256, 0, stream>>>(a, scale_log2);
    else if (hpw == 2)
        flash_prefill_kernel<2><<<grid, 256, 0, stream>>>(a, scale_log2);
    else
        flash_prefill_kernel<1><<<grid, 256, 0, stream>>>(a, scale_log2);
    return hipGetLastError();
}

}  // namespace q3
