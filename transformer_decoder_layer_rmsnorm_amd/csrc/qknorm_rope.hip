// Per-head Q/K RMSNorm, rotate-half RoPE and the K/V cache write, in one pass over the
// projections.
//
// "17. A modern architecture: Qwen3", section Attention with grouped KV heads and Q/K
// normalization: q_norm / k_norm are RMSNorms over each head's D features, one gain shared
// by all heads, applied after the reshape to heads and before RoPE; V is neither normalised
// nor rotated.  Section Rotary position embeddings: omega_i = theta^(-2i/D), feature i is
// paired with feature i + D/2 and the pair is turned by p * omega_i; keys enter the cache
// already rotated.  The token's cache slot and its position differ for left-padded batches
// ("lesson 6", section 8: positions count a row's real tokens) and for rolling-buffer caches of
// local layers (section 7: the token overwrites the one that just left the window).
//
// One 256-thread workgroup per token; the cos/sin of each rotation pair are computed once per
// token from an angle formed in fp64 (p * omega_i / 2pi, reduced exactly to [-1/2, 1/2] turn,
// then evaluated in fp32) and reused for every head.  The frequencies omega_i = theta^(-2i/D)
// come in fp64, computed once per layer handle.
//
// bf16, D = 128: 16 lanes per head, four heads per wave instruction.  Lane j of a head owns
// features 4j..4j+3 and their rotation partners 64+4j..64+4j+3 (8-byte loads and stores, the
// rotation stays inside the lane) and the head's sum of squares is a 16-lane DPP reduction.
// Other shapes and the RoPE variants (partial rotation of the first rotary_dim features,
// "apply_rope rotates only the first cos.shape[-1] features"; adjacent pairs (2i, 2i+1), the
// original paper's convention; linear position scaling, folded into the frequency table;
// zero-centred gains 1 + g): lane l of a wave owns one rotation pair, one head per wave at a
// time.
#include "common.hpp"
#include "kernels.hpp"

namespace q3 {

template <typename T>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(QkRopeArgs a) {
    const int tok = blockIdx.x;            // 0 .. B*T-1
    const int b = tok / a.T;
    const int t = tok - b * a.T;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int D = a.D;
    const int half = D >> 1;
    const bool active = lane < half;
    const int lin = seq_pos(a.pos, b) + t;   // cache slot of the token in a linear cache
    int pad_lo, pad_hi;
    seq_pad(a.pos, b, pad_lo, pad_hi);
    const int pos = slot_position(lin, pad_lo, pad_hi);    // RoPE position (real tokens before it)
    const int slot = a.local.rolling ? rolling_slot(a.local, pos) : lin;

    // Lane l (< D/2) owns two features f0, f1: rotation pair l when l < rotary_dim/2 - (l, l + r/2)
    // split-half or (2l, 2l+1) adjacent - and otherwise two features past rotary_dim, which are
    // normalised but not rotated (partial RoPE).
    const int rh = a.rotary_dim >> 1;
    const bool rotates = lane < rh;
    const int f0 = rotates ? (a.adjacent ? 2 * lane : lane) : a.rotary_dim + 2 * (lane - rh);
    const int f1 = rotates ? (a.adjacent ? 2 * lane + 1 : lane + rh) : f0 + 1;

    // cos / sin of p * omega_lane.  The angle is formed in fp64 in turns (p * omega / 2pi),
    // reduced exactly to [-1/2, 1/2] turn, and only then evaluated in fp32 on [-pi, pi].
    float c = 1.f, s = 0.f;
    if (active && rotates) {
        const double turns = (double)pos * a.turns[lane];
        const float r = (float)(turns - rint(turns)) * 6.283185307179586f;
        sincosf(r, &s, &c);
    }

    const T* src = static_cast<const T*>(a.qkv) + (int64_t)tok * (a.Hq + 2 * a.Hkv) * D;
    const int nheads = a.Hq + 2 * a.Hkv;
    // The wave's heads are wave, wave + 4, ...; loads for HB of them are issued before any is
    // processed, so their latencies overlap instead of adding up.
    constexpr int HB = 8;
    for (int hs0 = wave; hs0 < nheads; hs0 += 4 * HB) {
        float x0[HB], x1[HB];
#pragma unroll
        for (int i = 0; i < HB; ++i) {
            const int hs = hs0 + 4 * i;
            x0[i] = x1[i] = 0.f;
            if (active && hs < nheads) {
                x0[i] = to_f32(src[hs * D + f0]);
                x1[i] = to_f32(src[hs * D + f1]);
            }
        }
#pragma unroll
        for (int i = 0; i < HB; ++i) {
            const int hs = hs0 + 4 * i;
            if (hs >= nheads) break;
            if (hs >= a.Hq + a.Hkv) {  // value head: copied to its cache slot unchanged
                const int kh = hs - a.Hq - a.Hkv;
                T* dst = static_cast<T*>(a.v_cache) + (((int64_t)b * a.Hkv + kh) * a.cap + slot) * D;
                if (active) {
                    dst[f0] = from_f32<T>(x0[i]);
                    dst[f1] = from_f32<T>(x1[i]);
                }
                continue;
            }
            const bool is_q = hs < a.Hq;
            const T* gain = static_cast<const T*>(is_q ? a.q_norm : a.k_norm);
            const float ss = wave_sum(x0[i] * x0[i] + x1[i] * x1[i]);
            const float rstd = rsqrtf(ss / (float)D + a.eps);
            if (!active) continue;
            const float n0 = (a.goff + to_f32(gain[f0])) * (x0[i] * rstd);
            const float n1 = (a.goff + to_f32(gain[f1])) * (x1[i] * rstd);
            const float r0 = n0 * c - n1 * s;
            const float r1 = n1 * c + n0 * s;
            T* dst;
            if (is_q) {
                dst = static_cast<T*>(a.qhat) + (((int64_t)b * a.Hq + hs) * a.T + t) * D;
            } else {
                const int kh = hs - a.Hq;
                dst = static_cast<T*>(a.k_cache) + (((int64_t)b * a.Hkv + kh) * a.cap + slot) * D;
            }
            dst[f0] = from_f32<T>(r0);
            dst[f1] = from_f32<T>(r1);
        }
    }
}


template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// Sum over each 16-lane row of the wave, result in every lane of the row (DPP, no LDS).
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f32<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_f32<0x141>(v);   // row_half_mirror: the other quad of the half row
    v += dpp_f32<0x140>(v);   // row_mirror: the other half row
    return v;
}

// PART: the projections arrive as a.qkv_splits fp32 slabs (split-K skinny QKV), summed in slab
// order, rounded to bf16 and also stored to a.qkv_sum here.
template <bool PART>
__global__ __launch_bounds__(256) void qknorm_rope_d128_bf16(QkRopeArgs a) {
    constexpr int D = 128;
    const int tok = blockIdx.x;
    const int b = tok / a.T;
    const int t = tok - b * a.T;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slot = lane >> 4;          // head slot within a group of four heads
    const int j = lane & 15;             // features 4j..4j+3 and 64+4j..64+4j+3
    const int lin = seq_pos(a.pos, b) + t;     // cache slot of the token in a linear cache
    int pad_lo, pad_hi;
    seq_pad(a.pos, b, pad_lo, pad_hi);
    const int pos = slot_position(lin, pad_lo, pad_hi);
    const int cslot = a.local.rolling ? rolling_slot(a.local, pos) : lin;

    float cs[4], sn[4], gq[8], gk[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // v_sin_f32 / v_cos_f32 take the angle in turns; the fp64 turn count is reduced
        // exactly to [-1/2, 1/2] first
        const double turns = (double)pos * a.turns[4 * j + e];
        const float r = (float)(turns - rint(turns));
        sn[e] = __builtin_amdgcn_sinf(r);
        cs[e] = __builtin_amdgcn_cosf(r);
    }
    {
        const bf16x4 q0 = *reinterpret_cast<const bf16x4*>(static_cast<const bf16*>(a.q_norm) + 4 * j);
        const bf16x4 q1 = *reinterpret_cast<const bf16x4*>(static_cast<const bf16*>(a.q_norm) + 64 + 4 * j);
        const bf16x4 k0 = *reinterpret_cast<const bf16x4*>(static_cast<const bf16*>(a.k_norm) + 4 * j);
        const bf16x4 k1 = *reinterpret_cast<const bf16x4*>(static_cast<const bf16*>(a.k_norm) + 64 + 4 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            gq[e] = a.goff + (float)q0[e]; gq[4 + e] = a.goff + (float)q1[e];
            gk[e] = a.goff + (float)k0[e]; gk[4 + e] = a.goff + (float)k1[e];
        }
    }

    const int nheads = a.Hq + 2 * a.Hkv;
    const int ngroups = (nheads + 3) >> 2;
    const bf16* src = static_cast<const bf16*>(a.qkv) + (int64_t)tok * nheads * D + 4 * j;
    bf16* q_dst = static_cast<bf16*>(a.qhat) + ((int64_t)b * a.Hq * a.T + t) * D + 4 * j;
    bf16* k_dst = static_cast<bf16*>(a.k_cache) + ((int64_t)b * a.Hkv * a.cap + cslot) * D + 4 * j;
    bf16* v_dst = static_cast<bf16*>(a.v_cache) + ((int64_t)b * a.Hkv * a.cap + cslot) * D + 4 * j;
    const int64_t q_stride = (int64_t)a.T * D, kv_stride = (int64_t)a.cap * D;

    // Groups of four heads: workgroup y of the token takes groups 4 y + wave + gs i (gs = 4 x the
    // workgroups per token); loads for GB of them are issued first.  The slab form runs one group
    // per wave (gridDim.y covers them) so that all of its slab loads are in flight at once.
    constexpr int GB = PART ? 1 : 4;
    const int gs = 4 * (int)gridDim.y;
    for (int g0 = 4 * (int)blockIdx.y + wave; g0 < ngroups; g0 += gs * GB) {
        bf16x4 lo[GB], hi[GB];
        if constexpr (PART) {
            const float* psrc = a.qkv_part + (int64_t)tok * nheads * D + 4 * j;
            const int64_t slab = (int64_t)a.B * a.T * nheads * D;
            f32x4 slo[GB], shi[GB];
#pragma unroll
            for (int i = 0; i < GB; ++i) slo[i] = shi[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            // eight slabs' loads are issued before their sums (in slab order)
            constexpr int SU = 8;
            for (int sp0 = 0; sp0 < a.qkv_splits; sp0 += SU) {
                f32x4 plo[SU][GB], phi[SU][GB];
#pragma unroll
                for (int u = 0; u < SU; ++u)
#pragma unroll
                    for (int i = 0; i < GB; ++i) {
                        const int h = min(4 * (g0 + gs * i) + slot, nheads - 1);
                        const int sp = min(sp0 + u, a.qkv_splits - 1);
                        plo[u][i] = *reinterpret_cast<const f32x4*>(psrc + sp * slab + h * D);
                        phi[u][i] = *reinterpret_cast<const f32x4*>(psrc + sp * slab + h * D + 64);
                    }
#pragma unroll
                for (int u = 0; u < SU; ++u)
                    if (sp0 + u < a.qkv_splits) {
#pragma unroll
                        for (int i = 0; i < GB; ++i) {
                            slo[i] += plo[u][i];
                            shi[i] += phi[u][i];
                        }
                    }
            }
            bf16* sum = static_cast<bf16*>(a.qkv_sum) + (int64_t)tok * nheads * D + 4 * j;
#pragma unroll
            for (int i = 0; i < GB; ++i) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo[i][e] = (bf16)slo[i][e];
                    hi[i][e] = (bf16)shi[i][e];
                }
                if (g0 + gs * i < ngroups && 4 * (g0 + gs * i) + slot < nheads) {
                    const int h = 4 * (g0 + gs * i) + slot;
                    *reinterpret_cast<bf16x4*>(sum + h * D) = lo[i];
                    *reinterpret_cast<bf16x4*>(sum + h * D + 64) = hi[i];
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < GB; ++i) {
                const int h = min(4 * (g0 + gs * i) + slot, nheads - 1);
                lo[i] = *reinterpret_cast<const bf16x4*>(src + h * D);
                hi[i] = *reinterpret_cast<const bf16x4*>(src + h * D + 64);
            }
        }
#pragma unroll
        for (int i = 0; i < GB; ++i) {
            if (g0 + gs * i >= ngroups) break;    // uniform across the wave
            const int h = 4 * (g0 + gs * i) + slot;
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) { x[e] = (float)lo[i][e]; x[4 + e] = (float)hi[i][e]; }
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
            const float rstd = rsqrtf(row16_sum(ss) * (1.0f / D) + a.eps);
            if (h >= nheads) continue;
            bf16x4 olo, ohi;
            bf16* dst;
            if (h >= a.Hq + a.Hkv) {          // value head: copied to its cache slot unchanged
                olo = lo[i];
                ohi = hi[i];
                dst = v_dst + (h - a.Hq - a.Hkv) * kv_stride;
            } else {
                const bool is_q = h < a.Hq;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float n0 = (is_q ? gq[e] : gk[e]) * (x[e] * rstd);
                    const float n1 = (is_q ? gq[4 + e] : gk[4 + e]) * (x[4 + e] * rstd);
                    olo[e] = (bf16)(n0 * cs[e] - n1 * sn[e]);
                    ohi[e] = (bf16)(n1 * cs[e] + n0 * sn[e]);
                }
                dst = is_q ? q_dst + h * q_stride : k_dst + (h - a.Hq) * kv_stride;
            }
            *reinterpret_cast<bf16x4*>(dst) = olo;
            *reinterpret_cast<bf16x4*>(dst + 64) = ohi;
        }
    }
}

hipError_t launch_qknorm_rope(const QkRopeArgs& args, DType t, hipStream_t stream) {
    const int64_t tokens = (int64_t)args.B * args.T;
    if (tokens <= 0) return hipSuccess;
    if (args.D > 128 || (args.D & 1)) return hipErrorInvalidValue;
    if (args.rotary_dim > args.D || (args.rotary_dim & 1) || args.rotary_dim < 0) return hipErrorInvalidValue;
    // the vectorised kernel covers the Qwen3 layout (all 128 features rotated, split-half pairs)
    const bool d128 = t == DType::BF16 && args.D == 128 && args.rotary_dim == 128 && !args.adjacent;
    if (args.qkv_splits > 0) {
        if (!d128 || !args.qkv_part || !args.qkv_sum) return hipErrorInvalidValue;
        const int ngroups = (args.Hq + 2 * args.Hkv + 3) / 4;
        qknorm_rope_d128_bf16<true><<<dim3((unsigned)tokens, (unsigned)((ngroups + 3) / 4)), 256, 0, stream>>>(args);
    } else if (d128)
        qknorm_rope_d128_bf16<false><<<(unsigned)tokens, 256, 0, stream>>>(args);
    else if (t == DType::BF16)
        qknorm_rope_kernel<bf16><<<(unsigned)tokens, 256, 0, stream>>>(args);
    else
        qknorm_rope_kernel<float><<<(unsigned)tokens, 256, 0, stream>>>(args);
    return hipGetLastError();
}

}  // namespace q3
