// Per-head Q/K RMSNorm, rotate-half RoPE and the K/V cache write, in one pass over the
// projections.
//
// "17. A modern architecture: Qwen3", section Attention with grouped KV heads and Q/K
// normalization: q_norm / k_norm are RMSNorms over each head's D features, one gain shared
// by all heads, applied after the reshape to heads and before RoPE; V is neither normalised
// nor rotated.  Section Rotary position embeddings: omega_i = theta^(-2i/D), feature i is
// paired with feature i + D/2 and the pair is turned by p * omega_i; keys enter the cache
// already rotated.
//
// One 256-thread workgroup per token.  Lane l of a wave owns the rotate-half pair
// (l, l + D/2), so the rotation needs no data exchange; the pair's cos/sin are computed once
// per token from an angle formed in fp64 and reused for every head.  The four waves split the
// Hq + 2 Hkv heads of the token and issue all their loads before processing any head.
// The frequencies omega_i = theta^(-2i/D) come in fp64 (computed once per layer handle).
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
    const int pos = seq_pos(a.pos, b) + t;   // position == cache slot

    // cos / sin of p * omega_lane.  The angle is formed in fp64 in turns (p * omega / 2pi),
    // reduced exactly to [-1/2, 1/2] turn, and only then evaluated in fp32 on [-pi, pi].
    float c = 1.f, s = 0.f;
    if (active) {
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
                x0[i] = to_f32(src[hs * D + lane]);
                x1[i] = to_f32(src[hs * D + lane + half]);
            }
        }
#pragma unroll
        for (int i = 0; i < HB; ++i) {
            const int hs = hs0 + 4 * i;
            if (hs >= nheads) break;
            if (hs >= a.Hq + a.Hkv) {  // value head: copied to its cache slot unchanged
                const int kh = hs - a.Hq - a.Hkv;
                T* dst = static_cast<T*>(a.v_cache) + (((int64_t)b * a.Hkv + kh) * a.cap + pos) * D;
                if (active) {
                    dst[lane] = from_f32<T>(x0[i]);
                    dst[lane + half] = from_f32<T>(x1[i]);
                }
                continue;
            }
            const bool is_q = hs < a.Hq;
            const T* gain = static_cast<const T*>(is_q ? a.q_norm : a.k_norm);
            const float ss = wave_sum(x0[i] * x0[i] + x1[i] * x1[i]);
            const float rstd = rsqrtf(ss / (float)D + a.eps);
            if (!active) continue;
            const float n0 = to_f32(gain[lane]) * (x0[i] * rstd);
            const float n1 = to_f32(gain[lane + half]) * (x1[i] * rstd);
            const float r0 = n0 * c - n1 * s;
            const float r1 = n1 * c + n0 * s;
            T* dst;
            if (is_q) {
                dst = static_cast<T*>(a.qhat) + (((int64_t)b * a.Hq + hs) * a.T + t) * D;
            } else {
                const int kh = hs - a.Hq;
                dst = static_cast<T*>(a.k_cache) + (((int64_t)b * a.Hkv + kh) * a.cap + pos) * D;
            }
            dst[lane] = from_f32<T>(r0);
            dst[lane + half] = from_f32<T>(r1);
        }
    }
}

hipError_t launch_qknorm_rope(const QkRopeArgs& args, DType t, hipStream_t stream) {
    const int64_t tokens = (int64_t)args.B * args.T;
    if (tokens <= 0) return hipSuccess;
    if (args.D > 128 || (args.D & 1)) return hipErrorInvalidValue;
    if (t == DType::BF16)
        qknorm_rope_kernel<bf16><<<(unsigned)tokens, 256, 0, stream>>>(args);
    else
        qknorm_rope_kernel<float><<<(unsigned)tokens, 256, 0, stream>>>(args);
    return hipGetLastError();
}

}  // namespace q3
