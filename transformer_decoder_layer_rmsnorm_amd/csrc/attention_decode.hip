// Decode attention: one new query per sequence against a long cache of rotated keys, bf16,
// head_dim 128.  HBM-bound: every cached key and value is read exactly once per step and
// shared by the g query heads of its KV head ("lesson 6", section 3: each new token reads its
// own sequence's cache, which nobody shares; grouping makes each byte serve g heads).
//
// Split-KV: workgroup (split, kv head, sequence) takes 512 consecutive keys and produces, for
// each of the g heads, a partial output with its running max (base 2) and sum; a second kernel
// merges the splits.  Inside a workgroup each wave owns 128 keys.  A wave reads 4 whole key
// rows per load instruction (lane = 16-byte chunk l%16 of key l/16), so every access is a
// fully coalesced 1 KB; the per-key dot products are finished with a butterfly over the 16
// lanes of a key that also splits the g heads across those lanes (log2(g) fewer exchanges).
// Values are streamed the same way and accumulated per lane for its 8 features.
#include "common.hpp"
#include "kernels.hpp"

namespace q3 {

namespace {

constexpr int HD = 128;
constexpr int SK = kDecodeSplitKeys;  // keys per workgroup
constexpr int KPW = SK / 4;           // keys per wave

// Reduce s[0..G) over the 16 lanes sharing a key.  On return s[0] holds the full sum for head
// `head` (which depends on the lane), every head being held by 16/G of the lanes.
template <int G>
__device__ __forceinline__ float key_reduce(float (&s)[G], int lane, int& head) {
    int n = G;
    head = 0;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
        if (n > 1) {
            const bool hi = (lane & off) != 0;
            const int half = n >> 1;
#pragma unroll
            for (int i = 0; i < G / 2; ++i) {
                if (i < half) {
                    const float send = hi ? s[i] : s[i + half];
                    const float keep = hi ? s[i + half] : s[i];
                    s[i] = keep + __shfl_xor(send, off, 64);
                }
            }
            if (hi) head += half;
            n = half;
        } else {
            s[0] += __shfl_xor(s[0], off, 64);
        }
    }
    return s[0];
}

template <int G>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeAttnArgs p, float scale_log2) {
    static_assert(G >= 1 && G <= 16, "heads per KV head");
    __shared__ float sP[SK * G];          // [key][head]: scores, then probabilities
    __shared__ float sRed[4][G][HD];      // per-wave partial outputs
    __shared__ float sM[4][G], sL[4][G];  // per-wave running max (base 2) and sum

    const AttnArgs& a = p.a;
    const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kv_len = seq_pos(a.pos, b) + 1;
    const int key0 = split * SK;
    if (key0 >= kv_len) return;
    const int nk = min(SK, kv_len - key0);
    const int dc = lane & 15, ks = lane >> 4;

    float q[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        load8(static_cast<const bf16*>(a.qhat) + ((int64_t)b * a.Hq + kvh * G + h) * HD + 8 * dc, q[h]);
#pragma unroll
        for (int e = 0; e < 8; ++e) q[h][e] *= scale_log2;
    }
    const int64_t base = (((int64_t)b * a.Hkv + kvh) * a.cap + key0) * HD + 8 * dc;
    const bf16* kg = static_cast<const bf16*>(a.k_cache) + base;
    const bf16* vg = static_cast<const bf16*>(a.v_cache) + base;

    // ---- scores for this wave's keys
#pragma unroll 4
    for (int i = 0; i < KPW / 4; ++i) {
        const int kk = wave * KPW + 4 * i + ks;
        float kv[8];
        load8(kg + (int64_t)min(kk, nk - 1) * HD, kv);
        float s[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf(q[h][e], kv[e], acc);
            s[h] = acc;
        }
        int head;
        const float sum = key_reduce<G>(s, lane, head);
        if ((dc & ((16 / G) - 1)) == 0) sP[kk * G + head] = kk < nk ? sum : -INFINITY;
    }
    __syncthreads();

    // ---- per-wave softmax statistics over its 128 keys
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const int k1 = wave * KPW + lane, k2 = k1 + 64;
        const float s1 = sP[k1 * G + h], s2 = sP[k2 * G + h];
        const float m = wave_max(fmaxf(s1, s2));
        const float mref = (m == -INFINITY) ? 0.f : m;
        const float p1 = fast_exp2(s1 - mref), p2 = fast_exp2(s2 - mref);
        sP[k1 * G + h] = p1;
        sP[k2 * G + h] = p2;
        const float l = wave_sum(p1 + p2);
        if (lane == 0) {
            sM[wave][h] = m;
            sL[wave][h] = l;
        }
    }
    __syncthreads();

    // ---- partial output: lane accumulates its 8 features over keys ks, ks+4, ...
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll 4
    for (int i = 0; i < KPW / 4; ++i) {
        const int kk = wave * KPW + 4 * i + ks;
        float vv[8];
        load8(vg + (int64_t)min(kk, nk - 1) * HD, vv);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float pr = sP[kk * G + h];   // 0 for keys beyond the cache
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pr, vv[e], acc[h][e]);
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[h][e] += __shfl_xor(acc[h][e], 16, 64);
            acc[h][e] += __shfl_xor(acc[h][e], 32, 64);
        }
    if (ks == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) sRed[wave][h][8 * dc + e] = acc[h][e];
    }
    __syncthreads();

    // ---- merge the four waves and write this split's partials
    const int S = p.splits;
    for (int idx = threadIdx.x; idx < G * HD; idx += 256) {
        const int h = idx / HD, d = idx % HD;
        float m = sM[0][h];
#pragma unroll
        for (int w = 1; w < 4; ++w) m = fmaxf(m, sM[w][h]);
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            if (sM[w][h] != -INFINITY) o += sRed[w][h][d] * fast_exp2(sM[w][h] - m);
        const int64_t row = ((int64_t)b * a.Hq + kvh * G + h) * S + split;
        p.part_o[row * HD + d] = o;
        if (d == 0) {
            float l = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                if (sM[w][h] != -INFINITY) l += sL[w][h] * fast_exp2(sM[w][h] - m);
            p.part_ml[row * 2] = m;
            p.part_ml[row * 2 + 1] = l;
        }
    }
}

__global__ __launch_bounds__(HD) void decode_combine_kernel(DecodeAttnArgs p) {
    const AttnArgs& a = p.a;
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int kv_len = seq_pos(a.pos, b) + 1;
    const int ns = (kv_len + SK - 1) / SK;
    const int64_t row0 = ((int64_t)b * a.Hq + h) * p.splits;
    float m = -INFINITY;
    for (int s = 0; s < ns; ++s) m = fmaxf(m, p.part_ml[(row0 + s) * 2]);
    float l = 0.f, o = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float w = fast_exp2(p.part_ml[(row0 + s) * 2] - m);
        l += p.part_ml[(row0 + s) * 2 + 1] * w;
        o += p.part_o[(row0 + s) * HD + d] * w;
    }
    static_cast<bf16*>(a.out)[(int64_t)b * a.Hq * HD + (int64_t)h * HD + d] = (bf16)(o / l);
}

template <int G>
hipError_t launch_g(const DecodeAttnArgs& p, float scale_log2, hipStream_t s) {
    const dim3 grid((unsigned)p.splits, (unsigned)p.a.Hkv, (unsigned)p.a.B);
    decode_split_kernel<G><<<grid, 256, 0, s>>>(p, scale_log2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_decode_split_bf16(const DecodeAttnArgs& p, hipStream_t stream) {
    const AttnArgs& a = p.a;
    if (a.D != HD || a.T != 1 || a.Hkv <= 0 || a.Hq % a.Hkv || p.split_keys != SK) return hipErrorInvalidValue;
    if (a.B <= 0) return hipSuccess;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    switch (a.Hq / a.Hkv) {
        case 1: return launch_g<1>(p, scale_log2, stream);
        case 2: return launch_g<2>(p, scale_log2, stream);
        case 4: return launch_g<4>(p, scale_log2, stream);
        case 8: return launch_g<8>(p, scale_log2, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attention_decode_combine_bf16(const DecodeAttnArgs& p, hipStream_t stream) {
    const AttnArgs& a = p.a;
    if (a.D != HD || a.T != 1) return hipErrorInvalidValue;
    if (a.B <= 0) return hipSuccess;
    decode_combine_kernel<<<dim3((unsigned)a.Hq, (unsigned)a.B), HD, 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace q3
