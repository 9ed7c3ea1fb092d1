// Decode attention: one new query per sequence against a long cache of rotated keys, bf16,
// head_dim 128.  HBM-bound: every cached key and value is read exactly once per step and
// shared by the g query heads of its KV head ("lesson 6", section 3: each new token reads its
// own sequence's cache, which nobody shares; grouping makes each byte serve g heads).
//
// Split-KV: workgroup (split, kv head, sequence) takes kDecodeSplitKeys (1024) consecutive keys
// and produces, for each of the g heads, a partial output with its running max (base 2) and sum;
// a second kernel merges the splits.  Inside a workgroup each wave owns a quarter of the keys.  A wave reads 4 whole key
// rows per load instruction (lane = 16-byte chunk l%16 of key l/16), so every access is a
// fully coalesced 1 KB; the per-key dot products are finished with a butterfly over the 16
// lanes of a key that also splits the g heads across those lanes (log2(g) fewer exchanges).
// Values are streamed the same way and accumulated per lane for its 8 features.
// Local layers ("lesson 6", section 7): on a linear cache, splits wholly before the window start
// (and after the sinks) write an empty partial without reading anything; on a rolling buffer
// every filled slot is visible and nothing is masked.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace q3 {

namespace {

constexpr int HD = 128;
constexpr int SK = kDecodeSplitKeys;  // keys per workgroup

// Cache slots holding the keys of sequence b's new token: slots 0 .. P (P = cache length before
// it, its own slot included), or every filled slot of a rolling buffer of a.cap slots.
__device__ __forceinline__ int decode_kv_len(const AttnArgs& a, int b) {
    const int p = seq_pos(a.pos, b);
    return a.local.rolling ? min(p + 1, a.cap) : p + 1;
}
constexpr int KPW = SK / 4;           // keys per wave
static_assert(KPW % 64 == 0, "the softmax pass gives each lane whole keys");

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// Partner exchange within the 16-lane row of a key, step k = 0..3: lane i pairs with i ^ 8
// (row_ror:8), 7 - i within its half row (row_half_mirror), then i ^ 2 and i ^ 1 (quad
// permutes).  Each pairing flips lane bit 3, 2, 1, 0 respectively.
template <int STEP>
__device__ __forceinline__ float partner(float x) {
    if constexpr (STEP == 0) return dpp_f32<0x128>(x);
    else if constexpr (STEP == 1) return dpp_f32<0x141>(x);
    else if constexpr (STEP == 2) return dpp_f32<0x4E>(x);
    else return dpp_f32<0xB1>(x);
}

// Reduce s[0..G) over the 16 lanes sharing a key.  On return s[0] holds the full sum for head
// `head` (which depends on the lane), every head being held by 16/G of the lanes: at each step
// a lane keeps one half of its heads and receives its partner's partial sums of that half.
template <int G>
__device__ __forceinline__ float key_reduce(float (&s)[G], int lane, int& head) {
    head = 0;
    auto step = [&](auto stepc) {
        constexpr int STEP = decltype(stepc)::value;
        constexpr int n = G >> STEP;              // heads still held per lane before this step
        const bool hi = (lane & (8 >> STEP)) != 0;
        if constexpr (n > 1) {
            constexpr int half = n >> 1;
#pragma unroll
            for (int i = 0; i < half; ++i) {
                const float send = hi ? s[i] : s[i + half];
                const float keep = hi ? s[i + half] : s[i];
                s[i] = keep + partner<STEP>(send);
            }
            if (hi) head += half;
        } else {
            s[0] += partner<STEP>(s[0]);
        }
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
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
    const int kv_len = decode_kv_len(a, b);
    const int key0 = split * SK;
    if (key0 >= kv_len) return;
    int pad_lo, pad_hi;   // left-padding slots of this sequence: never attended by the new token
    seq_pad(a.pos, b, pad_lo, pad_hi);
    // local layer on a linear cache: keys before the window start are skipped, except sinks
    const int win_lo = (a.local.window > 0 && !a.local.rolling) ? kv_len - a.local.window : 0;
    const int sinks = win_lo > 0 ? a.local.sinks : 0;
    if (key0 + SK <= win_lo && key0 >= sinks) {
        // no visible key in this split: an empty partial (weight 0 in the merge)
        const int S = p.splits;
        for (int idx = threadIdx.x; idx < G * HD; idx += 256) {
            const int h = idx / HD, d = idx % HD;
            const int64_t row = ((int64_t)b * a.Hq + kvh * G + h) * S + split;
            p.part_o[row * HD + d] = 0.f;
            if (d == 0) {
                p.part_ml[row * 2] = -INFINITY;
                p.part_ml[row * 2 + 1] = 0.f;
            }
        }
        return;
    }
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
        const int key = key0 + kk;
        const bool visible = (kk < nk) & ((key < pad_lo) | (key >= pad_hi)) & ((key >= win_lo) | (key < sinks));
        if ((dc & ((16 / G) - 1)) == 0) sP[kk * G + head] = visible ? sum : -INFINITY;
    }
    // the first value rows are requested now, so HBM stays busy through the softmax phase
    constexpr int VPRE = 4;
    bf16x8 vpre[VPRE];
#pragma unroll
    for (int i = 0; i < VPRE; ++i)
        vpre[i] = *reinterpret_cast<const bf16x8*>(vg + (int64_t)min(wave * KPW + 4 * i + ks, nk - 1) * HD);
    __syncthreads();

    // ---- per-wave softmax statistics over its KPW keys (lane takes keys lane + 64 i)
    constexpr int KPL = KPW / 64;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float sv[KPL];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            sv[i] = sP[(wave * KPW + lane + 64 * i) * G + h];
            mx = fmaxf(mx, sv[i]);
        }
        const float m = wave_max(mx);
        const float mref = (m == -INFINITY) ? 0.f : m;
        float ls = 0.f;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            const float pr = fast_exp2(sv[i] - mref);
            sP[(wave * KPW + lane + 64 * i) * G + h] = pr;
            ls += pr;
        }
        const float l = wave_sum(ls);
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
    auto accumulate = [&](int kk, const bf16x8& raw) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float pr = sP[kk * G + h];   // 0 for keys beyond the cache
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pr, (float)raw[e], acc[h][e]);
        }
    };
#pragma unroll
    for (int i = 0; i < VPRE; ++i) accumulate(wave * KPW + 4 * i + ks, vpre[i]);
#pragma unroll 4
    for (int i = VPRE; i < KPW / 4; ++i) {
        const int kk = wave * KPW + 4 * i + ks;
        accumulate(kk, *reinterpret_cast<const bf16x8*>(vg + (int64_t)min(kk, nk - 1) * HD));
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

// Merge the splits of one (head, sequence).  The global max of the split maxima comes from a
// block reduction; then, chunk by chunk, the split weights 2^(m_s - m) go to LDS and the 256
// threads split the (split, feature) pairs: thread (half, d) sums feature d over splits half,
// half + 2, ... of the chunk, in four independent chains; the two halves combine through LDS.
// The partial outputs of the first chunk (up to 64 splits: every split of a 64K-key cache) are
// requested before the maximum is formed, so a call costs one memory round trip, not two.
constexpr int kCombineThreads = 256;
constexpr int kSplitChunk = 64;          // splits per chunk: 32 partial outputs per thread
constexpr int kPerThread = kSplitChunk / 2;

__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DecodeAttnArgs p) {
    __shared__ float sW[kSplitChunk];
    __shared__ float sRed[kCombineThreads / 64];
    __shared__ float sO[2][HD];
    const AttnArgs& a = p.a;
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int kv_len = decode_kv_len(a, b);
    const int ns = (kv_len + SK - 1) / SK;
    const int64_t row0 = ((int64_t)b * a.Hq + h) * p.splits;
    const float* ml = p.part_ml + row0 * 2;
    const int d = tid & (HD - 1), half = tid >> 7;
    const float* po = p.part_o + row0 * HD + d;

    // partial outputs of chunk c0: this thread's splits c0 + half + 2i (zero past the last split)
    float ov[kPerThread];
    auto request = [&](int c0) {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int sp = c0 + half + 2 * i;
            ov[i] = sp < ns ? po[(int64_t)sp * HD] : 0.f;
        }
    };
    request(0);

    float m = -INFINITY;
    for (int sp = tid; sp < ns; sp += kCombineThreads) m = fmaxf(m, ml[2 * sp]);
    m = wave_max(m);
    if (lane == 0) sRed[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(sRed[0], sRed[1]), fmaxf(sRed[2], sRed[3]));

    float l = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
    for (int c0 = 0; c0 < ns; c0 += kSplitChunk) {
        const int n = min(kSplitChunk, ns - c0);
        __syncthreads();                        // previous chunk's weights are no longer read
        if (tid < n) {
            const float w = fast_exp2(ml[2 * (c0 + tid)] - m);
            sW[tid] = w;
            l = fmaf(w, ml[2 * (c0 + tid) + 1], l);
        }
        if (tid >= n && tid < kSplitChunk) sW[tid] = 0.f;   // splits past the last: weight 0
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPerThread; i += 4) {
            o0 = fmaf(ov[i], sW[half + 2 * i], o0);
            o1 = fmaf(ov[i + 1], sW[half + 2 * i + 2], o1);
            o2 = fmaf(ov[i + 2], sW[half + 2 * i + 4], o2);
            o3 = fmaf(ov[i + 3], sW[half + 2 * i + 6], o3);
        }
        if (c0 + kSplitChunk < ns) request(c0 + kSplitChunk);
    }
    l = wave_sum(l);
    __syncthreads();
    if (lane == 0) sRed[wave] = l;
    sO[half][d] = (o0 + o1) + (o2 + o3);
    __syncthreads();
    l = sRed[0] + sRed[1] + sRed[2] + sRed[3];
    if (half == 0)
        static_cast<bf16*>(a.out)[(int64_t)b * a.Hq * HD + (int64_t)h * HD + d] = (bf16)((sO[0][d] + sO[1][d]) / l);
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
    decode_combine_kernel<<<dim3((unsigned)a.Hq, (unsigned)a.B), kCombineThreads, 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace q3
