// fp32 causal grouped-query attention, any even head_dim <= 128, prefill or decode.
//
// Same definition as the bf16 kernels ("lesson 6", section 3: query head h reads KV head
// floor(h / g); scores scaled by D^-1/2; key visible iff its slot <= the query's and it is not
// left padding, or it is the query's own token), for the fp32 storage configuration.  One
// wavefront per (sequence, head, query): lane l holds features l and l + 64, each key costs one
// wave reduction, and the softmax is accumulated online in fp32 with exact expf.  Meant for
// small problems; no tiling.
#include "common.hpp"
#include "kernels.hpp"

namespace q3 {

namespace {

__global__ __launch_bounds__(256) void attention_f32_kernel(AttnArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t total = (int64_t)a.B * a.Hq * a.T;
    if (gw >= total) return;
    const int t = (int)(gw % a.T);
    const int h = (int)((gw / a.T) % a.Hq);
    const int b = (int)(gw / ((int64_t)a.T * a.Hq));
    const int kvh = h / (a.Hq / a.Hkv);
    const int D = a.D;
    int pos = seq_pos(a.pos, b) + t;          // the query's cache slot (linear cache)
    int pad_lo, pad_hi;                       // left-padding slots, seen only by themselves
    seq_pad(a.pos, b, pad_lo, pad_hi);
    // local layer: keys pos - window < j <= pos and the first `sinks`; on a rolling buffer every
    // filled slot (the query's own included) is visible
    int win_lo = (a.local.window > 0) ? pos - a.local.window + 1 : 0;
    if (a.local.rolling) {
        pos = min(pos, a.cap - 1);
        win_lo = 0;
    }
    const int sinks = a.local.sinks;

    const float* q = static_cast<const float*>(a.qhat) + (((int64_t)b * a.Hq + h) * a.T + t) * D;
    const float* kb = static_cast<const float*>(a.k_cache) + ((int64_t)b * a.Hkv + kvh) * a.cap * D;
    const float* vb = static_cast<const float*>(a.v_cache) + ((int64_t)b * a.Hkv + kvh) * a.cap * D;
    const bool in0 = lane < D, in1 = lane + 64 < D;
    const float q0 = in0 ? q[lane] : 0.f, q1 = in1 ? q[lane + 64] : 0.f;

    float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
    for (int j = 0; j <= pos; ++j) {
        if (j >= pad_lo && j < pad_hi && j != pos) continue;
        if (j < win_lo && j >= sinks) continue;
        const float* kr = kb + (int64_t)j * D;
        const float* vr = vb + (int64_t)j * D;
        const float s = wave_sum((in0 ? q0 * kr[lane] : 0.f) + (in1 ? q1 * kr[lane + 64] : 0.f)) * a.scale;
        const float m_new = fmaxf(m, s);
        const float corr = expf(m - m_new);
        const float p = expf(s - m_new);
        l = l * corr + p;
        acc0 = acc0 * corr + (in0 ? p * vr[lane] : 0.f);
        acc1 = acc1 * corr + (in1 ? p * vr[lane + 64] : 0.f);
        m = m_new;
    }
    float* o = static_cast<float*>(a.out) + ((int64_t)b * a.T + t) * a.Hq * D + (int64_t)h * D;
    if (in0) o[lane] = acc0 / l;
    if (in1) o[lane + 64] = acc1 / l;
}

}  // namespace

hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t stream) {
    if (a.D > 128 || a.Hkv <= 0 || a.Hq % a.Hkv) return hipErrorInvalidValue;
    const int64_t waves = (int64_t)a.B * a.Hq * a.T;
    if (waves <= 0) return hipSuccess;
    attention_f32_kernel<<<(unsigned)((waves + 3) / 4), 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace q3
