// RMSNorm, one 64-lane wavefront per row.
//
// "17. A modern architecture: Qwen3", section RMSNorm: y_i = g_i x_i / sqrt(mean_j x_j^2 + eps),
// mean of squares in fp32 whatever the storage type.  Here the normalised value is multiplied
// by the gain in fp32 and rounded once to the output type (the page rounds to the input type
// before the gain; the difference is below one output ulp).  Zero-centred gains (the page's
// parity detail 2: Gemma and the Qwen3.5 family store g and apply 1 + g) take goff = 1.
//
// Memory-bound: each row is read once (16-byte loads, kept in registers up to 4096 wide; wider
// rows are read twice) and written once.  Four rows per 256-thread workgroup.
//
// Split-K residual form: when o_proj's K range is split across workgroups, its fp32 partial
// slabs are summed here, in a fixed order (deterministic), together with the residual:
// x1 = x + sum_s part_s, written in fp32, then normalised ("17. A modern architecture: Qwen3",
// section The whole model, Qwen3Layer: x1 = x + attn(...), then post_attention_layernorm(x1)).
#include "common.hpp"
#include "kernels.hpp"

namespace q3 {

// EARLY_G: the gains are requested together with the row (a call of a few rows then waits for
// one memory round trip, not two); for many rows the kernel is bandwidth-bound and the extra
// registers would only cost occupancy, so the gains are read after the reduction.
template <typename TX, typename TY, int MAXC, bool EARLY_G>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const TX* __restrict__ x, const TY* __restrict__ g,
                                                      TY* __restrict__ y, int64_t rows, int width, float eps,
                                                      float goff) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const TX* xr = x + row * width;
    TY* yr = y + row * width;
    const int nchunk = width >> 3;   // chunks of 8 elements

    if (MAXC > 0 && nchunk <= MAXC * kWave) {
        float v[MAXC][8], gv[EARLY_G ? MAXC : 1][8];
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < MAXC; ++j) {
            const int c = lane + j * kWave;
            if (c < nchunk) {
                load8(xr + c * 8, v[j]);
                if constexpr (EARLY_G) load8(g + c * 8, gv[j]);
#pragma unroll
                for (int i = 0; i < 8; ++i) ss = fmaf(v[j][i], v[j][i], ss);
            }
        }
        const float rstd = rsqrtf(wave_sum(ss) / (float)width + eps);
#pragma unroll
        for (int j = 0; j < MAXC; ++j) {
            const int c = lane + j * kWave;
            if (c < nchunk) {
                float o[8];
                if constexpr (!EARLY_G) load8(g + c * 8, gv[0]);
                const float* gj = gv[EARLY_G ? j : 0];
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = (goff + gj[i]) * (v[j][i] * rstd);
                store8(yr + c * 8, o);
            }
        }
    } else {
        float ss = 0.f;
        for (int c = lane; c < nchunk; c += kWave) {
            float v[8];
            load8(xr + c * 8, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
        }
        const float rstd = rsqrtf(wave_sum(ss) / (float)width + eps);
        for (int c = lane; c < nchunk; c += kWave) {
            float v[8], gv[8], o[8];
            load8(xr + c * 8, v);
            load8(g + c * 8, gv);
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = (goff + gv[i]) * (v[i] * rstd);
            store8(yr + c * 8, o);
        }
    }
}

// Input RMSNorm (bf16) plus the RoPE table row of each token: lane i of the row's wave forms the
// angle of frequency i (see RopeTable).  Rows up to 64 NC wide stay in registers between the
// reduction and the output; wider rows (NC = 0) are read twice.  EARLY_G as in rmsnorm_kernel.
template <int NC, bool EARLY_G>
__global__ __launch_bounds__(256) void rmsnorm_rope_kernel(const bf16* __restrict__ x, const bf16* __restrict__ g,
                                                           bf16* __restrict__ y, int64_t rows, int width, float eps,
                                                           float goff, RopeTable rope) {
    constexpr bool WIDE = NC == 0;
    constexpr int MAXC = WIDE ? 1 : NC;
    static_assert(!(WIDE && EARLY_G), "wide rows read the gains in the output pass");
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const bf16* xr = x + row * width;
    bf16* yr = y + row * width;
    const int nchunk = width >> 3;
    float v[MAXC][8], gv0[EARLY_G ? MAXC : 1][8];
    float ss = 0.f;
    if constexpr (WIDE) {
        for (int c = lane; c < nchunk; c += kWave) {
            load8(xr + c * 8, v[0]);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = fmaf(v[0][i], v[0][i], ss);
        }
    } else {
#pragma unroll
        for (int j = 0; j < MAXC; ++j) {
            const int c = lane + j * kWave;
            if (c < nchunk) {
                load8(xr + c * 8, v[j]);
                if constexpr (EARLY_G) load8(g + c * 8, gv0[j]);
#pragma unroll
                for (int i = 0; i < 8; ++i) ss = fmaf(v[j][i], v[j][i], ss);
            }
        }
    }
    // the angle of frequency `lane` at this token's position, while the loads are in flight
    const int b = (int)(row / rope.T), t = (int)(row - (int64_t)b * rope.T);
    const int lin = seq_pos(rope.pos, b) + t;
    int pad_lo, pad_hi;
    seq_pad(rope.pos, b, pad_lo, pad_hi);
    const double turns = (double)slot_position(lin, pad_lo, pad_hi) * rope.turns[lane];
    const float rr = (float)(turns - rint(turns));
    const float2 cs = make_float2(__builtin_amdgcn_cosf(rr), __builtin_amdgcn_sinf(rr));
    reinterpret_cast<float2*>(rope.cs)[row * 64 + lane] = cs;
    if (lane == 0) rope.slot[row] = lin;
    const float rstd = rsqrtf(wave_sum(ss) / (float)width + eps);
    if constexpr (WIDE) {
        for (int c = lane; c < nchunk; c += kWave) {
            float gv[8], o[8];
            load8(xr + c * 8, v[0]);
            load8(g + c * 8, gv);
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = (goff + gv[i]) * (v[0][i] * rstd);
            store8(yr + c * 8, o);
        }
    } else {
#pragma unroll
        for (int j = 0; j < MAXC; ++j) {
            const int c = lane + j * kWave;
            if (c < nchunk) {
                float gv[8], o[8];
                if constexpr (EARLY_G) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) gv[i] = gv0[j][i];
                } else {
                    load8(g + c * 8, gv);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = (goff + gv[i]) * (v[j][i] * rstd);
                store8(yr + c * 8, o);
            }
        }
    }
}

hipError_t launch_rmsnorm_rope(const void* x, const void* g, void* y, int64_t rows, int width, float eps, float goff,
                               const RopeTable& rope, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if ((width & 7) || rope.T <= 0 || !rope.cs || !rope.slot) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)((rows + 3) / 4);
#define Q3_RMS_ROPE(NC, EG)                                                                                      \
    rmsnorm_rope_kernel<NC, EG><<<grid, 256, 0, s>>>(static_cast<const bf16*>(x), static_cast<const bf16*>(g), \
                                                    static_cast<bf16*>(y), rows, width, eps, goff, rope)
    // rows up to 1024 wide: two chunks per lane, the gains requested with the row (one memory round
    // trip per row instead of two, and few enough registers for full occupancy)
    if (width <= 2 * 8 * kWave)
        Q3_RMS_ROPE(2, true);
    else if (width <= 8 * 8 * kWave)
        Q3_RMS_ROPE(8, false);
    else
        Q3_RMS_ROPE(0, false);
#undef Q3_RMS_ROPE
    return hipGetLastError();
}

template <typename TX, typename TY>
static hipError_t launch_typed(const void* x, const void* g, void* y, int64_t rows, int width, float eps,
                               float goff, hipStream_t s) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (width <= 2 * 8 * kWave)   // two chunks per lane: the gains with the row, one round trip
        rmsnorm_kernel<TX, TY, 2, true><<<grid, 256, 0, s>>>(static_cast<const TX*>(x), static_cast<const TY*>(g),
                                                             static_cast<TY*>(y), rows, width, eps, goff);
    else if (rows <= 1024)   // fewer rows than one per wave slot of the chip: latency-bound
        rmsnorm_kernel<TX, TY, 8, true><<<grid, 256, 0, s>>>(static_cast<const TX*>(x), static_cast<const TY*>(g),
                                                             static_cast<TY*>(y), rows, width, eps, goff);
    else
        rmsnorm_kernel<TX, TY, 8, false><<<grid, 256, 0, s>>>(static_cast<const TX*>(x), static_cast<const TY*>(g),
                                                              static_cast<TY*>(y), rows, width, eps, goff);
    return hipGetLastError();
}


// x + the split-K slabs of one 8-element chunk, summed in a fixed order (deterministic)
template <typename TX>
__device__ __forceinline__ void resid_chunk(const TX* x, const float* part, int splits, int64_t slab, int64_t o,
                                            float* v) {
    load8(x + o, v);
    for (int sp = 0; sp < splits; ++sp) {
        float pv[8];
        load8(part + sp * slab + o, pv);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] += pv[i];
    }
}

// Rows up to 4096 wide keep x1 in registers between the reduction and the output; wider rows
// (WIDE) form x1 again in the output pass (same operands, same order, same value).
template <typename TX, typename TY, bool WIDE>
__global__ __launch_bounds__(256) void residual_rmsnorm_kernel(const TX* __restrict__ x, const float* __restrict__ part,
                                                               int splits, float* __restrict__ x1,
                                                               const TY* __restrict__ g, TY* __restrict__ y,
                                                               int64_t rows, int width, float eps, float goff) {
    constexpr int MAXC = 8;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int64_t off = row * width;
    const int64_t slab = rows * width;
    const int nchunk = width >> 3;
    float ss = 0.f;
    if constexpr (WIDE) {
        for (int c = lane; c < nchunk; c += kWave) {
            float v[8];
            resid_chunk(x, part, splits, slab, off + c * 8, v);
            store8(x1 + off + c * 8, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
        }
        const float rstd = rsqrtf(wave_sum(ss) / (float)width + eps);
        for (int c = lane; c < nchunk; c += kWave) {
            float v[8], gv[8], o[8];
            resid_chunk(x, part, splits, slab, off + c * 8, v);
            load8(g + c * 8, gv);
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = (goff + gv[i]) * (v[i] * rstd);
            store8(y + off + c * 8, o);
        }
    } else {
        float v[MAXC][8];
#pragma unroll
        for (int j = 0; j < MAXC; ++j) {
            const int c = lane + j * kWave;
            if (c < nchunk) {
                resid_chunk(x, part, splits, slab, off + c * 8, v[j]);
                store8(x1 + off + c * 8, v[j]);
#pragma unroll
                for (int i = 0; i < 8; ++i) ss = fmaf(v[j][i], v[j][i], ss);
            }
        }
        const float rstd = rsqrtf(wave_sum(ss) / (float)width + eps);
#pragma unroll
        for (int j = 0; j < MAXC; ++j) {
            const int c = lane + j * kWave;
            if (c < nchunk) {
                float gv[8], o[8];
                load8(g + c * 8, gv);
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = (goff + gv[i]) * (v[j][i] * rstd);
                store8(y + off + c * 8, o);
            }
        }
    }
}

hipError_t launch_residual_rmsnorm(const void* x, DType xt, const float* part, int splits, float* x1, const void* g,
                                   void* y, DType yt, int64_t rows, int width, float eps, float goff, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if ((width & 7) || splits < 1) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((rows + 3) / 4));
    const bool wide = width > 8 * 8 * kWave;
#define Q3_RESID_RMS(TX, TY, W)                                                                                   \
    residual_rmsnorm_kernel<TX, TY, W><<<grid, 256, 0, s>>>(static_cast<const TX*>(x), part, splits, x1,         \
                                                             static_cast<const TY*>(g), static_cast<TY*>(y), rows, \
                                                             width, eps, goff)
    if (xt == DType::BF16 && yt == DType::BF16) {
        if (wide) Q3_RESID_RMS(bf16, bf16, true); else Q3_RESID_RMS(bf16, bf16, false);
    } else if (xt == DType::F32 && yt == DType::F32) {
        if (wide) Q3_RESID_RMS(float, float, true); else Q3_RESID_RMS(float, float, false);
    } else {
        return hipErrorInvalidValue;
    }
#undef Q3_RESID_RMS
    return hipGetLastError();
}

// y = x1 + sum_s part_s, rounded once to bf16 (the residual add of a split-K down projection):
// eight elements per thread, the slabs summed in a fixed order.
__global__ __launch_bounds__(256) void residual_sum_kernel(const float* __restrict__ x1, const float* __restrict__ part,
                                                           int splits, bf16* __restrict__ y, int64_t n) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i >= n) return;
    float v[8];
    load8(x1 + i, v);
    for (int sp = 0; sp < splits; ++sp) {
        float pv[8];
        load8(part + sp * n + i, pv);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += pv[e];
    }
    store8(y + i, v);
}

hipError_t launch_residual_sum_bf16(const float* x1, const float* part, int splits, void* y, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if ((n & 7) || splits < 1) return hipErrorInvalidValue;
    residual_sum_kernel<<<(unsigned)((n / 8 + 255) / 256), 256, 0, s>>>(x1, part, splits, static_cast<bf16*>(y), n);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const void* x, DType xt, const void* g, void* y, DType yt, int64_t rows, int width,
                          float eps, float goff, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    if (xt == DType::BF16 && yt == DType::BF16) return launch_typed<bf16, bf16>(x, g, y, rows, width, eps, goff, stream);
    if (xt == DType::F32 && yt == DType::BF16) return launch_typed<float, bf16>(x, g, y, rows, width, eps, goff, stream);
    if (xt == DType::F32 && yt == DType::F32) return launch_typed<float, float>(x, g, y, rows, width, eps, goff, stream);
    return hipErrorInvalidValue;
}

}  // namespace q3
