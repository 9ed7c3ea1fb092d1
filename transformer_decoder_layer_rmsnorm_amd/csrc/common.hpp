// Device helpers shared by the gfx950 kernels of the Qwen3 decoder layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q3 {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }  // RNE

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// Eight consecutive elements <-> eight floats (16-byte bf16 or 2x16-byte fp32 accesses).
__device__ __forceinline__ void load8(const bf16* p, float* out) {
    bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
}
__device__ __forceinline__ void load8(const float* p, float* out) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { out[i] = a[i]; out[4 + i] = b[i]; }
}
__device__ __forceinline__ void store8(bf16* p, const float* v) {
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (bf16)v[i];
    *reinterpret_cast<bf16x8*>(p) = o;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[4 + i]; }
    *reinterpret_cast<f32x4*>(p) = a;
    *reinterpret_cast<f32x4*>(p + 4) = b;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// silu(g) * u in fp32 (silu(z) = z * sigmoid(z)).
// SiLU(g) * u = g * u / (1 + e^-g).  The reciprocal is the hardware's v_rcp_f32 (about 1 ulp):
// an IEEE-exact division expands to about ten instructions per element, which the SwiGLU
// epilogues pay with the matrix cores idle, and the result is rounded to bf16 (or compared at
// 1e-4 in fp32) anyway.  g -> -inf gives NaN either way; a finite g far below zero gives -0.
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

}  // namespace q3
