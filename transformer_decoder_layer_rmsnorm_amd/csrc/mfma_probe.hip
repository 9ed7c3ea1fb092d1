// Matrix-core rate probe: the ceiling that the bf16 GEMMs' roofline fraction is read against.
//
// Every wave issues back-to-back v_mfma_f32_32x32x16_bf16 on operands held in registers (16
// independent 32x32 accumulators, the same instruction and accumulator count per wave as the
// large-tile GEMMs), so the launch moves no operand data through memory or LDS at all.  Its rate
// is what the matrix cores sustain under the chip's power management with GEMM-like
// (pseudo-random, non-zero) bf16 operands; the published dense peak assumes the top clock at
// every cycle.  Not a step of the layer.
#include "common.hpp"
#include "kernels.hpp"

namespace q3 {

namespace {

// Operand values in [-1, 1) from a linear congruential sequence seeded by lane and salt.
__device__ bf16x8 probe_operand(int salt) {
    bf16x8 v;
    unsigned h = (threadIdx.x + 1) * 2654435761u ^ ((unsigned)salt * 40503u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h = h * 1664525u + 1013904223u;
        v[i] = (bf16)((float)(int)(h >> 8) * (1.0f / 8388608.0f) - 1.0f);
    }
    return v;
}

__global__ __launch_bounds__(256) void mfma_probe_kernel(float* out, int iters) {
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = probe_operand(i);
        b[i] = probe_operand(7 + i);
    }
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    // one sum per lane, so that no MFMA can be dropped
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += acc[i][j][r];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_probe(float* out, int workgroups, int iters, hipStream_t stream) {
    mfma_probe_kernel<<<(unsigned)workgroups, 256, 0, stream>>>(out, iters);
    return hipGetLastError();
}

}  // namespace q3
