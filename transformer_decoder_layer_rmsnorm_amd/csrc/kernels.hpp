// Host-side launch interface of the gfx950 kernels (one .hip file per kernel family).
// Every launcher only enqueues work on `stream` and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q3 {

enum class DType : int { F32 = 0, BF16 = 1 };

// Per-sequence placement of the tokens of a call.
//  * first slot: cache slot of token 0 of each sequence (prefill on an empty cache: 0; prefill
//    onto a cache: its length; decode: the cache length).
//  * padding: an optional run of cache slots [pad_lo, pad_lo + pad_n) per sequence holding
//    left-padding tokens ("lesson 6", section 8, batched generation): no other token attends
//    them (a padding token still attends itself and the real keys before it), and positions
//    count real tokens only: slot s sits at position s below the run, s - pad_n above it, and
//    max(pad_lo - 1, 0) inside it (number of real tokens up to it, minus one, clamped at 0).
// Up to kInlinePositions sequences the values travel by value in the kernel arguments (no
// host-to-device copy); beyond, through device arrays.
constexpr int kInlinePositions = 64;
struct SeqPositions {
    const int32_t* dev;                 // device array [B] of first slots, or nullptr
    const int32_t* dev_pad;             // device array [2B]: pad_lo[B] then pad_n[B], or nullptr
    int32_t n_inline;                   // when dev == nullptr: inl[b] for b < n_inline, else 0
    int32_t n_pad_inline;               // when dev_pad == nullptr: padding of b < n_pad_inline
    int32_t inl[kInlinePositions];
    int32_t pad_lo[kInlinePositions];
    int32_t pad_n[kInlinePositions];
};
__device__ __forceinline__ int seq_pos(const SeqPositions& p, int b) {
    return p.dev ? p.dev[b] : (b < p.n_inline ? p.inl[b] : 0);
}
// padding run [lo, hi) of sequence b (lo == hi when it has none)
__device__ __forceinline__ void seq_pad(const SeqPositions& p, int b, int& lo, int& hi) {
    if (p.dev_pad) {
        lo = p.dev_pad[b];
        hi = lo + p.dev_pad[p.n_pad_inline + b];   // n_pad_inline holds B when dev_pad is set
    } else if (b < p.n_pad_inline) {
        lo = p.pad_lo[b];
        hi = lo + p.pad_n[b];
    } else {
        lo = hi = 0;
    }
}
// position of cache slot `slot` of a sequence with padding run [lo, hi)
__device__ __forceinline__ int slot_position(int slot, int lo, int hi) {
    return slot < lo ? slot : (slot >= hi ? slot - (hi - lo) : max(lo - 1, 0));
}

// Local (sliding-window) attention ("lesson 6", section 7): token i sees token j iff
// i - window < j <= i, plus the first `sinks` tokens (attention sinks); window 0 = global.
// With `rolling`, a decode cache is a rolling buffer of sinks + window slots: token i lives in
// slot i below `sinks` and in slot sinks + (i - sinks) mod window above, so the buffer holds
// exactly the keys the newest token sees and no mask is needed.
struct LocalAttn {
    int32_t window;
    int32_t sinks;
    int32_t rolling;
};
__device__ __forceinline__ int rolling_slot(const LocalAttn& w, int pos) {
    return pos < w.sinks ? pos : w.sinks + (pos - w.sinks) % w.window;
}

inline int dtype_size(DType t) { return t == DType::F32 ? 4 : 2; }

// ---------------------------------------------------------------- RMSNorm
// y[r, :] = g * x[r, :] / sqrt(mean(x[r, :]^2) + eps), fp32 reduction, one rounding.
// x1 = x + sum_s part[s] (fp32, written), then y = g * x1 / rms(x1): the residual add of a
// split-K projection fused with the following RMSNorm.  part holds `splits` slabs [rows, width].
// goff: gain offset, 0 for the pages' gains, 1 for zero-centred gains applied as (1 + g).
hipError_t launch_residual_rmsnorm(const void* x, DType xt, const float* part, int splits, float* x1,
                                   const void* g, void* y, DType yt, int64_t rows, int width, float eps,
                                   float goff, hipStream_t stream);
// RoPE angle table of a prefill call ("17. A modern architecture: Qwen3", section Rotary position
// embeddings): for token row m = b T + t and frequency i < 64 (head_dim 128, rotate-half over
// the whole head), cs[m][i] = (cos, sin) of 2 pi * turns[i] * position(m), the turn count formed
// in fp64 and reduced to [-1/2, 1/2] before the fp32 sin / cos, and slot[m] = the row's cache
// slot.  Written by the input RMSNorm (one row per wave, one frequency per lane) for the QKV
// epilogue that rotates q and k and stores k and v.
struct RopeTable {
    float* cs;               // [rows, 64, 2] (cos, sin)
    int32_t* slot;           // [rows] cache slot of each token row
    SeqPositions pos;        // first slot and padding of each sequence
    int T;                   // tokens per sequence
    double turns[64];        // position scale * omega_i / (2 pi)
};
// y = bf16(x1 + sum of `splits` fp32 slabs of n elements): the residual add after a split-K
// down projection
hipError_t launch_residual_sum_bf16(const float* x1, const float* part, int splits, void* y, int64_t n,
                                    hipStream_t stream);
// bf16 input RMSNorm that also writes the RoPE table of its rows
hipError_t launch_rmsnorm_rope(const void* x, const void* g, void* y, int64_t rows, int width, float eps,
                               float goff, const RopeTable& rope, hipStream_t stream);
hipError_t launch_rmsnorm(const void* x, DType xt, const void* g, void* y, DType yt,
                          int64_t rows, int width, float eps, float goff, hipStream_t stream);

// ---------------------------------------------------------------- projections (C = A * B^T)
enum class Epilogue : int {
    Store = 0,         // out(dtype)  = C
    ResidToF32 = 1,    // out(fp32)   = resid(dtype) + C        (o_proj: x1 = x + attn Wo^T)
    SwiGLU = 2,        // out(dtype)  = silu(C_gate) * C_up     (B0 = gate, B1 = up)
    ResidF32In = 3,    // out(dtype)  = resid(fp32) + C         (down: y = x1 + act Wd^T)
    PartialF32 = 4,    // out(fp32) + split*M*N = C over the split's K range (split-K partials)
};

struct GemmArgs {
    const void* a;          // [M, K] row-major, dtype
    const void* b[3];       // weight segments, each [rows, K] row-major (nn.Linear layout)
    int b_rows[3];          // rows of each segment; segments are stacked along N
    int nseg;
    void* out;              // [M, N] row-major (N = sum of segment rows, or I for SwiGLU)
    const void* resid;      // [M, N] residual for the two residual epilogues
    int M, N, K;
    Epilogue epi;
    int splits;             // PartialF32: K is cut into `splits` equal ranges, one fp32 slab each
};

// Split-K form of a skinny (M <= 16) projection: column groups of 16 cg outputs, kslices k
// slices of 256 nit; kslices = 0 when the shape is not split.  launch_gemv_bf16 with the
// PartialF32 epilogue and splits = kslices writes the [kslices][M][N] fp32 slabs.
struct SkinnyPlan {
    int cg, nit, kslices, groups;
};
SkinnyPlan skinny_plan(int M, int N, int K);

hipError_t launch_gemm_bf16(const GemmArgs& args, hipStream_t stream);   // MFMA, large M
// Split count for a bf16 projection whose partial sums can be reduced by the next kernel: 2 when
// the output has too few 128x128 tiles to fill the CUs and K splits evenly, else 1 (no split).
int gemm_bf16_splits(int M, int N, int K);
hipError_t launch_gemv_bf16(const GemmArgs& args, hipStream_t stream);   // MFMA, M <= 64
hipError_t launch_gemm_f32(const GemmArgs& args, hipStream_t stream);    // fp32 FMA, any shape
bool gemm_bf16_supported(int N_segment_rows, int K);

// ---------------------------------------------------------------- QK-norm + RoPE + cache write
struct QkRopeArgs {
    const void* qkv;        // [M, (Hq + 2 Hkv) D] token-major projections
    const void* q_norm;     // [D]
    const void* k_norm;     // [D]
    void* qhat;             // [B, Hq, T, D]
    void* k_cache;          // [B, Hkv, cap, D]
    void* v_cache;          // [B, Hkv, cap, D]
    SeqPositions pos;       // position (and cache slot) of token 0 of each sequence
    LocalAttn local;        // rolling: the cache slot is rolling_slot(position)
    int B, T, Hq, Hkv, D, cap;
    float eps;
    float goff;             // q_norm / k_norm gain offset (1 for zero-centred gains)
    int rotary_dim;         // features rotated per head (== D unless partial RoPE)
    int adjacent;           // 1: pairs (2i, 2i+1); 0: pairs (i, i + rotary_dim/2)
    double turns[64];       // position scale * omega_i / (2 pi) for pair i < rotary_dim/2,
                            // omega_i = theta^(-2i/rotary_dim), fp64
    const float* rope_cs;   // RopeTable::cs and ::slot of these rows, or nullptr (the fused QKV
    const int32_t* rope_slot;  // epilogue needs them; launch_qknorm_rope works them out itself)
    // qkv_splits > 0: the projections are the sum of qkv_splits fp32 slabs [splits][M][N] at
    // qkv_part (a split-K skinny projection), rounded to bf16 as the one-kernel form stores them
    // and stored to qkv_sum ([M, N] bf16, the workspace's projection intermediate); bf16,
    // head_dim 128, full split-half RoPE only
    const float* qkv_part;
    int qkv_splits;
    void* qkv_sum;
};
hipError_t launch_qknorm_rope(const QkRopeArgs& args, DType t, hipStream_t stream);
// QKV projection with QK-norm + RoPE + cache write fused into its epilogue (bf16, head_dim 128,
// full split-half RoPE over the head, prefill shapes on 256 x 256 or 256 x 128 ping-pong tiles or
// 128 x 128 register tiles, rope_cs / rope_slot set); `fusable` says whether the combination
// applies, else the caller runs the GEMM and launch_qknorm_rope separately.
bool gemm_qkv_fusable(const GemmArgs& g, const QkRopeArgs& a);
hipError_t launch_gemm_qkv_qkrope(const GemmArgs& g, const QkRopeArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- attention
struct AttnArgs {
    const void* qhat;       // [B, Hq, T, D]
    const void* k_cache;    // [B, Hkv, cap, D]
    const void* v_cache;    // [B, Hkv, cap, D]
    void* out;              // [B, T, Hq, D] (token-major rows of width Hq * D)
    SeqPositions pos;       // position of query 0 of each sequence
    LocalAttn local;        // window / sinks mask; rolling decode caches
    int B, T, Hq, Hkv, D, cap;
    float scale;            // D^-1/2
    // q_norm / k_norm gains (and their offset) of the layer, or nullptr: every q-hat and k-hat
    // is a gain times a unit-RMS head vector (rotated), so |q-hat . k-hat| <= D max|g_q| max|g_k|,
    // which lets the prefill attention skip the running maximum when the bound is small
    const void* q_norm;
    const void* k_norm;
    float goff;
};
// Causal prefill: query t of sequence b sits at position pos0(b) + t and sees keys 0 .. pos.
hipError_t launch_attention_prefill_bf16(const AttnArgs& args, hipStream_t stream);
// Generic fp32 attention (any D <= 128), prefill or decode (T = 1).
hipError_t launch_attention_f32(const AttnArgs& args, hipStream_t stream);

// Split-KV decode (T = 1): partials then combine.
struct DecodeAttnArgs {
    AttnArgs a;
    float* part_o;          // [B, Hq, S, D]
    float* part_ml;         // [B, Hq, S, 2]
    int splits;             // S
    int split_keys;
};
hipError_t launch_attention_decode_split_bf16(const DecodeAttnArgs& args, hipStream_t stream);
hipError_t launch_attention_decode_combine_bf16(const DecodeAttnArgs& args, hipStream_t stream);
constexpr int kDecodeSplitKeys = 1024;

// Matrix-core rate probe (mfma_probe.hip): workgroups x 4 waves, each iters x 16 bf16 32x32x16
// MFMAs on register operands; out receives workgroups x 256 floats.
hipError_t launch_mfma_probe(float* out, int workgroups, int iters, hipStream_t stream);

}  // namespace q3
