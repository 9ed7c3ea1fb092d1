// C ABI of the Qwen3-style decoder layer: argument validation, workspace layout and the
// kernel sequence of prefill and decode.  Declarations and contracts: include/qwen3_layer.h.
//
// Kernel sequence of one layer ("17. A modern architecture: Qwen3", section The whole model:
// x = x + attn(input_layernorm(x)); x = x + mlp(post_attention_layernorm(x))):
//   1 rmsnorm        x  -> h
//   2 gemm (store)   h  -> qkv          q | k | v projections in one pass over the three weights
//   3 qknorm_rope    qkv -> qhat, k/v cache slots
//   4 attention      qhat, cache -> attn
//   5 gemm (+resid)  attn, x -> x1 (fp32 residual stream)
//   6 rmsnorm        x1 -> h2
//   7 gemm (swiglu)  h2 -> act = silu(h2 Wg^T) * (h2 Wu^T)
//   8 gemm (+resid)  act, x1 -> y
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/qwen3_layer.h"
#include "kernels.hpp"

using namespace q3;

namespace {

thread_local std::string g_last_error;

qwen3_status fail(qwen3_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
qwen3_status fail(qwen3_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

struct StageRec {
    int stage;
    hipEvent_t start, stop;
};

}  // namespace

struct qwen3_layer {
    qwen3_config cfg;
    qwen3_layer_weights w;
    double rope_turns[64];   // omega_i / (2 pi), omega_i = theta^(-2i/D), i < D/2
    bool profiling = false;
    std::mutex prof_mu;
    std::vector<std::string> stage_names;
    std::vector<StageRec> pending;
    std::vector<hipEvent_t> free_events;
};

namespace {

DType dt(const qwen3_config& c) { return c.dtype == QWEN3_BF16 ? DType::BF16 : DType::F32; }

qwen3_status validate_config(const qwen3_config* c) {
    if (!c) return fail(QWEN3_ERR_INVALID_ARGUMENT, "config is NULL");
    if (c->hidden_size <= 0 || c->num_attention_heads <= 0 || c->num_key_value_heads <= 0 ||
        c->head_dim <= 0 || c->intermediate_size <= 0 || c->max_position_embeddings <= 0)
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "config sizes must be positive");
    if (c->head_dim % 2)
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "head_dim %d is odd: RoPE pairs feature i with i + head_dim/2",
                    c->head_dim);
    if (!(c->rope_theta > 0.0) || !std::isfinite(c->rope_theta))
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "rope_theta must be positive and finite");
    if (!(c->rms_norm_eps >= 0.f) || !std::isfinite(c->rms_norm_eps))
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "rms_norm_eps must be non-negative and finite");
    if (c->dtype != QWEN3_F32 && c->dtype != QWEN3_BF16)
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)c->dtype);
    if (c->rotary_dim < 0 || c->rotary_dim > c->head_dim || (c->rotary_dim & 1))
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "rotary_dim %d must be even and within [0, head_dim %d]",
                    c->rotary_dim, c->head_dim);
    if (c->rope_adjacent_pairs != 0 && c->rope_adjacent_pairs != 1)
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "rope_adjacent_pairs must be 0 or 1");
    if (c->norm_unit_offset != 0 && c->norm_unit_offset != 1)
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "norm_unit_offset must be 0 or 1");
    if (!(c->rope_position_scale >= 0.0) || !std::isfinite(c->rope_position_scale))
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "rope_position_scale must be non-negative and finite");
    if (c->num_attention_heads % c->num_key_value_heads)
        return fail(QWEN3_ERR_UNSUPPORTED, "num_attention_heads %d is not a multiple of num_key_value_heads %d",
                    c->num_attention_heads, c->num_key_value_heads);
    const int64_t H = c->hidden_size, D = c->head_dim, I = c->intermediate_size;
    const int64_t Hq = c->num_attention_heads, Hkv = c->num_key_value_heads;
    if (H % 8) return fail(QWEN3_ERR_UNSUPPORTED, "hidden_size must be a multiple of 8");
    if ((Hq + 2 * Hkv) * D >= (int64_t)1 << 30 || H * I >= (int64_t)1 << 31 || H * Hq * D >= (int64_t)1 << 31)
        return fail(QWEN3_ERR_UNSUPPORTED, "layer too large for 32-bit weight indexing");
    if (c->dtype == QWEN3_BF16) {
        if (D != 128) return fail(QWEN3_ERR_UNSUPPORTED, "bf16 kernels need head_dim 128 (got %d)", (int)D);
        const int g = (int)(Hq / Hkv);
        if (g != 1 && g != 2 && g != 4 && g != 8)
            return fail(QWEN3_ERR_UNSUPPORTED, "bf16 decode supports 1, 2, 4 or 8 query heads per KV head (got %d)", g);
        if (H % 128 || I % 128)
            return fail(QWEN3_ERR_UNSUPPORTED, "bf16 kernels need hidden_size and intermediate_size multiples of 128");
    } else {
        if (D > 128) return fail(QWEN3_ERR_UNSUPPORTED, "fp32 kernels need head_dim <= 128 (got %d)", (int)D);
    }
    return QWEN3_OK;
}

struct Layout {
    size_t h, qkv, qhat, attn, x1, h2, act, part_gemm, prefill_end;
    size_t lens, part_o, part_ml, total;
    int splits;
};

// Split-K geometry of the skinny (M <= 16, bf16) QKV projection, whose fp32 slabs the QK-norm +
// RoPE kernel adds (head_dim 128 split-half RoPE only); kslices = 0: not split.  o_proj and
// down keep the one-kernel form: their slabs would need another pass over the residual.
SkinnyPlan skinny_qkv_split(const qwen3_config& c, int64_t M) {
    if (c.dtype != QWEN3_BF16 || M > 16 || c.head_dim != 128 || c.rotary_dim != 128 || c.rope_adjacent_pairs)
        return SkinnyPlan{};
    return skinny_plan((int)M, (c.num_attention_heads + 2 * c.num_key_value_heads) * c.head_dim, c.hidden_size);
}

Layout make_layout(const qwen3_config& c, int64_t B, int64_t T, int64_t cap) {
    const int64_t M = B * T;
    const int64_t es = c.dtype == QWEN3_BF16 ? 2 : 4;
    const int64_t H = c.hidden_size, D = c.head_dim, I = c.intermediate_size;
    const int64_t Hq = c.num_attention_heads, Hkv = c.num_key_value_heads;
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
    L.h = take(M * H * es);
    L.qkv = take(M * (Hq + 2 * Hkv) * D * es);
    L.qhat = take(M * Hq * D * es);
    L.attn = take(M * Hq * D * es);
    L.x1 = take(M * H * 4);
    L.h2 = take(M * H * es);
    L.act = take(M * I * es);
    // split-K partial slabs of o_proj (bf16 prefill with few output tiles)
    int64_t splits = 0;
    if (c.dtype == QWEN3_BF16 && M <= 0x7fffffff) {
        const int so = std::max(gemm_bf16_splits((int)M, (int)H, (int)(Hq * D)),
                                gemm_bf16_splits((int)M, (int)H, (int)I));
        splits = so > 1 ? so : 0;
    }
    // or the slabs of a split skinny QKV projection
    const int64_t skinny_bytes = (int64_t)skinny_qkv_split(c, M).kslices * M * (Hq + 2 * Hkv) * D * 4;
    L.part_gemm = take(std::max<int64_t>(splits * M * H * 4, skinny_bytes));
    L.prefill_end = off;
    L.splits = cap > 0 ? (int)((cap + kDecodeSplitKeys - 1) / kDecodeSplitKeys) : 0;
    L.lens = take(B * 4 * 3);   // first slots, padding starts, padding lengths
    L.part_o = take(c.dtype == QWEN3_BF16 ? B * Hq * L.splits * D * 4 : 0);
    L.part_ml = take(c.dtype == QWEN3_BF16 ? B * Hq * L.splits * 2 * 4 : 0);
    L.total = off;
    return L;
}

qwen3_status check_sizes(const qwen3_layer* L, int32_t batch, int32_t seq_len, int32_t cap) {
    if (!L) return fail(QWEN3_ERR_INVALID_ARGUMENT, "layer is NULL");
    if (batch <= 0 || seq_len <= 0) return fail(QWEN3_ERR_INVALID_ARGUMENT, "batch and seq_len must be positive");
    if (cap < 0) return fail(QWEN3_ERR_INVALID_ARGUMENT, "cache_capacity must be non-negative");
    const qwen3_config& c = L->cfg;
    const int64_t M = (int64_t)batch * seq_len;
    const int64_t widest = std::max<int64_t>({(int64_t)c.intermediate_size,
                                              (int64_t)(c.num_attention_heads + 2 * c.num_key_value_heads) * c.head_dim,
                                              (int64_t)c.hidden_size});
    if (M * widest >= (int64_t)1 << 31)
        return fail(QWEN3_ERR_UNSUPPORTED, "batch*seq_len too large for 32-bit activation indexing");
    if ((int64_t)batch * c.num_key_value_heads * std::max(cap, seq_len) * c.head_dim >= (int64_t)1 << 40)
        return fail(QWEN3_ERR_UNSUPPORTED, "cache too large");
    if (((int64_t)std::max(cap, seq_len) + 64) * c.head_dim * 4 >= (int64_t)1 << 31)
        return fail(QWEN3_ERR_UNSUPPORTED, "cache_capacity too large for 32-bit per-sequence offsets");
    return QWEN3_OK;
}

// Per-sequence values (first slots, padding runs) of batches above kInlinePositions sequences go
// to the workspace through kernel arguments, kFillChunk values per launch: a host-to-device copy
// from host memory the caller does not pin would make the host wait for it, and a captured copy
// would read host memory that no longer exists when the graph is replayed.
constexpr int kFillChunk = 256;
struct I32Chunk {
    int32_t v[kFillChunk];
};
__global__ __launch_bounds__(kFillChunk) void fill_i32_kernel(int32_t* __restrict__ dst, I32Chunk c, int n) {
    const int i = threadIdx.x;
    if (i < n) dst[i] = c.v[i];
}

hipError_t upload_i32(int32_t* dst, const std::vector<int32_t>& host, hipStream_t s) {
    for (size_t o = 0; o < host.size(); o += kFillChunk) {
        const int n = (int)std::min<size_t>(kFillChunk, host.size() - o);
        I32Chunk c;
        std::memcpy(c.v, host.data() + o, sizeof(int32_t) * n);
        fill_i32_kernel<<<1, kFillChunk, 0, s>>>(dst + o, c, n);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ------------------------------------------------------------------ profiling helpers
hipEvent_t take_event(qwen3_layer* L) {
    if (!L->free_events.empty()) {
        hipEvent_t e = L->free_events.back();
        L->free_events.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

int stage_id(qwen3_layer* L, const char* name) {
    for (size_t i = 0; i < L->stage_names.size(); ++i)
        if (L->stage_names[i] == name) return (int)i;
    L->stage_names.emplace_back(name);
    return (int)L->stage_names.size() - 1;
}

template <typename F>
qwen3_status run_stage(qwen3_layer* L, bool prof, const char* name, hipStream_t s, F&& launch) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (prof) {
        std::lock_guard<std::mutex> g(L->prof_mu);
        e0 = take_event(L);
        e1 = take_event(L);
        if (e0) hipEventRecord(e0, s);
    }
    const hipError_t err = launch();
    if (err != hipSuccess) return fail(QWEN3_ERR_DEVICE, "%s: %s", name, hipGetErrorString(err));
    if (prof && e0 && e1) {
        std::lock_guard<std::mutex> g(L->prof_mu);
        hipEventRecord(e1, s);
        L->pending.push_back({stage_id(L, name), e0, e1});
    }
    return QWEN3_OK;
}

GemmArgs gemm(const void* a, std::initializer_list<const void*> b, std::initializer_list<int> rows, void* out,
              const void* resid, int M, int N, int K, Epilogue epi) {
    GemmArgs g{};
    g.a = a;
    int i = 0;
    for (const void* p : b) g.b[i++] = p;
    g.nseg = i;
    i = 0;
    for (int r : rows) g.b_rows[i++] = r;
    g.out = out;
    g.resid = resid;
    g.M = M;
    g.N = N;
    g.K = K;
    g.epi = epi;
    return g;
}

// The whole layer on M = B*T tokens.  `pos` gives the position of token 0 of each sequence.
qwen3_status run_layer(qwen3_layer* L, const void* x, void* y, int B, int T, void* kc, void* vc, int cap,
                       char* ws, const Layout& lay, const SeqPositions& pos, const LocalAttn& local, bool decode,
                       hipStream_t s, bool allow_profiling = true) {
    const qwen3_config& c = L->cfg;
    const DType t = dt(c);
    const int M = B * T, H = c.hidden_size, D = c.head_dim, I = c.intermediate_size;
    const int Hq = c.num_attention_heads, Hkv = c.num_key_value_heads;
    const bool bf = t == DType::BF16;
    void* h = ws + lay.h;
    void* qkv = ws + lay.qkv;
    void* qhat = ws + lay.qhat;
    void* attn = ws + lay.attn;
    void* x1 = ws + lay.x1;
    void* h2 = ws + lay.h2;
    void* act = ws + lay.act;
    const float eps = c.rms_norm_eps;
    const float gain_off = c.norm_unit_offset ? 1.f : 0.f;
    auto proj = [&](const GemmArgs& g) {
        if (!bf) return launch_gemm_f32(g, s);
        return g.M <= 64 ? launch_gemv_bf16(g, s) : launch_gemm_bf16(g, s);
    };
    float* part = reinterpret_cast<float*>(ws + lay.part_gemm);   // split-K fp32 slabs
    qwen3_status st;
    const bool prof = allow_profiling && L->profiling;
#define STAGE(name, expr)                                    \
    if ((st = run_stage(L, prof, name, s, [&]() { return (expr); })) != QWEN3_OK) return st;

    QkRopeArgs qa{};
    qa.qkv = qkv;
    qa.q_norm = L->w.q_norm;
    qa.k_norm = L->w.k_norm;
    qa.qhat = qhat;
    qa.k_cache = kc;
    qa.v_cache = vc;
    qa.pos = pos;
    qa.local = local;
    qa.B = B;
    qa.T = T;
    qa.Hq = Hq;
    qa.Hkv = Hkv;
    qa.D = D;
    qa.cap = cap;
    qa.eps = eps;
    std::memcpy(qa.turns, L->rope_turns, sizeof(qa.turns));
    qa.goff = gain_off;
    qa.rotary_dim = c.rotary_dim;
    qa.adjacent = c.rope_adjacent_pairs;
    // QKV projection; for prefill shapes (256 x 256 or 256 x 128 ping-pong tiles, else 128 x 128) the
    // QK-norm + RoPE + cache write runs in the GEMM's epilogue (one kernel), otherwise as its own
    // kernel.  The fused epilogue reads each row's RoPE angles and cache slot from a table that
    // the input RMSNorm writes into the x1 and h2 regions, which are free until o_proj.
    const GemmArgs gq = gemm(h, {L->w.q_proj, L->w.k_proj, L->w.v_proj}, {Hq * D, Hkv * D, Hkv * D}, qkv, nullptr,
                             M, (Hq + 2 * Hkv) * D, H, Epilogue::Store);
    if (bf && !decode) {
        qa.rope_cs = reinterpret_cast<const float*>(x1);
        qa.rope_slot = reinterpret_cast<const int32_t*>(h2);
    }
    const bool fused_qkv = bf && !decode && gemm_qkv_fusable(gq, qa);
    if (fused_qkv) {
        RopeTable rt{};
        rt.cs = static_cast<float*>(x1);
        rt.slot = static_cast<int32_t*>(h2);
        rt.pos = pos;
        rt.T = T;
        std::memcpy(rt.turns, L->rope_turns, sizeof(rt.turns));
        STAGE("rmsnorm_input", launch_rmsnorm_rope(x, L->w.input_layernorm, h, M, H, eps, gain_off, rt, s));
    } else {
        STAGE("rmsnorm_input", launch_rmsnorm(x, t, L->w.input_layernorm, h, t, M, H, eps, gain_off, s));
    }
    if (fused_qkv) {
        STAGE("gemm_qkv_qknorm_rope", launch_gemm_qkv_qkrope(gq, qa, s));
    } else if (const SkinnyPlan sq = skinny_qkv_split(c, M); sq.kslices > 1) {
        GemmArgs gs = gq;
        gs.out = part;
        gs.epi = Epilogue::PartialF32;
        gs.splits = sq.kslices;
        qa.qkv_part = part;
        qa.qkv_splits = sq.kslices;
        qa.qkv_sum = qkv;
        STAGE("gemm_qkv", launch_gemv_bf16(gs, s));
        STAGE("qknorm_rope", launch_qknorm_rope(qa, t, s));
    } else {
        STAGE("gemm_qkv", proj(gq));
        STAGE("qknorm_rope", launch_qknorm_rope(qa, t, s));
    }
    AttnArgs aa{};
    aa.qhat = qhat;
    aa.k_cache = kc;
    aa.v_cache = vc;
    aa.out = attn;
    aa.pos = pos;
    aa.local = local;
    aa.B = B;
    aa.T = T;
    aa.Hq = Hq;
    aa.Hkv = Hkv;
    aa.D = D;
    aa.cap = cap;
    aa.scale = (float)(1.0 / std::sqrt((double)D));
    aa.q_norm = L->w.q_norm;
    aa.k_norm = L->w.k_norm;
    aa.goff = gain_off;
    if (!bf) {
        STAGE("attention", launch_attention_f32(aa, s));
    } else if (decode) {
        DecodeAttnArgs da{};
        da.a = aa;
        da.part_o = reinterpret_cast<float*>(ws + lay.part_o);
        da.part_ml = reinterpret_cast<float*>(ws + lay.part_ml);
        da.splits = lay.splits;
        da.split_keys = kDecodeSplitKeys;
        STAGE("attention_decode_split", launch_attention_decode_split_bf16(da, s));
        STAGE("attention_decode_combine", launch_attention_decode_combine_bf16(da, s));
    } else {
        STAGE("attention", launch_attention_prefill_bf16(aa, s));
    }
    // o_proj + residual.  With few output tiles the K range is split and the fp32 partial sums are
    // added to the residual inside the post-attention RMSNorm (which reads x1 anyway).
    const int so = bf ? gemm_bf16_splits(M, H, Hq * D) : 1;
    if (so > 1) {
        GemmArgs go = gemm(attn, {L->w.o_proj}, {H}, part, nullptr, M, H, Hq * D, Epilogue::PartialF32);
        go.splits = so;
        STAGE("gemm_o_residual", launch_gemm_bf16(go, s));
        STAGE("rmsnorm_post", launch_residual_rmsnorm(x, t, part, so, static_cast<float*>(x1),
                                                      L->w.post_attention_layernorm, h2, t, M, H, eps, gain_off, s));
    } else {
        STAGE("gemm_o_residual", proj(gemm(attn, {L->w.o_proj}, {H}, x1, x, M, H, Hq * D, Epilogue::ResidToF32)));
        STAGE("rmsnorm_post",
              launch_rmsnorm(x1, DType::F32, L->w.post_attention_layernorm, h2, t, M, H, eps, gain_off, s));
    }
    STAGE("gemm_gate_up_swiglu", proj(gemm(h2, {L->w.gate_proj, L->w.up_proj}, {I, I}, act, nullptr, M, I, H,
                                           Epilogue::SwiGLU)));
    // down_proj + residual: in the GEMM epilogue, or with few output tiles as a split-K GEMM whose
    // fp32 partial slabs a small pass adds to the residual
    const int sd = bf ? gemm_bf16_splits(M, H, I) : 1;
    if (sd > 1) {
        GemmArgs gd = gemm(act, {L->w.down_proj}, {H}, part, nullptr, M, H, I, Epilogue::PartialF32);
        gd.splits = sd;
        STAGE("gemm_down_residual", launch_gemm_bf16(gd, s));
        STAGE("residual_add", launch_residual_sum_bf16(static_cast<const float*>(x1), part, sd, y, (int64_t)M * H, s));
    } else {
        STAGE("gemm_down_residual", proj(gemm(act, {L->w.down_proj}, {H}, y, x1, M, H, I, Epilogue::ResidF32In)));
    }
#undef STAGE
    return QWEN3_OK;
}

}  // namespace

extern "C" {

const char* qwen3_status_string(qwen3_status s) {
    switch (s) {
        case QWEN3_OK: return "ok";
        case QWEN3_ERR_INVALID_ARGUMENT: return "invalid argument";
        case QWEN3_ERR_UNSUPPORTED: return "unsupported";
        case QWEN3_ERR_OUT_OF_RANGE: return "out of range";
        case QWEN3_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case QWEN3_ERR_DEVICE: return "device error";
    }
    return "unknown status";
}

const char* qwen3_last_error(void) { return g_last_error.c_str(); }

qwen3_status qwen3_layer_create(const qwen3_config* config, const qwen3_layer_weights* weights,
                                qwen3_layer** out_layer) {
    if (!out_layer) return fail(QWEN3_ERR_INVALID_ARGUMENT, "out_layer is NULL");
    *out_layer = nullptr;
    qwen3_status st = validate_config(config);
    if (st != QWEN3_OK) return st;
    if (!weights) return fail(QWEN3_ERR_INVALID_ARGUMENT, "weights is NULL");
    const void* ptrs[] = {weights->input_layernorm, weights->q_proj, weights->k_proj, weights->v_proj,
                          weights->q_norm, weights->k_norm, weights->o_proj, weights->post_attention_layernorm,
                          weights->gate_proj, weights->up_proj, weights->down_proj};
    for (const void* p : ptrs) {
        if (!p) return fail(QWEN3_ERR_INVALID_ARGUMENT, "a weight pointer is NULL");
        if (!aligned16(p)) return fail(QWEN3_ERR_INVALID_ARGUMENT, "weight pointers must be 16-byte aligned");
    }
    qwen3_layer* L = new qwen3_layer();
    L->cfg = *config;
    L->w = *weights;
    // RoPE frequencies ("17. A modern architecture: Qwen3", Rotary position embeddings):
    // omega_i = theta^(-2i/r) over the r = rotary_dim rotated features, kept in fp64 and in turns
    // for the kernel's exact range reduction; linear position scaling is folded in.
    if (L->cfg.rotary_dim == 0) L->cfg.rotary_dim = config->head_dim;
    if (L->cfg.rope_position_scale == 0.0) L->cfg.rope_position_scale = 1.0;
    const int r = L->cfg.rotary_dim;
    for (int i = 0; i < 64; ++i)
        L->rope_turns[i] = i < r / 2 ? L->cfg.rope_position_scale * std::pow(config->rope_theta, -2.0 * i / r) /
                                           (2.0 * M_PI)
                                     : 0.0;
    *out_layer = L;
    return QWEN3_OK;
}

void qwen3_layer_destroy(qwen3_layer* L) {
    if (!L) return;
    for (auto& r : L->pending) {
        hipEventDestroy(r.start);
        hipEventDestroy(r.stop);
    }
    for (hipEvent_t e : L->free_events) hipEventDestroy(e);
    delete L;
}

qwen3_status qwen3_layer_workspace_size(const qwen3_layer* L, int32_t batch, int32_t seq_len, int32_t cap,
                                        size_t* bytes) {
    if (!bytes) return fail(QWEN3_ERR_INVALID_ARGUMENT, "bytes is NULL");
    qwen3_status st = check_sizes(L, batch, seq_len, cap);
    if (st != QWEN3_OK) return st;
    // prefill (with room for device-side start positions) or decode over `cap` slots
    *bytes = std::max(make_layout(L->cfg, batch, seq_len, 0).total, make_layout(L->cfg, batch, 1, cap).total);
    return QWEN3_OK;
}

qwen3_status qwen3_layer_workspace_layout(const qwen3_layer* L, int32_t batch, int32_t seq_len, int32_t cap,
                                          qwen3_workspace_layout* out) {
    if (!out) return fail(QWEN3_ERR_INVALID_ARGUMENT, "layout is NULL");
    qwen3_status st = check_sizes(L, batch, seq_len, cap);
    if (st != QWEN3_OK) return st;
    const Layout lay = make_layout(L->cfg, batch, seq_len, cap);
    out->h = lay.h;
    out->qkv = lay.qkv;
    out->qhat = lay.qhat;
    out->attn = lay.attn;
    out->x1 = lay.x1;
    out->h2 = lay.h2;
    out->act = lay.act;
    out->part_gemm = lay.part_gemm;
    out->lens = lay.lens;
    out->part_o = lay.part_o;
    out->part_ml = lay.part_ml;
    out->total = lay.total;
    out->decode_splits = lay.splits;
    out->split_keys = kDecodeSplitKeys;
    return QWEN3_OK;
}

}  // extern "C"

namespace {

qwen3_status prefill_impl(qwen3_layer* L, const void* x, void* y, int32_t batch, int32_t seq_len,
                          const int32_t* start_positions, const int32_t* pad_lens, const LocalAttn& local,
                          void* k_cache, void* v_cache, int32_t cache_capacity, void* workspace,
                          size_t workspace_bytes, void* stream) {
    qwen3_status st = check_sizes(L, batch, seq_len, cache_capacity);
    if (st != QWEN3_OK) return st;
    if (!x || !y || !k_cache || !v_cache || !workspace)
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "x, y, k_cache, v_cache and workspace must be non-NULL");
    if (!aligned16(x) || !aligned16(y) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace))
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
    bool any_start = false, any_pad = false;
    for (int b = 0; b < batch; ++b) {
        const int64_t p0 = start_positions ? start_positions[b] : 0;
        const int64_t pad = pad_lens ? pad_lens[b] : 0;
        if (p0 < 0) return fail(QWEN3_ERR_OUT_OF_RANGE, "start_positions[%d] = %lld is negative", b, (long long)p0);
        if (pad < 0 || pad > seq_len)
            return fail(QWEN3_ERR_OUT_OF_RANGE, "pad_lens[%d] = %lld is outside [0, seq_len = %d]", b, (long long)pad,
                        seq_len);
        if (p0 + seq_len > cache_capacity)
            return fail(QWEN3_ERR_OUT_OF_RANGE, "sequence %d: start %lld + seq_len %d exceeds cache_capacity %d", b,
                        (long long)p0, seq_len, cache_capacity);
        if (p0 + seq_len > L->cfg.max_position_embeddings)
            return fail(QWEN3_ERR_OUT_OF_RANGE, "sequence %d: start %lld + seq_len %d exceeds max_position_embeddings %d",
                        b, (long long)p0, seq_len, L->cfg.max_position_embeddings);
        any_start |= p0 != 0;
        any_pad |= pad != 0;
    }
    const Layout lay = make_layout(L->cfg, batch, seq_len, 0);
    const bool via_workspace = (any_start || any_pad) && batch > kInlinePositions;
    const size_t need = via_workspace ? lay.total : lay.prefill_end;
    if (workspace_bytes < need)
        return fail(QWEN3_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, prefill needs %zu", workspace_bytes, need);
    char* ws = static_cast<char*>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    SeqPositions pos{};
    if (via_workspace) {
        std::vector<int32_t> host(3 * (size_t)batch, 0);
        for (int b = 0; b < batch; ++b) {
            host[b] = start_positions ? start_positions[b] : 0;
            host[batch + b] = host[b];
            host[2 * batch + b] = pad_lens ? pad_lens[b] : 0;
        }
        const hipError_t e = upload_i32(reinterpret_cast<int32_t*>(ws + lay.lens), host, s);
        if (e != hipSuccess) return fail(QWEN3_ERR_DEVICE, "uploading start positions: %s", hipGetErrorString(e));
        pos.dev = reinterpret_cast<const int32_t*>(ws + lay.lens);
        if (any_pad) {
            pos.dev_pad = pos.dev + batch;
            pos.n_pad_inline = batch;
        }
    } else {
        if (any_start) {
            pos.n_inline = batch;
            for (int b = 0; b < batch; ++b) pos.inl[b] = start_positions[b];
        }
        if (any_pad) {
            pos.n_pad_inline = batch;
            for (int b = 0; b < batch; ++b) {
                pos.pad_lo[b] = start_positions ? start_positions[b] : 0;
                pos.pad_n[b] = pad_lens[b];
            }
        }
    }
    return run_layer(L, x, y, batch, seq_len, k_cache, v_cache, cache_capacity, ws, lay, pos, local, false, s);
}

}  // namespace

extern "C" {

qwen3_status qwen3_layer_prefill_padded(qwen3_layer* L, const void* x, void* y, int32_t batch, int32_t seq_len,
                                        const int32_t* start_positions, const int32_t* pad_lens, void* k_cache,
                                        void* v_cache, int32_t cache_capacity, void* workspace,
                                        size_t workspace_bytes, void* stream) {
    return prefill_impl(L, x, y, batch, seq_len, start_positions, pad_lens, LocalAttn{0, 0, 0}, k_cache, v_cache,
                        cache_capacity, workspace, workspace_bytes, stream);
}

qwen3_status qwen3_layer_prefill_window(qwen3_layer* L, const void* x, void* y, int32_t batch, int32_t seq_len,
                                        const int32_t* start_positions, int32_t window, int32_t sinks,
                                        void* k_cache, void* v_cache, int32_t cache_capacity, void* workspace,
                                        size_t workspace_bytes, void* stream) {
    if (window < 0 || sinks < 0)
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "window (%d) and sinks (%d) must be non-negative", window, sinks);
    return prefill_impl(L, x, y, batch, seq_len, start_positions, nullptr, LocalAttn{window, window > 0 ? sinks : 0, 0},
                        k_cache, v_cache, cache_capacity, workspace, workspace_bytes, stream);
}

qwen3_status qwen3_layer_prefill_at(qwen3_layer* L, const void* x, void* y, int32_t batch, int32_t seq_len,
                                    const int32_t* start_positions, void* k_cache, void* v_cache,
                                    int32_t cache_capacity, void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl(L, x, y, batch, seq_len, start_positions, nullptr, LocalAttn{0, 0, 0}, k_cache, v_cache,
                        cache_capacity, workspace, workspace_bytes, stream);
}

qwen3_status qwen3_layer_prefill(qwen3_layer* L, const void* x, void* y, int32_t batch, int32_t seq_len,
                                 void* k_cache, void* v_cache, int32_t cache_capacity, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    return prefill_impl(L, x, y, batch, seq_len, nullptr, nullptr, LocalAttn{0, 0, 0}, k_cache, v_cache,
                        cache_capacity, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

qwen3_status decode_impl(qwen3_layer* L, const void* x, void* y, int32_t batch, const int32_t* cache_lens,
                         const int32_t* pad_starts, const int32_t* pad_lens, const LocalAttn& local, void* k_cache,
                         void* v_cache, int32_t cache_capacity, void* workspace, size_t workspace_bytes,
                         void* stream, bool allow_profiling = true) {
    qwen3_status st = check_sizes(L, batch, 1, cache_capacity);
    if (st != QWEN3_OK) return st;
    if (!x || !y || !k_cache || !v_cache || !workspace || !cache_lens)
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "x, y, cache_lens, k_cache, v_cache and workspace must be non-NULL");
    if ((pad_starts == nullptr) != (pad_lens == nullptr))
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "pad_starts and pad_lens must both be given or both be NULL");
    if (!aligned16(x) || !aligned16(y) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace))
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
    bool any_pad = false;
    for (int b = 0; b < batch; ++b) {
        const int n = cache_lens[b];
        if (n < 0 || (!local.rolling && n >= cache_capacity))
            return fail(QWEN3_ERR_OUT_OF_RANGE, "cache_lens[%d] = %d leaves no free slot in a cache of %d", b, n,
                        cache_capacity);
        if (n >= L->cfg.max_position_embeddings)
            return fail(QWEN3_ERR_OUT_OF_RANGE, "position %d of sequence %d reaches max_position_embeddings %d", n, b,
                        L->cfg.max_position_embeddings);
        if (pad_lens) {
            const int64_t lo = pad_starts[b], pn = pad_lens[b];
            if (lo < 0 || pn < 0 || lo + pn > n)
                return fail(QWEN3_ERR_OUT_OF_RANGE, "sequence %d: padding [%lld, %lld) is not inside its %d cached slots",
                            b, (long long)lo, (long long)(lo + pn), n);
            any_pad |= pn != 0;
        }
    }
    const Layout lay = make_layout(L->cfg, batch, 1, cache_capacity);
    if (workspace_bytes < lay.total)
        return fail(QWEN3_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, decode needs %zu", workspace_bytes,
                    lay.total);
    char* ws = static_cast<char*>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    SeqPositions pos{};
    if (batch <= kInlinePositions) {
        pos.n_inline = batch;
        for (int b = 0; b < batch; ++b) pos.inl[b] = cache_lens[b];
        if (any_pad) {
            pos.n_pad_inline = batch;
            for (int b = 0; b < batch; ++b) {
                pos.pad_lo[b] = pad_starts[b];
                pos.pad_n[b] = pad_lens[b];
            }
        }
    } else {
        std::vector<int32_t> host(3 * (size_t)batch, 0);
        for (int b = 0; b < batch; ++b) {
            host[b] = cache_lens[b];
            host[batch + b] = any_pad ? pad_starts[b] : 0;
            host[2 * batch + b] = any_pad ? pad_lens[b] : 0;
        }
        const hipError_t e = upload_i32(reinterpret_cast<int32_t*>(ws + lay.lens), host, s);
        if (e != hipSuccess) return fail(QWEN3_ERR_DEVICE, "uploading cache_lens: %s", hipGetErrorString(e));
        pos.dev = reinterpret_cast<const int32_t*>(ws + lay.lens);
        if (any_pad) {
            pos.dev_pad = pos.dev + batch;
            pos.n_pad_inline = batch;
        }
    }
    return run_layer(L, x, y, batch, 1, k_cache, v_cache, cache_capacity, ws, lay, pos, local, true, s,
                     allow_profiling);
}

// ------------------------------------------------------------------ allocation-free decode
// For callers that cannot allocate (code under stream capture, tight serving loops): the decode
// intermediates live in this file-scope device array instead of a caller workspace.  Each GPU
// the library runs on holds its own copy from module load until the process ends.  In host code
// `scratch` only names the symbol: its device address comes from hipGetSymbolAddress, taken once
// per device (with that device current) and kept below.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

qwen3_status scratch_of_current_device(hipStream_t s, char** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(QWEN3_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(QWEN3_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
    if (s) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(s, &sdev);
        if (e != hipSuccess) return fail(QWEN3_ERR_DEVICE, "hipStreamGetDevice: %s", hipGetErrorString(e));
        if (sdev != dev)
            return fail(QWEN3_ERR_INVALID_ARGUMENT, "the stream belongs to device %d, the current device is %d",
                        (int)sdev, dev);
    }
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(QWEN3_ERR_DEVICE, "locating the scratch array on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = static_cast<char*>(ptr);
    }
    *out = g_scratch_ptr[dev];
    return QWEN3_OK;
}

}  // namespace

extern "C" {

qwen3_status qwen3_layer_decode_padded(qwen3_layer* L, const void* x, void* y, int32_t batch,
                                       const int32_t* cache_lens, const int32_t* pad_starts, const int32_t* pad_lens,
                                       void* k_cache, void* v_cache, int32_t cache_capacity, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    return decode_impl(L, x, y, batch, cache_lens, pad_starts, pad_lens, LocalAttn{0, 0, 0}, k_cache, v_cache,
                       cache_capacity, workspace, workspace_bytes, stream);
}

qwen3_status qwen3_layer_decode_window(qwen3_layer* L, const void* x, void* y, int32_t batch,
                                       const int32_t* positions, int32_t window, int32_t sinks, int32_t rolling,
                                       void* k_cache, void* v_cache, int32_t cache_capacity, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    if (window < 0 || sinks < 0)
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "window (%d) and sinks (%d) must be non-negative", window, sinks);
    if (rolling) {
        if (window == 0) return fail(QWEN3_ERR_INVALID_ARGUMENT, "a rolling buffer needs a window > 0");
        if ((int64_t)sinks + window != cache_capacity)
            return fail(QWEN3_ERR_INVALID_ARGUMENT, "a rolling buffer holds sinks + window = %lld slots, not %d",
                        (long long)sinks + window, cache_capacity);
    }
    const LocalAttn local{window, window > 0 ? sinks : 0, rolling ? 1 : 0};
    return decode_impl(L, x, y, batch, positions, nullptr, nullptr, local, k_cache, v_cache, cache_capacity,
                       workspace, workspace_bytes, stream);
}

qwen3_status qwen3_layer_decode(qwen3_layer* L, const void* x, void* y, int32_t batch, const int32_t* cache_lens,
                                void* k_cache, void* v_cache, int32_t cache_capacity, void* workspace,
                                size_t workspace_bytes, void* stream) {
    return decode_impl(L, x, y, batch, cache_lens, nullptr, nullptr, LocalAttn{0, 0, 0}, k_cache, v_cache,
                       cache_capacity, workspace, workspace_bytes, stream);
}

qwen3_status qwen3_layer_decode_noalloc(qwen3_layer* L, const void* x, void* y, int32_t batch,
                                        const int32_t* cache_lens, void* k_cache, void* v_cache,
                                        int32_t cache_capacity, void* stream) {
    qwen3_status st = check_sizes(L, batch, 1, cache_capacity);
    if (st != QWEN3_OK) return st;
    const size_t need = make_layout(L->cfg, batch, 1, cache_capacity).total;
    if (need > kScratchBytes)
        return fail(QWEN3_ERR_WORKSPACE_TOO_SMALL,
                    "a decode of %d sequences over %d cache slots needs %zu bytes of scratch; the allocation-free "
                    "entry point holds %zu",
                    batch, cache_capacity, need, kScratchBytes);
    if (!x || !y || !k_cache || !v_cache || !cache_lens)
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "x, y, cache_lens, k_cache and v_cache must be non-NULL");
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = nullptr;
    if ((st = scratch_of_current_device(s, &ws)) != QWEN3_OK) return st;
    // no profiling events here even when profiling is on: creating them allocates
    return decode_impl(L, x, y, batch, cache_lens, nullptr, nullptr, LocalAttn{0, 0, 0}, k_cache, v_cache,
                       cache_capacity, ws, kScratchBytes, stream, false);
}

qwen3_status qwen3_rmsnorm(const void* x, const void* weight, void* y, int64_t rows, int32_t width, float eps,
                           qwen3_dtype dtype, void* stream) {
    return qwen3_rmsnorm_gain_offset(x, weight, y, rows, width, eps, 0.f, dtype, stream);
}

qwen3_status qwen3_rmsnorm_gain_offset(const void* x, const void* weight, void* y, int64_t rows, int32_t width,
                                       float eps, float gain_offset, qwen3_dtype dtype, void* stream) {
    if (!std::isfinite(gain_offset)) return fail(QWEN3_ERR_INVALID_ARGUMENT, "gain_offset must be finite");
    if (!x || !weight || !y) return fail(QWEN3_ERR_INVALID_ARGUMENT, "x, weight and y must be non-NULL");
    if (rows <= 0 || width <= 0) return fail(QWEN3_ERR_INVALID_ARGUMENT, "rows and width must be positive");
    if (!aligned16(x) || !aligned16(weight) || !aligned16(y))
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
    if (dtype != QWEN3_F32 && dtype != QWEN3_BF16) return fail(QWEN3_ERR_INVALID_ARGUMENT, "unknown dtype");
    if (width % 8) return fail(QWEN3_ERR_UNSUPPORTED, "width must be a multiple of 8");
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(QWEN3_ERR_INVALID_ARGUMENT, "eps must be non-negative");
    const DType t = dtype == QWEN3_BF16 ? DType::BF16 : DType::F32;
    const hipError_t e = launch_rmsnorm(x, t, weight, y, t, rows, width, eps, gain_offset,
                                        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(QWEN3_ERR_DEVICE, "rmsnorm: %s", hipGetErrorString(e));
    return QWEN3_OK;
}

qwen3_status qwen3_probe_mfma_rate(float* out, int32_t workgroups, int32_t iterations, void* stream) {
    if (!out) return fail(QWEN3_ERR_INVALID_ARGUMENT, "out must be non-NULL");
    if (workgroups < 1 || iterations < 1)
        return fail(QWEN3_ERR_INVALID_ARGUMENT, "workgroups (%d) and iterations (%d) must be positive", workgroups,
                    iterations);
    const hipError_t e = launch_mfma_probe(out, workgroups, iterations, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(QWEN3_ERR_DEVICE, "mfma probe: %s", hipGetErrorString(e));
    return QWEN3_OK;
}

qwen3_status qwen3_layer_set_profiling(qwen3_layer* L, int32_t enabled) {
    if (!L) return fail(QWEN3_ERR_INVALID_ARGUMENT, "layer is NULL");
    L->profiling = enabled != 0;
    return QWEN3_OK;
}

qwen3_status qwen3_layer_read_profile(qwen3_layer* L, qwen3_stage_time* out, int32_t max_entries, int32_t* n) {
    if (!L || !n || (max_entries > 0 && !out)) return fail(QWEN3_ERR_INVALID_ARGUMENT, "NULL argument");
    std::lock_guard<std::mutex> g(L->prof_mu);
    std::vector<double> total(L->stage_names.size(), 0.0);
    std::vector<int> count(L->stage_names.size(), 0);
    qwen3_status st = QWEN3_OK;
    for (auto& r : L->pending) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(r.stop);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
        if (e != hipSuccess) st = fail(QWEN3_ERR_DEVICE, "profile events: %s", hipGetErrorString(e));
        total[r.stage] += ms;
        count[r.stage] += 1;
        L->free_events.push_back(r.start);
        L->free_events.push_back(r.stop);
    }
    L->pending.clear();
    int k = 0;
    for (size_t i = 0; i < L->stage_names.size(); ++i) {
        if (!count[i]) continue;
        if (k < max_entries) {
            std::memset(out[k].name, 0, sizeof(out[k].name));
            std::strncpy(out[k].name, L->stage_names[i].c_str(), sizeof(out[k].name) - 1);
            out[k].launches = count[i];
            out[k].total_ms = total[i];
        }
        ++k;
    }
    *n = std::min(k, max_entries);
    return st;
}

}  // extern "C"
