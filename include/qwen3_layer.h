/*
 * qwen3_layer.h - C ABI of a Qwen3-style pre-norm decoder layer on one AMD
 * Instinct MI355X (gfx950).
 *
 * The layer computes, for every token x of a sequence,
 *   h    = RMSNorm_in(x)
 *   q,k,v = h Wq^T, h Wk^T, h Wv^T                     (no biases)
 *   qhat = RoPE_p(q_norm(q)), khat = RoPE_p(k_norm(k)) (per head, over head_dim)
 *   o    = causal GQA attention(qhat, khat, v), scale head_dim^-1/2
 *   x1   = x + o Wo^T
 *   y    = x1 + down( silu(gate h2) * up h2 ),  h2 = RMSNorm_post(x1)
 * as defined on "17. A modern architecture: Qwen3" (sections RMSNorm, Rotary
 * position embeddings, Attention with grouped KV heads and Q/K normalization,
 * SwiGLU, The whole model) and "Transformer architectures: from BERT to
 * diffusion, lesson 6" (sections 3 and 5).
 *
 * Conventions for every entry point:
 *  - Device pointers are caller-owned, contiguous, 16-byte aligned and hold the
 *    configuration's dtype (bf16 or fp32) unless stated otherwise.  Weights use
 *    the nn.Linear layout [out_features, in_features], row-major.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Every call is
 *    asynchronous on it and never synchronises the host, except where noted.
 *  - Arguments are validated on the host before anything is launched; on any
 *    status other than QWEN3_OK nothing was launched (QWEN3_ERR_DEVICE excepted:
 *    a launch failed after earlier kernels of the call were queued).
 *    qwen3_last_error() describes the most recent failure of the calling thread.
 *  - The library allocates no device memory after qwen3_layer_create: prefill
 *    and decode use the caller's workspace.
 */
#ifndef QWEN3_LAYER_H
#define QWEN3_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QWEN3_OK = 0,
    QWEN3_ERR_INVALID_ARGUMENT = 1,   /* null pointer, non-positive size, odd head_dim, misalignment */
    QWEN3_ERR_UNSUPPORTED = 2,        /* shape/dtype the kernels do not implement; Hq % Hkv != 0 */
    QWEN3_ERR_OUT_OF_RANGE = 3,       /* tokens beyond the cache or max_position_embeddings */
    QWEN3_ERR_WORKSPACE_TOO_SMALL = 4,
    QWEN3_ERR_DEVICE = 5              /* a HIP call or kernel launch failed */
} qwen3_status;

typedef enum { QWEN3_F32 = 0, QWEN3_BF16 = 1 } qwen3_dtype;

/* The per-layer fields of a Qwen3 config.json ("lesson 6", section 5, printed
 * config; "17. A modern architecture: Qwen3", opening contract).  head_dim is
 * its own field: Hq*head_dim need not equal hidden_size. */
typedef struct {
    int32_t hidden_size;
    int32_t num_attention_heads;      /* Hq */
    int32_t num_key_value_heads;      /* Hkv; Hq must be a multiple of it */
    int32_t head_dim;                 /* D, even */
    int32_t intermediate_size;        /* I */
    int32_t max_position_embeddings;  /* positions must stay below this */
    double  rope_theta;               /* RoPE base: omega_i = theta^(-2i/D) */
    float   rms_norm_eps;             /* added to the mean square inside the root */
    qwen3_dtype dtype;                /* storage type of weights, activations and cache */
    /* RoPE and RMSNorm variants ("17. A modern architecture: Qwen3", sections
     * RMSNorm and Rotary position embeddings, and its exercises).  All zero gives
     * Qwen3 itself. */
    int32_t rotary_dim;               /* features rotated per head (partial RoPE: only the
                                         first rotary_dim, frequencies theta^(-2i/rotary_dim),
                                         the rest pass through); 0 = head_dim; even */
    int32_t rope_adjacent_pairs;      /* 1: pair features (2i, 2i+1) (the original paper);
                                         0: (i, i + rotary_dim/2) (split-half, Qwen/Llama) */
    double  rope_position_scale;      /* linear RoPE scaling: angles use position * scale;
                                         0 = 1 (no scaling) */
    int32_t norm_unit_offset;         /* 1: zero-centred RMSNorm gains (Gemma, Qwen3.5): every
                                         norm of the layer applies (1 + g) instead of g */
} qwen3_config;

/* Device pointers to one layer's tensors (parameter names of the Qwen3
 * checkpoint, "lesson 6" section 6).  Shapes: input_layernorm [H],
 * q_proj [Hq*D, H], k_proj [Hkv*D, H], v_proj [Hkv*D, H], q_norm [D],
 * k_norm [D], o_proj [H, Hq*D], post_attention_layernorm [H],
 * gate_proj [I, H], up_proj [I, H], down_proj [H, I].
 * The handle keeps these pointers (it does not copy or own the tensors): the
 * caller keeps them alive and unchanged until qwen3_layer_destroy. */
typedef struct {
    const void *input_layernorm, *q_proj, *k_proj, *v_proj, *q_norm, *k_norm,
               *o_proj, *post_attention_layernorm, *gate_proj, *up_proj, *down_proj;
} qwen3_layer_weights;

typedef struct qwen3_layer qwen3_layer;

/* Byte offsets, inside the caller's workspace, of the intermediates a call
 * leaves behind (M = batch * seq_len rows; es = 2 for bf16, 4 for fp32):
 *   h     [M, H]            input RMSNorm output (dtype)
 *   qkv   [M, (Hq+2Hkv)*D]  q | k | v projections, token-major (dtype)
 *   qhat  [B, Hq, T, D]     normalised, rotated queries (dtype)
 *   attn  [M, Hq*D]         attention output, token-major (dtype)
 *   x1    [M, H]            residual after attention (always fp32)
 *   h2    [M, H]            post-attention RMSNorm output (dtype)
 *   act   [M, I]            silu(gate) * up (dtype)
 *   part_gemm [P, M, H]     fp32 split-K partial sums of o_proj and down (bf16 prefill
 *                           when even 64 x 128 output tiles are too few to fill the GPU;
 *                           P = 0 otherwise); for bf16
 *                           with M <= 16 and head_dim 128, the QKV projection's split-K
 *                           slabs [P, M, (Hq+2Hkv)*D] (their bf16 sum is stored to qkv)
 *   lens  [3, B]            int32 copies of the first slots (decode cache lengths / prefill
 *                           start positions), padding starts and padding lengths
 *   part_o  [B, Hq, S, D]   fp32 split-KV partial outputs (decode)
 *   part_ml [B, Hq, S, 2]   fp32 split-KV running max (log2 units) and sum
 * where S = number of key splits for cache_capacity keys. */
typedef struct {
    size_t h, qkv, qhat, attn, x1, h2, act, part_gemm, lens, part_o, part_ml;
    size_t total;
    int32_t decode_splits;   /* S */
    int32_t split_keys;      /* keys per split */
} qwen3_workspace_layout;

/* Validates *config and *weights and returns a handle.  Host only: no HIP call
 * is made, and the handle is not tied to a device - each call runs on the device
 * that owns `stream` (the weights must live there).
 * Errors: INVALID_ARGUMENT (null pointer, a size <= 0, odd head_dim, a weight
 * pointer not 16-byte aligned), UNSUPPORTED (Hq % Hkv != 0 - the pages raise
 * on it in Qwen3Attention; a dtype or head_dim the kernels lack: bf16 needs
 * head_dim 128, fp32 head_dim <= 128; bf16 widths H, I, Hq*D, Hkv*D must be
 * multiples of 128, 1/2/4/8 query heads per KV head), INVALID_ARGUMENT also for
 * an odd or out-of-range rotary_dim, a negative or non-finite
 * rope_position_scale, or flags other than 0/1. */
qwen3_status qwen3_layer_create(const qwen3_config* config, const qwen3_layer_weights* weights,
                                qwen3_layer** out_layer);

/* Frees the handle (not the weights).  NULL is ignored. */
void qwen3_layer_destroy(qwen3_layer* layer);

/* Workspace bytes for a prefill of [batch, seq_len] tokens (also onto a
 * non-empty cache) and for a decode of `batch` tokens over caches of
 * `cache_capacity` slots (pass seq_len = 1 for decode only).  Host only.
 * cache_capacity is an argument because the decode attention's per-split
 * partial results grow with the cache length it may have to cover. */
qwen3_status qwen3_layer_workspace_size(const qwen3_layer* layer, int32_t batch, int32_t seq_len,
                                        int32_t cache_capacity, size_t* bytes);

/* Offsets of the intermediates within that workspace (see the struct). */
qwen3_status qwen3_layer_workspace_layout(const qwen3_layer* layer, int32_t batch, int32_t seq_len,
                                          int32_t cache_capacity, qwen3_workspace_layout* layout);

/* Prefill: x, y are [batch, seq_len, H]; token t of each sequence sits at
 * position t (empty cache).  Writes khat and v of every token to slot t of
 * k_cache / v_cache, laid out [batch, Hkv, cache_capacity, D] (keys are cached
 * already rotated, "17. A modern architecture: Qwen3", end of Rotary position
 * embeddings).  y may alias x.
 * Errors: INVALID_ARGUMENT, OUT_OF_RANGE (seq_len > cache_capacity or
 * seq_len > max_position_embeddings), WORKSPACE_TOO_SMALL, DEVICE. */
qwen3_status qwen3_layer_prefill(qwen3_layer* layer, const void* x, void* y, int32_t batch,
                                 int32_t seq_len, void* k_cache, void* v_cache,
                                 int32_t cache_capacity, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Prefill onto a non-empty cache (chunked or prefix prefill): x, y are
 * [batch, seq_len, H]; start_positions is a HOST array [batch] (NULL means all
 * zero, which is qwen3_layer_prefill).  Sequence b already holds
 * start_positions[b] rotated keys and values in slots 0..start_positions[b]-1;
 * its token t sits at position start_positions[b] + t, its khat / v go to that
 * slot, and it attends keys 0..start_positions[b] + t of its own sequence
 * ("17. A modern architecture: Qwen3", section The whole model: positions
 * continue from the cache length; "Transformer architectures: from BERT to
 * diffusion, lesson 6", section 8: a shared prefix's keys and values are
 * computed once and reused).  Running a prompt as prefill(T1) followed by
 * prefill_at(T2, start T1) gives the rows of prefill(T1 + T2).  Up to 64
 * sequences the start positions travel as launch arguments; for more, small
 * kernels whose launch arguments carry them (256 values each) write them into
 * the workspace (which must then also cover the `lens` region of
 * qwen3_layer_workspace_layout), with no host-to-device copy.  y may alias x.
 * Errors: INVALID_ARGUMENT, OUT_OF_RANGE (start_positions[b] < 0,
 * start_positions[b] + seq_len > cache_capacity or > max_position_embeddings),
 * WORKSPACE_TOO_SMALL, DEVICE. */
qwen3_status qwen3_layer_prefill_at(qwen3_layer* layer, const void* x, void* y, int32_t batch,
                                    int32_t seq_len, const int32_t* start_positions, void* k_cache,
                                    void* v_cache, int32_t cache_capacity, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Prefill of left-padded rows ("Transformer architectures: from BERT to
 * diffusion, lesson 6", section 8, batched generation: prompts of different
 * lengths are padded on the left so that every row ends in the same column;
 * padding gets no attention; positions are counted from each row's first real
 * token; every token may attend itself).  As qwen3_layer_prefill_at, plus
 * pad_lens, a HOST array [batch] (NULL = no padding): the first pad_lens[b]
 * tokens of sequence b are padding.  Their keys and values are still written to
 * slots start_positions[b] .. start_positions[b] + pad_lens[b] - 1 (the padding
 * run), but no other token attends them; a padding token attends the keys before
 * the run (a shared prefix) and itself.  Positions count real tokens: token t
 * of sequence b sits at position start_b + t - pad_b when it is real and at
 * max(start_b - 1, 0) when it is padding; its cache slot is start_b + t either
 * way.  Later decode steps pass the same run to qwen3_layer_decode_padded.
 * Up to 64 sequences the per-sequence values travel as launch arguments; for
 * more they are written into the workspace's `lens` region by small kernels
 * whose launch arguments carry them (no host-to-device copy).
 * Errors: as qwen3_layer_prefill_at, plus OUT_OF_RANGE for pad_lens[b] < 0 or
 * pad_lens[b] > seq_len. */
qwen3_status qwen3_layer_prefill_padded(qwen3_layer* layer, const void* x, void* y, int32_t batch,
                                        int32_t seq_len, const int32_t* start_positions,
                                        const int32_t* pad_lens, void* k_cache, void* v_cache,
                                        int32_t cache_capacity, void* workspace, size_t workspace_bytes,
                                        void* stream);

/* Decode: one new token per sequence; x, y are [batch, 1, H].  cache_lens is a
 * HOST array [batch]: sequence b already holds cache_lens[b] rotated keys and
 * values in slots 0..cache_lens[b]-1.  The new token is at position
 * cache_lens[b], its khat / v are written to that slot and it attends keys
 * 0..cache_lens[b] of its own sequence.  cache_lens is not modified (the caller
 * advances it).  y may alias x.  Up to 64 sequences the lengths travel to the
 * kernels as launch arguments; for more, small kernels whose launch arguments
 * carry them (256 values each) write them into the workspace, with no
 * host-to-device copy.  Either way the host array may be reused once the call
 * returns.
 * Errors: INVALID_ARGUMENT, OUT_OF_RANGE (cache_lens[b] < 0,
 * cache_lens[b] >= cache_capacity, cache_lens[b] >= max_position_embeddings),
 * WORKSPACE_TOO_SMALL, DEVICE. */
qwen3_status qwen3_layer_decode(qwen3_layer* layer, const void* x, void* y, int32_t batch,
                                const int32_t* cache_lens, void* k_cache, void* v_cache,
                                int32_t cache_capacity, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Decode after a left-padded prefill ("lesson 6", section 8: each generated
 * token is a real column; the padding stays unattended).  As qwen3_layer_decode,
 * plus two HOST arrays [batch] (both NULL = no padding): sequence b's padding run
 * occupies slots pad_starts[b] .. pad_starts[b] + pad_lens[b] - 1 of its cache.
 * The new token is written to slot cache_lens[b], sits at position
 * cache_lens[b] - pad_lens[b] (the real tokens before it) and attends every
 * cached key outside the run, and itself.
 * Errors: as qwen3_layer_decode, plus INVALID_ARGUMENT when exactly one of the
 * two arrays is NULL and OUT_OF_RANGE when a run is not inside
 * [0, cache_lens[b]). */
qwen3_status qwen3_layer_decode_padded(qwen3_layer* layer, const void* x, void* y, int32_t batch,
                                       const int32_t* cache_lens, const int32_t* pad_starts,
                                       const int32_t* pad_lens, void* k_cache, void* v_cache,
                                       int32_t cache_capacity, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Local (sliding-window) layers ("Transformer architectures: from BERT to
 * diffusion, lesson 6", section 7): token i attends token j iff
 * i - window < j <= i, itself included, plus the first `sinks` tokens of its
 * sequence (attention sinks; they stay visible to every later token).
 * window = 0 means a global layer (plain causal attention; sinks ignored).
 *
 * Prefill with that banded mask on a linear cache: as qwen3_layer_prefill_at
 * (start_positions may be NULL), keys and values of every token are cached at
 * their slots as usual, only the attention mask changes.  Each query block
 * visits only the key tiles of its window and the sink tiles, so the attention
 * work grows with seq_len * window instead of seq_len^2.
 * Errors: as qwen3_layer_prefill_at, plus INVALID_ARGUMENT for a negative
 * window or sinks. */
qwen3_status qwen3_layer_prefill_window(qwen3_layer* layer, const void* x, void* y, int32_t batch,
                                        int32_t seq_len, const int32_t* start_positions, int32_t window,
                                        int32_t sinks, void* k_cache, void* v_cache, int32_t cache_capacity,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* Decode of a local layer.  positions is a HOST array [batch]: the new token of
 * sequence b sits at position positions[b] (the number of tokens it has seen).
 *  - rolling = 0: a linear cache as in qwen3_layer_decode (positions[b] is the
 *    cache length, the token goes to slot positions[b]); it attends the cached
 *    keys of its window and the sinks.  Key splits wholly outside both are not
 *    read at all.
 *  - rolling = 1: a rolling buffer (section 7: at most window keys, each token
 *    written over the one that has just left the window; here with `sinks`
 *    fixed slots in front): cache_capacity must equal sinks + window; the token
 *    goes to slot p below sinks and to slot sinks + (p - sinks) mod window above,
 *    and attends every filled slot (min(p + 1, sinks + window) of them) with no
 *    mask: the buffer holds exactly its visible keys.  positions[b] may exceed
 *    cache_capacity.  Running a sequence token by token from an empty buffer
 *    reproduces qwen3_layer_prefill_window (the page's banded-vs-rolling check).
 * Errors: as qwen3_layer_decode (the free-slot rule applies to linear caches
 * only), plus INVALID_ARGUMENT for a negative window or sinks, or rolling with
 * window = 0 or cache_capacity != sinks + window. */
qwen3_status qwen3_layer_decode_window(qwen3_layer* layer, const void* x, void* y, int32_t batch,
                                       const int32_t* positions, int32_t window, int32_t sinks,
                                       int32_t rolling, void* k_cache, void* v_cache,
                                       int32_t cache_capacity, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Allocation-free decode, for callers that cannot allocate device memory or
 * call hipMalloc (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The same computation, kernels and errors as
 * qwen3_layer_decode, but the intermediates live in a static device array of
 * the library (32 MiB; each GPU the library runs on holds its own copy until
 * the process ends) instead of a caller workspace.  The call allocates nothing:
 * no hipMalloc / hipFree, no profiling events (qwen3_layer_set_profiling has no
 * effect on it).  Its first call on a device looks the array up on that device
 * (hipGetSymbolAddress), so it must run with `stream`'s device current.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (several streams or threads at once) race and must not be issued; calls in
 * order on one stream are fine.  Nothing in the array needs clearing between
 * calls (every value a call reads was written earlier in the same call).
 * Errors: as qwen3_layer_decode; WORKSPACE_TOO_SMALL when the decode of `batch`
 * sequences over `cache_capacity` slots needs more than the 32 MiB (the sizes
 * qwen3_layer_workspace_size reports for the same call); INVALID_ARGUMENT when
 * the stream belongs to another device than the current one. */
qwen3_status qwen3_layer_decode_noalloc(qwen3_layer* layer, const void* x, void* y, int32_t batch,
                                        const int32_t* cache_lens, void* k_cache, void* v_cache,
                                        int32_t cache_capacity, void* stream);

/* RMSNorm of `rows` rows of `width` elements ("17. A modern architecture:
 * Qwen3", section RMSNorm): y = weight * x / sqrt(mean(x^2) + eps), reduced in
 * fp32.  x, weight and y all hold `dtype`; used for the final norm after a
 * stack of layers (section The whole model).  width must be a multiple of 8.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, DEVICE. */
qwen3_status qwen3_rmsnorm(const void* x, const void* weight, void* y, int64_t rows, int32_t width,
                           float eps, qwen3_dtype dtype, void* stream);

/* As qwen3_rmsnorm, with the gain applied as (gain_offset + weight): 1 for the
 * zero-centred final norm of a model whose layers set norm_unit_offset, 0 is
 * qwen3_rmsnorm. */
qwen3_status qwen3_rmsnorm_gain_offset(const void* x, const void* weight, void* y, int64_t rows,
                                       int32_t width, float eps, float gain_offset, qwen3_dtype dtype,
                                       void* stream);

/* Matrix-core rate probe, a measurement aid and not a step of the layer: each
 * of `workgroups` workgroups (4 waves) issues `iterations` x 16 back-to-back
 * bf16 32x32x16 MFMAs (the GEMMs' instruction, 32 x 32 x 16 multiply-adds
 * each) on pseudo-random operands held in registers, so the launch's rate is
 * what the matrix cores sustain under the chip's power management with no
 * memory or LDS traffic: the ceiling beside the published dense bf16 peak that
 * the GEMMs' fraction can be read against.  Work per launch:
 * workgroups x 4 x iterations x 16 x 32768 flops.  out: device buffer of
 * workgroups x 256 floats (caller-owned), overwritten with one sum per lane.
 * Asynchronous on `stream`.  Errors: INVALID_ARGUMENT (NULL out, workgroups
 * or iterations < 1), DEVICE (launch failure). */
qwen3_status qwen3_probe_mfma_rate(float* out, int32_t workgroups, int32_t iterations, void* stream);

/* Per-kernel timing of prefill / decode calls made while profiling is on:
 * every launch is bracketed by two hipEvents on the call's stream. */
typedef struct {
    char name[48];
    int32_t launches;
    double total_ms;
} qwen3_stage_time;

qwen3_status qwen3_layer_set_profiling(qwen3_layer* layer, int32_t enabled);

/* Waits for the recorded events (host synchronisation), returns the per-kernel
 * totals accumulated since the last read, and clears them. */
qwen3_status qwen3_layer_read_profile(qwen3_layer* layer, qwen3_stage_time* out,
                                      int32_t max_entries, int32_t* n_entries);

const char* qwen3_status_string(qwen3_status status);
const char* qwen3_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* QWEN3_LAYER_H */
