// Causal grouped-query attention for prefill, head_dim 128, bf16 operands on gfx950 matrix
// cores with an fp32 online softmax.
//
// What it computes ("Transformer architectures: from BERT to diffusion, lesson 6", section 3;
// "17. A modern architecture: Qwen3", section Attention with grouped KV heads and Q/K
// normalization): for query head h and KV head floor(h / g), g = Hq / Hkv,
//   o_i = sum_{j : pos_j <= pos_i} softmax_j(q_i . k_j / sqrt(D)) v_j.
// The score matrix is never written out: keys and values stream through LDS in tiles of 64 and
// the softmax is accumulated online (running max and sum per query, rescaling the output).
//
// Layout choices for CDNA4:
//  * A workgroup (4 waves) serves up to 4 query heads of ONE KV head, so each K/V tile staged in
//    LDS is read by every head of its group (one read of a shared KV head serves g query heads).
//    Each wave owns 32 queries of one head.  When the grid would leave CUs idle (short sequences,
//    g = 2), the two waves of a head pair split every 64-key tile in halves of 32 keys instead of
//    taking separate queries; their partial (max, sum, O) are merged through LDS at the end.
//    Two workgroups share a CU (<= 256 registers per lane, 80 KB of LDS each).
//  * The grid is one-dimensional and ordered so that workgroup L, which the dispatcher places on
//    XCD L % 8, always serves KV heads of one XCD: a head's K/V (1-4 MB here) stays in that XCD's
//    L2 instead of being fetched by all eight.  The heaviest query tiles are dispatched first;
//    when the whole grid is resident at once, heavy and light tiles are paired per CU instead.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: in the 32x32
//    accumulator a lane holds 16 keys of ONE query (column = lane % 32), so the row max is a
//    per-lane reduction plus one exchange with lane ^ 32.
//  * Software pipeline: the scores of tile t+1 are issued to the matrix core before tile t is
//    exponentiated, so MFMA and VALU work overlap.  K is staged two tiles ahead and V one tile
//    ahead (two LDS slots each), which needs a single barrier per tile.
//  * The probabilities stay in registers and feed O^T += V^T P^T directly as the B operand.  V
//    stays row-major in LDS; its A-operand fragments come from ds_read_b64_tr_b16 transpose reads
//    whose per-lane row choice reproduces the accumulator's key order (4 consecutive keys from
//    each lane half, see v_rd below), so no register transpose is needed.
//  * LDS rows are padded (K 272 B, V 320 B) so fragment reads hit all 64 banks once and every
//    fragment address is a per-lane base plus an immediate.
//  * K and V tiles are fetched with buffer loads whose descriptor covers exactly the visible
//    keys: the hardware returns zeros past the end, so the last tile needs no clamping.
//  * The output is rescaled only when some lane's running max grows by more than 8 (log2
//    units): the reference max may lag the true max, which only bounds the probabilities by
//    2^8 and cancels in the final normalisation.  The row sum accumulates the bf16-rounded
//    probabilities the PV product actually uses (v_dot2), so the weights sum exactly to one.
//  * Tiles above the diagonal are never visited; per wave, 32-key blocks that lie entirely
//    above its queries skip their MFMAs.
//  * Left-padded batches ("lesson 6", section 8): keys in a sequence's padding slots are masked
//    for every query but their own token, on the tiles that overlap the padding run.
//  * Local layers (section 7): a query at position i sees keys i - W < j <= i and the first
//    `sinks` keys; a workgroup visits only the sink tiles and the tiles from its first query's
//    window start on, so the work grows with T * W instead of T^2.
//  * Padding and local masks are compiled into a separate instantiation (MASKED), used only when
//    a call has either; the plain causal kernel carries none of that code.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace q3 {

namespace {

constexpr int HD = 128;               // head_dim
constexpr int KT = 64;                // keys per tile
constexpr int KP = HD + 8;            // K row pitch in elements (272 B)
constexpr int VP = HD + 32;           // V row pitch in elements (320 B)
constexpr int K_ELEMS = KT * KP;
constexpr int V_ELEMS = KT * VP;
constexpr int NT = 256;               // threads per workgroup (4 waves)
constexpr int CH = (KT * HD / 8) / NT;  // 16-byte chunks of K (and of V) staged per thread

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int int4v __attribute__((ext_vector_type(4)));

// v of lane l and of lane l ^ 32, in (a, b): v_permlane32_swap exchanges the upper 32 lanes of its
// first operand with the lower 32 lanes of its second, so with v in both each lane holds both
// values afterwards, at VALU latency (a ds_bpermute would be an LDS round trip).  Written as
// assembly because the compiler folds the builtin's two results into one when both operands
// hold the same value; the s_nop covers the VALU-write-to-permlane-read hazard.
__device__ __forceinline__ void pair_xor32(float v, float& a, float& b) {
    a = v;
    b = v;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// Fixed-reference softmax.  When every key of the sequence was normalised by this call (no
// cached prefix), each score is bounded: q-hat and k-hat are gains times unit-RMS vectors of D
// features (rotation keeps norms), so |q-hat . k-hat| <= D max|g_q| max|g_k|.  If that bound, in
// log2 units, is at most 60, the probabilities 2^s need no running maximum: they neither overflow
// nor underflow in fp32 or bf16, and the softmax, being shift-invariant, is the same up to
// rounding.  The scale D^-1/2 log2(e) then goes into Q once, so each score costs one exp2, half a
// conversion and half a row-sum step.  Otherwise (a cached prefix, or large gains) the running
// maximum is kept.  Returns the wave-uniform decision.
__device__ __forceinline__ int fixed_reference(const AttnArgs& a, int pos0, int lane, float sl2) {
    int fixed = 0;
    if (pos0 == 0 && a.q_norm && a.k_norm) {
        const bf16* gq = static_cast<const bf16*>(a.q_norm);
        const bf16* gk = static_cast<const bf16*>(a.k_norm);
        float mq = fmaxf(fabsf((float)gq[lane] + a.goff), fabsf((float)gq[lane + 64] + a.goff));
        float mk = fmaxf(fabsf((float)gk[lane] + a.goff), fabsf((float)gk[lane + 64] + a.goff));
        mq = wave_max(mq);
        mk = wave_max(mk);
        // 1.05: room for the bf16 rounding of q-hat, k-hat and the scaled Q
        fixed = __builtin_amdgcn_readfirstlane((int)(mq * mk * (float)HD * sl2 * 1.05f <= 60.f));
    }
    return fixed;
}

template <int HPW, int KS, bool MASKED>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void flash_prefill_kernel(AttnArgs a, float sl2,
                                                                                                   bool pair_tiles) {
    constexpr int WPH = 4 / (HPW * KS);
    constexpr int QB = 32 * WPH;
    constexpr int NKB = 2 / KS;
    static_assert(HPW * KS * WPH == 4, "4 waves");
    __shared__ __attribute__((aligned(16))) bf16 sK[2 * K_ELEMS];
    __shared__ __attribute__((aligned(16))) bf16 sV[2 * V_ELEMS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // wave = (key half ph, query group wq, head hi); ph only varies when KS = 2
    const int hi = wave % HPW, wq = (wave / HPW) % WPH, ph = wave / (HPW * WPH);
    const int g = a.Hq / a.Hkv;
    const int subs = g / HPW;
    const int nqt = (a.T + QB - 1) / QB;
    int kvh, sub, b, qrank;
    {
        int r = blockIdx.x;
        if ((a.Hkv & 7) == 0) {
            // workgroup L runs on XCD L % 8: give each XCD whole KV heads so their K/V stay in its L2
            const int xcd = r & 7;
            r >>= 3;
            const int hpx = a.Hkv >> 3;
            const int m = r % hpx; r /= hpx;
            sub = r % subs; r /= subs;
            b = r % a.B; r /= a.B;
            qrank = r;
            kvh = xcd + 8 * m;
        } else {
            kvh = r % a.Hkv; r /= a.Hkv;
            sub = r % subs; r /= subs;
            b = r % a.B; r /= a.B;
            qrank = r;
        }
    }
    if (pair_tiles) {
        // every workgroup is resident at once: the second half of the dispatch order (which
        // fills each CU's second slot) runs the lightest query tiles first, so a CU pairs query
        // tile j with tile nqt-1-j and all CUs carry about the same number of key tiles
        const int half = (nqt + 1) >> 1;
        if (qrank >= half) qrank = nqt - 1 - (qrank - half);
    }
    const int h = kvh * g + sub * HPW + hi;
    const int q0 = (nqt - 1 - qrank) * QB;
    const int qw = q0 + wq * 32;
    const int pos0 = __builtin_amdgcn_readfirstlane(seq_pos(a.pos, b));
    int pad_lo = 0, pad_hi = 0;   // left-padding slots: attended by nobody but themselves
    if constexpr (MASKED) {
        seq_pad(a.pos, b, pad_lo, pad_hi);
        pad_lo = __builtin_amdgcn_readfirstlane(pad_lo);
        pad_hi = __builtin_amdgcn_readfirstlane(pad_hi);
    }
    const int kv_len = pos0 + min(q0 + QB, a.T);
    const int ntiles = (kv_len + KT - 1) / KT;
    const int my_pos = pos0 + qw + (lane & 31);
    const int wave_first = pos0 + qw;
    const int wave_last = pos0 + min(qw + 31, a.T - 1);
    // Key tiles visited: all of them for a global layer; for a local one the sink tiles and then
    // the tiles from the window start of the workgroup's first query on.
    const int win = MASKED ? a.local.window : 0, sinks = MASKED ? a.local.sinks : 0;
    int tw0 = 0, nsink_t = 0;
    if (win > 0) {
        tw0 = min(max(0, pos0 + q0 - win + 1) / KT, ntiles - 1);
        nsink_t = min((sinks + KT - 1) / KT, tw0);
    }
    const int nvis = nsink_t + (ntiles - tw0);
    auto tidx = [&](int u) { return u < nsink_t ? u : tw0 + (u - nsink_t); };

    // Q^T fragments (B operand): query qw + lane%32, d chunk 2s + lane/32.
    bf16x8 qf[8];
    {
        const bf16* qrow = static_cast<const bf16*>(a.qhat) +
                           (((int64_t)b * a.Hq + h) * a.T + min(qw + (lane & 31), a.T - 1)) * HD;
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + (2 * s + (lane >> 5)) * 8);
    }
    // fixed-reference softmax (see fixed_reference): no running maximum, Q pre-scaled; only in
    // the split-tile form (KS = 2), whose waves have the registers for a second loop body
    const int fixed = KS == 2 ? fixed_reference(a, pos0, lane, sl2) : 0;
    if (fixed) {
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[s][e] = (bf16)((float)qf[s][e] * sl2);
    }
    // Buffer descriptors over keys 0 .. kv_len-1 of this (sequence, KV head).
    const int64_t kv_base = ((int64_t)b * a.Hkv + kvh) * a.cap * HD;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.k_cache) + kv_base), (short)0, kv_len * HD * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.v_cache) + kv_base), (short)0, kv_len * HD * 2, 0x00020000);

    // Staging: thread moves 16-byte chunk st_ch of keys st_row + 16 j, j < CH.
    const int st_row = tid >> 4, st_ch = tid & 15;
    const int st_off = (st_row * HD + st_ch * 8) * 2;
    int4v rk[CH], rv[CH];
    auto load_k = [&](int t) {
#pragma unroll
        for (int j = 0; j < CH; ++j) rk[j] = __builtin_amdgcn_raw_buffer_load_b128(krs, st_off + (tidx(t) * KT + 16 * j) * HD * 2, 0, 0);
    };
    auto load_v = [&](int t) {
#pragma unroll
        for (int j = 0; j < CH; ++j) rv[j] = __builtin_amdgcn_raw_buffer_load_b128(vrs, st_off + (tidx(t) * KT + 16 * j) * HD * 2, 0, 0);
    };
    auto store_k = [&](int slot) {
        bf16* d = sK + slot * K_ELEMS + st_row * KP + st_ch * 8;
#pragma unroll
        for (int j = 0; j < CH; ++j) *reinterpret_cast<int4v*>(d + 16 * j * KP) = rk[j];
    };
    auto store_v = [&](int slot) {
        bf16* d = sV + slot * V_ELEMS + st_row * VP + st_ch * 8;
#pragma unroll
        for (int j = 0; j < CH; ++j) *reinterpret_cast<int4v*>(d + 16 * j * VP) = rv[j];
    };
    // K fragment (A of S^T = K Q^T): row kb*32 + lane%32, 16-byte chunk 2s + lane/32.
    const int k_rd = (lane & 31) * KP + (lane >> 5) * 8;
    // V^T fragment (A of O^T = V^T P^T) by transpose reads.  In the score accumulator, element j
    // of lane half q = lane/32 is key 8(j/4) + 4q + j%4 of its 16-key step.  Lane i' of 16-lane
    // group G reads row 4(G/2) + i'/4 (and +8), columns 16(G%2) + 4(i'%4): after the transpose
    // lane l holds rows 4q + 0..3 (and 8 + 4q + 0..3) of column l%32 - the same keys.
    const int G = lane >> 4, ip = lane & 15;
    const int v_rd = (4 * (G >> 1) + (ip >> 2)) * VP + 16 * (G & 1) + 4 * (ip & 3);

    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    float m_run = fixed ? 0.f : -1e30f, l_run = 0.f;   // with the fixed reference the maximum stays 0
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

    auto s_tile = [&](int t, f32x16 (&sacc)[NKB], bool (&live)[NKB]) {
        const bf16* sKb = sK + (t & 1) * K_ELEMS + k_rd;
#pragma unroll
        for (int i = 0; i < NKB; ++i) {
            const int kb = (KS == 1) ? i : ph;
            live[i] = (tidx(t) * KT + kb * 32) <= wave_last;
            if (live[i]) {
                const bf16x8 kf0 = *reinterpret_cast<const bf16x8*>(sKb + kb * 32 * KP);
                sacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0, qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
                for (int s = 1; s < 8; ++s) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sKb + kb * 32 * KP + s * 16);
                    sacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[i], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[i][r] = -INFINITY;
            }
        }
    };
    auto softmax_pv = [&](int t, f32x16 (&sacc)[NKB], const bool (&live)[NKB], auto fx) __attribute__((always_inline)) {
        constexpr bool FX = decltype(fx)::value;
        const int k0 = tidx(t) * KT;
        if (k0 + KT - 1 > wave_first ||
            (MASKED && ((k0 < pad_hi && k0 + KT > pad_lo) || (win > 0 && k0 <= wave_last - win)))) {
#pragma unroll
            for (int i = 0; i < NKB; ++i) {
                const int kb = (KS == 1) ? i : ph;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    // branch-free select (bitwise, not short-circuit operators)
                    const bool masked =
                        (key > my_pos) | (MASKED & (((key >= pad_lo) & (key < pad_hi) & (key != my_pos)) |
                                                    ((win > 0) & (my_pos - key >= win) & (key >= sinks))));
                    sacc[i][r] = masked ? -INFINITY : sacc[i][r];
                }
            }
        }
        if constexpr (!FX) {
            float mt = -INFINITY;
#pragma unroll
            for (int i = 0; i < NKB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[i][r]);
            {
                float m0v, m1v;
                pair_xor32(mt, m0v, m1v);
                mt = fmaxf(m0v, m1v) * sl2;
            }
            if (__any(mt > m_run + 8.f)) {
                const float m_new = fmaxf(m_run, mt);
                const float corr = fast_exp2(m_run - m_new);
                m_run = m_new;
                l_run *= corr;
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[db][r] *= corr;
            }
        }
        bf16x8 pf[NKB][2];
#pragma unroll
        for (int i = 0; i < NKB; ++i)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    pf[i][hf][j] = (bf16)fast_exp2(FX ? sacc[i][8 * hf + j] : fmaf(sacc[i][8 * hf + j], sl2, -m_run));
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    const bf16x2 pp = {pf[i][hf][j], pf[i][hf][j + 1]};
                    l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run, false);
                }
            }
        const bf16* sVb = sV + (t & 1) * V_ELEMS + v_rd;
#pragma unroll
        for (int i = 0; i < NKB; ++i) {
            if (!live[i]) continue;
            const int kb = (KS == 1) ? i : ph;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const bf16* p = sVb + (kb * 32 + hf * 16) * VP + db * 32;
                    const bf16x4 v0 = lds_read_tr(p);
                    const bf16x4 v1 = lds_read_tr(p + 8 * VP);
                    const bf16x8 vf = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[i][hf], o[db], 0, 0, 0);
                }
            }
        }
    };
    // one pipelined step: S of tile t+1 goes out before tile t's softmax and PV
    auto step = [&](int t, f32x16 (&cur)[NKB], const bool (&lcur)[NKB], f32x16 (&nxt)[NKB], bool (&lnxt)[NKB],
                    auto fx) __attribute__((always_inline)) {
        if (t + 2 < nvis) load_k(t + 2);
        if (t + 1 < nvis) load_v(t + 1);
        if (t + 1 < nvis) s_tile(t + 1, nxt, lnxt);
        softmax_pv(t, cur, lcur, fx);
        if (t + 2 < nvis) store_k(t & 1);
        if (t + 1 < nvis) store_v((t + 1) & 1);
        __syncthreads();
    };

    // One step over a tile with no mask and every key block live.  Between the rescale test and the
    // barrier it has no branch, so the scheduler can interleave, on this wave's own issue slots,
    // the score MFMAs of tile t+1 with the exponentials of tile t (one MFMA, then six VALU
    // instructions and one K fragment read, while the matrix core works through the MFMA), and the
    // PV MFMAs with their V fragment reads.  The global loads and LDS stores are unconditional (a
    // clamped tile index): past the last tile they refill a slot no later step reads.
    auto fast_step = [&](int t, f32x16 (&cur)[NKB], f32x16 (&nxt)[NKB], bool (&lnxt)[NKB], auto fx)
        __attribute__((always_inline)) {
        constexpr bool FX = decltype(fx)::value;
        load_k(min(t + 2, nvis - 1));
        load_v(min(t + 1, nvis - 1));
        if constexpr (!FX) {
            float mt = -INFINITY;
#pragma unroll
            for (int i = 0; i < NKB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) mt = fmaxf(mt, cur[i][r]);
            {
                float m0v, m1v;
                pair_xor32(mt, m0v, m1v);
                mt = fmaxf(m0v, m1v) * sl2;
            }
            if (__any(mt > m_run + 8.f)) {
                const float m_new = fmaxf(m_run, mt);
                const float corr = fast_exp2(m_run - m_new);
                m_run = m_new;
                l_run *= corr;
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[db][r] *= corr;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // scores of tile t+1
        const bf16* sKb = sK + ((t + 1) & 1) * K_ELEMS + k_rd;
#pragma unroll
        for (int i = 0; i < NKB; ++i) {
            const int kb = (KS == 1) ? i : ph;
            const bf16x8 kf0 = *reinterpret_cast<const bf16x8*>(sKb + kb * 32 * KP);
            nxt[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0, qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
            for (int s = 1; s < 8; ++s) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sKb + kb * 32 * KP + s * 16);
                nxt[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], nxt[i], 0, 0, 0);
            }
            lnxt[i] = true;
        }
        // probabilities of tile t
        bf16x8 pf[NKB][2];
#pragma unroll
        for (int i = 0; i < NKB; ++i)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    pf[i][hf][j] = (bf16)fast_exp2(FX ? cur[i][8 * hf + j] : fmaf(cur[i][8 * hf + j], sl2, -m_run));
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    const bf16x2 pp = {pf[i][hf][j], pf[i][hf][j + 1]};
                    l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run, false);
                }
            }
        // O^T += V^T P^T for tile t
        const bf16* sVb = sV + (t & 1) * V_ELEMS + v_rd;
#pragma unroll
        for (int i = 0; i < NKB; ++i) {
            const int kb = (KS == 1) ? i : ph;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const bf16* pv = sVb + (kb * 32 + hf * 16) * VP + db * 32;
                    const bf16x4 v0 = lds_read_tr(pv);
                    const bf16x4 v1 = lds_read_tr(pv + 8 * VP);
                    const bf16x8 vf = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[i][hf], o[db], 0, 0, 0);
                }
            }
        }
        // issue order: K reads ahead, then per score MFMA six VALU instructions of the softmax (four
        // with the fixed reference) and one more K read; then the PV MFMAs, two V reads ahead of each
        constexpr int NS = 8 * NKB;   // score MFMAs (= K fragment reads)
        constexpr int NV = FX ? 4 : 6;
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
            if (k + 4 < NS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (k + 2 < NS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        store_k(t & 1);
        store_v((t + 1) & 1);
        __syncthreads();
    };

    load_k(0);
    load_v(0);
    store_k(0);
    store_v(0);
    if (nvis > 1) {
        load_k(1);
        store_k(1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 sa[NKB], sb[NKB];
    bool la[NKB], lb[NKB];
    s_tile(0, sa, la);
    int t = 0;
    // the tile loop, instantiated with and without the running maximum
    auto run = [&](auto fx) __attribute__((always_inline)) {
        if constexpr (!MASKED) {
            // Tiles wholly at or below the first query of the workgroup need no mask and have every
            // key block live; all but the last (whose step would have no next tile to score) run the
            // branch-free step, in pairs so the two score buffers alternate statically.
            const int nfull = (pos0 + q0 + 1) / KT;
            const int nfast = min(nfull, nvis - 1) & ~1;
            for (; t < nfast; t += 2) {
                fast_step(t, sa, sb, lb, fx);
                fast_step(t + 1, sb, sa, la, fx);
            }
        }
        for (; t < nvis; t += 2) {
            step(t, sa, la, sb, lb, fx);
            if (t + 1 >= nvis) break;
            step(t + 1, sb, lb, sa, la, fx);
        }
    };
    if constexpr (KS == 2) {
        if (fixed)
            run(std::true_type{});
        else
            run(std::false_type{});
    } else {
        run(std::false_type{});
    }

    if constexpr (KS == 2) {
        // merge the two key halves: phase-1 waves hand (m, l, O) to phase-0 waves through LDS
        float* red = reinterpret_cast<float*>(sK);
        const int slot = hi + HPW * wq;
        float* mine = red + slot * (66 * 64) + lane;
        if (ph == 1) {
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) mine[(db * 16 + r) * 64] = o[db][r];
            mine[64 * 64] = m_run;
            mine[65 * 64] = l_run;
        }
        __syncthreads();
        if (ph == 1) return;
        const float m1 = mine[64 * 64], l1 = mine[65 * 64];
        const float m_new = fmaxf(m_run, m1);
        const float c0 = fast_exp2(m_run - m_new), c1 = fast_exp2(m1 - m_new);
        l_run = l_run * c0 + l1 * c1;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * c0 + mine[(db * 16 + r) * 64] * c1;
    }

    // normalise and store: lane holds d = db*32 + 8(r/4) + 4(lane/32) + r%4 of its query
    float l0v, l1v;
    pair_xor32(l_run, l0v, l1v);
    const float inv = 1.0f / (l0v + l1v);
    const int q = qw + (lane & 31);
    if (q < a.T) {
        bf16* orow = static_cast<bf16*>(a.out) + ((int64_t)b * a.T + q) * a.Hq * HD + (int64_t)h * HD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                bf16x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = (bf16)(o[db][4 * rq + e] * inv);
                *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * rq + 4 * (lane >> 5)) = v4;
            }
    }
}

// ------------------------------------------------------------------ ping-pong form (long causal prefill)
// Eight waves in two groups of four (one wave of each group per SIMD) share the K/V tiles of one
// KV head.  Group 1's queries follow group 0's.  The groups run one phase apart and alternate,
// with a barrier between phases: while one group's waves issue the matrix work of a tile (the PV
// product of the previous tile, then the scores of this one) the other group's waves, on the same
// SIMDs, run the softmax of their current tile on the vector ALU and stage the next K or V tile.
// So one wave's exponentials overlap the other's MFMAs by construction instead of by chance.
//   phase 2k:   group 0 matrix(k)                 group 1 softmax(k - 1), writes K(k + 1)
//   phase 2k+1: group 0 softmax(k), writes V(k)   group 1 matrix(k)
// K(t) is in LDS from phase 2t - 2 and last read in phase 2t + 1; V(t) from phase 2t + 1 to 2t + 3:
// two slots of each suffice.  Group 1 stages every K tile, group 0 every V tile, each through two
// sets of 16 registers, requested four phases before the LDS write (two phases left the vector
// phase waiting on L2 and HBM latency); the barriers wait for LDS operations only.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int HPW>
__global__ __launch_bounds__(512) void flash_prefill_pp_kernel(AttnArgs a, float sl2) {
    constexpr int QW = 4 / HPW;          // 32-query blocks per group
    constexpr int QG = 32 * QW;          // queries per group
    constexpr int QB = 2 * QG;           // queries per workgroup
    constexpr int NKB = 2;               // 32-key blocks per tile
    __shared__ __attribute__((aligned(16))) bf16 sK[2 * K_ELEMS];
    __shared__ __attribute__((aligned(16))) bf16 sV[2 * V_ELEMS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, wl = wave & 3;
    const int hi = wl % HPW, wq = wl / HPW;
    const int g = a.Hq / a.Hkv;
    const int subs = g / HPW;
    const int nqt = (a.T + QB - 1) / QB;
    int kvh, sub, b, qrank;
    {
        int r = blockIdx.x;
        if ((a.Hkv & 7) == 0) {
            // workgroup L runs on XCD L % 8: give each XCD whole KV heads so their K/V stay in its L2
            const int xcd = r & 7;
            r >>= 3;
            const int hpx = a.Hkv >> 3;
            const int m = r % hpx; r /= hpx;
            sub = r % subs; r /= subs;
            b = r % a.B; r /= a.B;
            qrank = r;
            kvh = xcd + 8 * m;
        } else {
            kvh = r % a.Hkv; r /= a.Hkv;
            sub = r % subs; r /= subs;
            b = r % a.B; r /= a.B;
            qrank = r;
        }
    }
    const int h = kvh * g + sub * HPW + hi;
    const int q0 = (nqt - 1 - qrank) * QB;                  // heaviest query tiles first
    const int qw = q0 + grp * QG + wq * 32;                 // this wave's first query
    const int pos0 = __builtin_amdgcn_readfirstlane(seq_pos(a.pos, b));
    const int kv_len = pos0 + min(q0 + QB, a.T);
    const int n = (kv_len + KT - 1) / KT;                   // key tiles of the workgroup
    const int my_pos = pos0 + qw + (lane & 31);
    const int wave_first = pos0 + qw;
    const int wave_last = pos0 + min(qw + 31, a.T - 1);
    const bool wave_active = qw < a.T;                      // a last, partial query tile may leave waves idle
    auto live = [&](int t) { return wave_active && t * KT <= wave_last; };

    bf16x8 qf[8];
    {
        const bf16* qrow = static_cast<const bf16*>(a.qhat) +
                           (((int64_t)b * a.Hq + h) * a.T + min(qw + (lane & 31), a.T - 1)) * HD;
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + (2 * s + (lane >> 5)) * 8);
    }
    // fixed-reference softmax (see fixed_reference): the vector phase shrinks to well under the
    // matrix phase
    const int fixed = fixed_reference(a, pos0, lane, sl2);
    if (fixed) {
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[s][e] = (bf16)((float)qf[s][e] * sl2);
    }
    const int64_t kv_base = ((int64_t)b * a.Hkv + kvh) * a.cap * HD;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.k_cache) + kv_base), (short)0, kv_len * HD * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.v_cache) + kv_base), (short)0, kv_len * HD * 2, 0x00020000);

    // staging by one group (256 threads): chunk st_ch of keys st_row + 16 j, j < CH
    const int tg = tid & 255;
    const int st_row = tg >> 4, st_ch = tg & 15;
    const int st_off = (st_row * HD + st_ch * 8) * 2;
    // two register sets: a tile is requested four phases before its LDS write
    int4v stg[2][CH];
    auto load_tile = [&](int4v (&r)[CH], __amdgpu_buffer_rsrc_t rs, int t) {
#pragma unroll
        for (int j = 0; j < CH; ++j) r[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, st_off + (t * KT + 16 * j) * HD * 2, 0, 0);
    };
    auto store_k = [&](const int4v (&r)[CH], int slot) {
        bf16* d = sK + slot * K_ELEMS + st_row * KP + st_ch * 8;
#pragma unroll
        for (int j = 0; j < CH; ++j) *reinterpret_cast<int4v*>(d + 16 * j * KP) = r[j];
    };
    auto store_v = [&](const int4v (&r)[CH], int slot) {
        bf16* d = sV + slot * V_ELEMS + st_row * VP + st_ch * 8;
#pragma unroll
        for (int j = 0; j < CH; ++j) *reinterpret_cast<int4v*>(d + 16 * j * VP) = r[j];
    };
    const int k_rd = (lane & 31) * KP + (lane >> 5) * 8;
    const int G = lane >> 4, ip = lane & 15;
    const int v_rd = (4 * (G >> 1) + (ip >> 2)) * VP + 16 * (G & 1) + 4 * (ip & 3);

    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    float m_run = -1e30f;
    float lsum[4] = {0.f, 0.f, 0.f, 0.f};   // row sum in four independent chains
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
    f32x16 sacc[NKB];
    bf16x8 pf[NKB][2];

    auto scores = [&](int t) {
        const bf16* sKb = sK + (t & 1) * K_ELEMS + k_rd;
#pragma unroll
        for (int i = 0; i < NKB; ++i) {
            const bf16x8 kf0 = *reinterpret_cast<const bf16x8*>(sKb + i * 32 * KP);
            sacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0, qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
            for (int s = 1; s < 8; ++s) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sKb + i * 32 * KP + s * 16);
                sacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[i], 0, 0, 0);
            }
        }
    };
    auto pv = [&](int t) {
        const bf16* sVb = sV + (t & 1) * V_ELEMS + v_rd;
#pragma unroll
        for (int i = 0; i < NKB; ++i)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const bf16* pv = sVb + (i * 32 + hf * 16) * VP + db * 32;
                    const bf16x4 v0 = lds_read_tr(pv);
                    const bf16x4 v1 = lds_read_tr(pv + 8 * VP);
                    const bf16x8 vf = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[i][hf], o[db], 0, 0, 0);
                }
    };
    // matrix phase of tile t: PV of tile t - 1, then the scores of tile t
    // Each half keeps its fragment reads ahead of the MFMAs that use them (eight V reads, i.e. four
    // PV MFMAs, and four K reads), so the matrix core does not wait out an LDS round trip per MFMA.
    auto matrix_phase = [&](int t) {
        if (t >= 1 && live(t - 1)) {
            pv(t - 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (k < 12) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
        }
        if (t < n && live(t)) {
            scores(t);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (k < 12) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
    };
    // softmax of tile t (probabilities into pf, row sum; with the running maximum, its lazy
    // rescale of o)
    auto softmax_phase = [&](int t) {
        if (t < 0 || t >= n || !live(t)) return;
        const int k0 = t * KT;
        if (k0 + KT - 1 > wave_first) {
#pragma unroll
            for (int i = 0; i < NKB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    sacc[i][r] = key > my_pos ? -INFINITY : sacc[i][r];
                }
        }
        if (fixed) {
#pragma unroll
            for (int i = 0; i < NKB; ++i)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int j = 0; j < 8; ++j) pf[i][hf][j] = (bf16)fast_exp2(sacc[i][8 * hf + j]);
        } else {
            float mt = -INFINITY;
#pragma unroll
            for (int i = 0; i < NKB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[i][r]);
            {
                float m0v, m1v;
                pair_xor32(mt, m0v, m1v);
                mt = fmaxf(m0v, m1v) * sl2;
            }
            if (__any(mt > m_run + 8.f)) {
                const float m_new = fmaxf(m_run, mt);
                const float corr = fast_exp2(m_run - m_new);
                m_run = m_new;
#pragma unroll
                for (int c = 0; c < 4; ++c) lsum[c] *= corr;
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[db][r] *= corr;
            }
#pragma unroll
            for (int i = 0; i < NKB; ++i)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        pf[i][hf][j] = (bf16)fast_exp2(fmaf(sacc[i][8 * hf + j], sl2, -m_run));
        }
#pragma unroll
        for (int i = 0; i < NKB; ++i)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    const bf16x2 pp = {pf[i][hf][j], pf[i][hf][j + 1]};
                    float& acc = lsum[(j >> 1) & 3];
                    acc = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, acc, false);
                }
    };
    // vector phase of tile t (register set t & 1): this group's staging and the softmax of tile t.
    // Group 0 writes V(t) and requests V(t + 2); group 1 writes K(t + 2) (slot t & 1) and requests
    // K(t + 4).  Every vector phase requests its tile, past the last one the last tile again
    // (loaded, never stored): with the same requests on every path the compiler sees that the
    // set being stored is the older one and waits for it alone (vmcnt(CH)), not also for the
    // other set requested only two phases before.
    // With two heads per wave the staging goes after the softmax, pinned there: the LDS stores then
    // meet the other group's fragment reads near their end instead of delaying this group's
    // exponentials (stack attention 258 -> 254.5 us); with four heads per wave, whose vector phase
    // is longer, the earlier request of the next tile matters more (8B attention 486 us before the
    // softmax, 499 after).
    auto staging = [&](int t, int4v (&r)[CH]) {
        if (grp == 0) {
            if (t >= 0 && t < n) store_v(r, t & 1);
            load_tile(r, vrs, min(t + 2, n - 1));
        } else {
            if (t + 2 < n) store_k(r, t & 1);
            load_tile(r, krs, min(t + 4, n - 1));
        }
    };
    auto vector_phase = [&](int t, int4v (&r)[CH]) {
        if constexpr (HPW == 2) {
            softmax_phase(t);
            __builtin_amdgcn_sched_barrier(0);
            staging(t, r);
        } else {
            staging(t, r);
            softmax_phase(t);
        }
    };

    // prologue: K(0) in LDS; group 0 holds V(0), V(1), group 1 K(1), K(2) in its registers (a
    // tile index past the last one loads the last tile).  In both groups set 1 is requested last,
    // as at the end of every loop step, so the compiler's wait before each set's LDS store is the
    // same exact count on every path into the loop.
    if (grp == 1) {
        load_tile(stg[0], krs, 0);
        store_k(stg[0], 0);
        load_tile(stg[0], krs, min(2, n - 1));
        load_tile(stg[1], krs, min(1, n - 1));
    } else {
        load_tile(stg[0], vrs, 0);
        load_tile(stg[1], vrs, min(1, n - 1));
    }
    lds_barrier();
    // Every wave runs matrix(k), vector(k) in turn; group 1 starts one phase later (its vector
    // phase of tile -1 stages K(1)) and group 0 ends with one more barrier, so both pass the same
    // barriers and phase j pairs group 0's work of step j / 2 with group 1's of step (j - 1) / 2.
    // Unrolled by two so each step's register set is fixed.
    if (grp == 1) {
        vector_phase(-1, stg[1]);
        lds_barrier();
    }
    // whole pairs in the loop (no conditional requests in its body), the odd last step after it
    int k = 0;
    // With four heads per wave the matrix phase runs at raised wave priority, so on each SIMD the
    // matrix wave's fragment reads and MFMAs issue ahead of the vector wave's instructions (8B
    // attention 500 -> 491 us on one box; with two heads per wave it was 1.5 % slower, so there
    // both groups keep the default priority)
    auto matrix_prio = [&](int t) {
        if constexpr (HPW == 4) __builtin_amdgcn_s_setprio(2);
        matrix_phase(t);
        if constexpr (HPW == 4) __builtin_amdgcn_s_setprio(0);
    };
    for (; k + 1 <= n; k += 2) {
        matrix_prio(k);
        lds_barrier();
        vector_phase(k, stg[0]);
        lds_barrier();
        matrix_prio(k + 1);
        lds_barrier();
        vector_phase(k + 1, stg[1]);
        lds_barrier();
    }
    if (k <= n) {
        matrix_phase(k);
        lds_barrier();
        vector_phase(k, stg[0]);
        lds_barrier();
    }
    if (grp == 0) lds_barrier();
    __builtin_amdgcn_s_waitcnt(0);   // the requests past the last tile

    // normalise and store: lane holds d = db*32 + 8(r/4) + 4(lane/32) + r%4 of its query
    float l0v, l1v;
    pair_xor32((lsum[0] + lsum[1]) + (lsum[2] + lsum[3]), l0v, l1v);
    const float inv = 1.0f / (l0v + l1v);
    const int q = qw + (lane & 31);
    if (wave_active && q < a.T) {
        bf16* orow = static_cast<bf16*>(a.out) + ((int64_t)b * a.T + q) * a.Hq * HD + (int64_t)h * HD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                bf16x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = (bf16)(o[db][4 * rq + e] * inv);
                *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * rq + 4 * (lane >> 5)) = v4;
            }
    }
}

template <bool MASKED>
hipError_t launch_hpw(const AttnArgs& a, int hpw, bool split, dim3 grid, float scale_log2, bool pair_tiles,
                      hipStream_t stream) {
    if (hpw == 4)
        flash_prefill_kernel<4, 1, MASKED><<<grid, NT, 0, stream>>>(a, scale_log2, pair_tiles);
    else if (hpw == 2 && split)
        flash_prefill_kernel<2, 2, MASKED><<<grid, NT, 0, stream>>>(a, scale_log2, pair_tiles);
    else if (hpw == 2)
        flash_prefill_kernel<2, 1, MASKED><<<grid, NT, 0, stream>>>(a, scale_log2, pair_tiles);
    else if (split)
        flash_prefill_kernel<1, 2, MASKED><<<grid, NT, 0, stream>>>(a, scale_log2, pair_tiles);
    else
        flash_prefill_kernel<1, 1, MASKED><<<grid, NT, 0, stream>>>(a, scale_log2, pair_tiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_prefill_bf16(const AttnArgs& a, hipStream_t stream) {
    if (a.D != HD || a.Hkv <= 0 || a.Hq % a.Hkv) return hipErrorInvalidValue;
    if (a.B <= 0 || a.T <= 0) return hipSuccess;
    const int g = a.Hq / a.Hkv;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const int hpw = (g % 4 == 0) ? 4 : (g % 2 == 0) ? 2 : 1;
    // Split tiles between waves (KS = 2) when whole-tile waves would give fewer than two
    // workgroups per CU.
    const int64_t wgs_whole = (int64_t)((a.T + 32 * (4 / hpw) - 1) / (32 * (4 / hpw))) * a.Hkv * (g / hpw) * a.B;
    const bool split = hpw < 4 && wgs_whole < 512;
    const int ks = split ? 2 : 1;
    const int qb = 32 * (4 / (hpw * ks));
    const int64_t wgs = (int64_t)((a.T + qb - 1) / qb) * a.Hkv * (g / hpw) * a.B;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs);
    const bool pair_tiles = wgs <= 512;   // two workgroups per CU on 256 CUs
    // the masking variant only when some sequence has left padding or the layer is local
    const bool masked = a.pos.dev_pad != nullptr || a.pos.n_pad_inline > 0 || a.local.window > 0;
    // Long causal prefill without masks: the ping-pong form, one 8-wave workgroup per CU, when it
    // still gives at least two workgroups per CU over the grid.
    if (!masked) {
        const int64_t qb_pp = 64 * (4 / hpw);
        const int64_t wgs_pp = (int64_t)((a.T + qb_pp - 1) / qb_pp) * a.Hkv * (g / hpw) * a.B;
        if (wgs_pp >= 512 && wgs_pp <= 0x7fffffff) {
            const dim3 gpp((unsigned)wgs_pp);
            if (hpw == 4) flash_prefill_pp_kernel<4><<<gpp, 512, 0, stream>>>(a, scale_log2);
            else if (hpw == 2) flash_prefill_pp_kernel<2><<<gpp, 512, 0, stream>>>(a, scale_log2);
            else flash_prefill_pp_kernel<1><<<gpp, 512, 0, stream>>>(a, scale_log2);
            return hipGetLastError();
        }
    }
    if (masked) return launch_hpw<true>(a, hpw, split, grid, scale_log2, pair_tiles, stream);
    return launch_hpw<false>(a, hpw, split, grid, scale_log2, pair_tiles, stream);
}

}  // namespace q3
