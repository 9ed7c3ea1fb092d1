"""GPU parity of the HIP path against the float64 oracle on small and ragged shapes.

Every call goes through the C ABI (Python binding).  Kernel-level tests feed the oracle
step the GPU's own input ("teacher forcing"), so each kernel is judged alone; layer tests
compare the whole layer with the oracle on the same seeded inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from gpu_support import (GpuLayer, assert_bf16_parity, assert_f32_parity, assert_rounded, check_decode_steps,
                         check_prefill_stages_full, log, oracle_layer_prefill_parallel, oracle_qk_from_proj,
                         small_bf16_cfg, to_dev, to_np)
from transformer_decoder_layer_rmsnorm_amd import _native as nat

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- RMSNorm entry point

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,width", [(1, 64), (7, 1024), (1000, 4096), (33, 5120), (5, 8)])
def test_rmsnorm_kernel(dtype, rows, width):
    log(f"rmsnorm {dtype} rows={rows} width={width}")
    cfg = si.LayerConfig(hidden_size=width, num_attention_heads=1, num_key_value_heads=1, head_dim=2,
                         intermediate_size=8, dtype=dtype)
    rng = np.random.default_rng(rows * 7 + width)
    x = si.round_to_bf16(rng.standard_normal((rows, width)).astype(np.float32) * 3) if dtype == "bf16" else \
        rng.standard_normal((rows, width)).astype(np.float32) * 3
    g = si.round_to_bf16((1 + 0.1 * rng.standard_normal(width)).astype(np.float32))
    xd, gd = to_dev(x, cfg), to_dev(g, cfg)
    y = torch.empty_like(xd)
    nat.rmsnorm(xd, gd, y, 1e-6)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(x, g, 1e-6)
    if dtype == "bf16":
        assert_rounded(to_np(y), ref, "rmsnorm bf16", abs_frac=1e-6)
    else:
        np.testing.assert_allclose(to_np(y), ref, rtol=2e-6, atol=1e-6)


# ---------------------------------------------------------------- fp32 layer (tiny config)

def test_tiny_f32_layer_matches_oracle():
    wl = si.WORKLOADS["tiny-f32-layer"]
    cfg = wl.cfg
    log(f"tiny fp32 layer B{wl.batch} T{wl.seq_len}")
    gl = GpuLayer.seeded(cfg, seed=wl.seed)
    x = si.layer_input(cfg, wl.batch, wl.seq_len, seed=wl.seed)
    y, kc, vc, ws = gl.prefill(to_dev(x, cfg))
    ref = oracle.layer_prefill(x, gl.w_np, cfg)
    assert_f32_parity(to_np(y), ref["y"], "y")
    inter = gl.intermediates(ws, wl.batch, wl.seq_len)
    for name in ["h", "qhat", "attn", "x1", "h2", "act"]:
        assert_f32_parity(inter[name], ref[name], name)
    assert_f32_parity(to_np(kc)[:, :, : wl.seq_len], ref["khat"], "k cache")
    assert_f32_parity(to_np(vc)[:, :, : wl.seq_len], ref["v"], "v cache")


@pytest.mark.parametrize("b,t,hq,hkv,d", [(2, 37, 4, 4, 64), (3, 5, 8, 2, 16), (1, 130, 6, 3, 128)])
def test_f32_layer_shapes(b, t, hq, hkv, d):
    cfg = si.LayerConfig(hidden_size=96, num_attention_heads=hq, num_key_value_heads=hkv, head_dim=d,
                         intermediate_size=136, dtype="f32")
    log(f"fp32 layer B{b} T{t} Hq{hq} Hkv{hkv} D{d}")
    gl = GpuLayer.seeded(cfg, seed=3)
    x = si.layer_input(cfg, b, t, seed=3)
    y, *_ = gl.prefill(to_dev(x, cfg), cap=t + 3)
    assert_f32_parity(to_np(y), oracle.layer_prefill(x, gl.w_np, cfg)["y"], "y")


def test_f32_decode_continues_prefill():
    cfg = si.TINY_F32
    gl = GpuLayer.seeded(cfg, seed=5)
    b, t = 3, 12
    x = si.layer_input(cfg, b, t, seed=5)
    full = oracle.layer_prefill(x, gl.w_np, cfg)
    lens = [11, 4, 0]
    cap = 16
    kc, vc = gl.alloc_cache(b, cap)
    for i, n in enumerate(lens):
        if n:
            gl.prefill(to_dev(x[i:i + 1, :n], cfg), caches=(kc[i:i + 1], vc[i:i + 1]), cap=cap)
    xin = np.stack([x[i, n] for i, n in enumerate(lens)])[:, None]
    y, _ = gl.decode(to_dev(xin, cfg), lens, kc, vc)
    for i, n in enumerate(lens):
        assert_f32_parity(to_np(y)[i, 0], full["y"][i, n], f"decode row {i} at position {n}")


# ---------------------------------------------------------------- bf16 kernels, teacher-forced

@pytest.mark.parametrize("hq,hkv,b,t", [(4, 2, 2, 77), (4, 4, 1, 130), (8, 2, 1, 200), (16, 2, 1, 64), (4, 1, 2, 33)])
def test_bf16_kernels_teacher_forced(hq, hkv, b, t):
    cfg = small_bf16_cfg(hq=hq, hkv=hkv)
    log(f"bf16 kernels Hq{hq} Hkv{hkv} B{b} T{t}")
    gl = GpuLayer.seeded(cfg, seed=hq * 10 + hkv)
    w = gl.w_np
    x = si.layer_input(cfg, b, t, seed=hq + t)
    cap = t + 5
    y, kc, vc, ws = gl.prefill(to_dev(x, cfg), cap=cap)
    it = gl.intermediates(ws, b, t)
    eps = cfg.rms_norm_eps
    kcn, vcn = to_np(kc), to_np(vc)
    for s in range(b):
        assert_rounded(it["h"][s], oracle.rmsnorm(x[s], w["input_layernorm"], eps), "rmsnorm_input")
        wqkv = np.concatenate([w["q_proj"], w["k_proj"], w["v_proj"]]).astype(np.float64)
        assert_rounded(it["qkv"][s], it["h"][s] @ wqkv.T, "gemm_qkv")
        qhat, khat, v = oracle_qk_from_proj(it["qkv"][s], w, cfg, np.arange(t))
        assert_rounded(it["qhat"][s], qhat, "qknorm_rope q")
        assert_rounded(kcn[s, :, :t], khat, "qknorm_rope k -> cache")
        assert np.array_equal(vcn[s, :, :t], v), "v copied to the cache unchanged"
        attn = oracle.gqa_causal_attention(it["qhat"][s], kcn[s, :, :t], vcn[s, :, :t], np.arange(t), np.arange(t))
        attn = attn.transpose(1, 0, 2).reshape(t, hq * 128)
        assert_bf16_parity(it["attn"][s], attn, "attention (bf16 probabilities)")
        x1 = x[s] + it["attn"][s] @ w["o_proj"].T.astype(np.float64)
        np.testing.assert_allclose(it["x1"][s], x1, rtol=1e-5, atol=2e-5)
        assert_rounded(it["h2"][s], oracle.rmsnorm(it["x1"][s], w["post_attention_layernorm"], eps), "rmsnorm_post")
        act = oracle.silu(it["h2"][s] @ w["gate_proj"].T.astype(np.float64)) * \
            (it["h2"][s] @ w["up_proj"].T.astype(np.float64))
        assert_rounded(it["act"][s], act, "gemm_gate_up_swiglu")
        yref = it["x1"][s] + it["act"][s] @ w["down_proj"].T.astype(np.float64)
        assert_rounded(to_np(y)[s], yref, "gemm_down_residual")


@pytest.mark.parametrize("hq,hkv,b,t", [(4, 2, 2, 77), (8, 8, 1, 96), (8, 1, 1, 150)])
def test_bf16_layer_matches_oracle(hq, hkv, b, t):
    cfg = small_bf16_cfg(hq=hq, hkv=hkv)
    log(f"bf16 layer Hq{hq} Hkv{hkv} B{b} T{t}")
    gl = GpuLayer.seeded(cfg, seed=7)
    x = si.layer_input(cfg, b, t, seed=7)
    y, *_ = gl.prefill(to_dev(x, cfg))
    assert_bf16_parity(to_np(y), oracle.layer_prefill(x, gl.w_np, cfg)["y"], "y")


@pytest.mark.parametrize("t", [1100, 700, 90])
def test_bf16_hidden_5120_layer(t):
    """hidden 5120, a width of the family above 4096 (16 / 8 heads, intermediate 1024).
    T = 1100: the fused QKV epilogue on 128 x 128 tiles, fed by the input RMSNorm that also
    writes the RoPE table, in its form for rows over 4096 wide.  T = 700: o_proj and down on the
    deep-ring 64 x 128 tiles with the residual added in their epilogues, the last row tile
    ragged.  T = 90: too few output tiles even for those: o_proj's K range is split and the
    post-attention RMSNorm sums its slabs, in its form for rows over 4096 wide; down split-K with
    the residual-sum pass.  Then one decode step on the prefilled cache (skinny GEMMs with
    K = 5120)."""
    cfg = small_bf16_cfg(hq=16, hkv=8, hidden=5120, inter=1024)
    log(f"bf16 layer hidden 5120, B1 T{t}")
    gl = GpuLayer.seeded(cfg, seed=t)
    x = si.layer_input(cfg, 1, t + 1, seed=t)
    cap = t + 1
    kc, vc = gl.alloc_cache(1, cap)
    y, kc, vc, ws = gl.prefill(to_dev(x[:, :t], cfg), cap=cap, caches=(kc, vc))
    ref = oracle.layer_prefill(x[:, :t], gl.w_np, cfg)
    it = gl.intermediates(ws, 1, t)
    eps = cfg.rms_norm_eps
    assert_rounded(it["h"][0], oracle.rmsnorm(x[0, :t], gl.w_np["input_layernorm"], eps), "rmsnorm_input (5120 wide)")
    assert_rounded(it["h2"][0], oracle.rmsnorm(it["x1"][0], gl.w_np["post_attention_layernorm"], eps),
                   "rmsnorm_post (5120 wide)")
    x1 = x[0, :t] + it["attn"][0] @ gl.w_np["o_proj"].T.astype(np.float64)
    np.testing.assert_allclose(it["x1"][0], x1, rtol=1e-5, atol=2e-5)
    assert_bf16_parity(to_np(y), ref["y"], "y")
    assert_bf16_parity(to_np(kc)[:, :, :t], ref["khat"], "k cache")
    yd, _ = gl.decode(to_dev(x[:, t:], cfg), [t], kc, vc)
    refd = oracle.layer_prefill_rows(x, gl.w_np, cfg, [(0, t)])
    assert_bf16_parity(to_np(yd)[0, 0], refd[0], "decode row at position T")


@pytest.mark.parametrize("b,t", [(1, 1000), (2, 750), (1, 2048)])
def test_bf16_thin_projections_deep_ring(b, t):
    """o_proj and down with too few 128 x 128 output tiles to fill the CUs but at least 128 tiles
    of 64 x 128 (hidden 1024 at 1000 to 2048 tokens): the deep-ring kernel, K not split, with the
    residual added in its epilogue (x1 = x + attn Wo^T in fp32, y = x1 + act Wd^T rounded once).
    The last row tile is ragged at 1000 and 1500 rows; every element is checked teacher-forced."""
    cfg = small_bf16_cfg(hq=8, hkv=4, hidden=1024, inter=3072)
    log(f"bf16 thin projections B{b} T{t}")
    gl = GpuLayer.seeded(cfg, seed=t + b)
    w = gl.w_np
    x = si.layer_input(cfg, b, t, seed=t + 2 * b)
    y, kc, vc, ws = gl.prefill(to_dev(x, cfg))
    it = gl.intermediates(ws, b, t)
    yn = to_np(y)
    for s in range(b):
        x1 = x[s] + it["attn"][s] @ w["o_proj"].T.astype(np.float64)
        np.testing.assert_allclose(it["x1"][s], x1, rtol=1e-5, atol=2e-5)
        yref = it["x1"][s] + it["act"][s] @ w["down_proj"].T.astype(np.float64)
        assert_rounded(yn[s], yref, "gemm_down_residual (deep ring)")


@pytest.mark.parametrize("hq,hkv,b,t", [(16, 4, 8, 1000), (16, 8, 8, 1000), (8, 8, 16, 960), (32, 8, 2, 2100)])
def test_bf16_attention_two_group_workgroups(hq, hkv, b, t):
    """Causal prefills long enough for the attention form whose 8-wave workgroups run two groups
    of waves in alternation (at least 512 workgroups): 4, 2 and 1 query heads per KV head,
    lengths that end mid-tile, and (T = 960 with one head per KV head) a last query tile whose
    final waves hold no query.  Every stage teacher-forced, then the whole layer."""
    cfg = small_bf16_cfg(hq=hq, hkv=hkv, hidden=256, inter=256)
    log(f"bf16 layer Hq{hq} Hkv{hkv} B{b} T{t} (two-group attention)")
    gl = GpuLayer.seeded(cfg, seed=hq + t)
    x = si.layer_input(cfg, b, t, seed=hq + t)
    y, kc, vc, ws = gl.prefill(to_dev(x, cfg))
    check_prefill_stages_full(gl, x, y, kc, vc, ws, f"Hq{hq} Hkv{hkv}")
    ref = oracle_layer_prefill_parallel(x, gl.w_np, cfg)
    assert_bf16_parity(to_np(y), ref["y"], "y (whole oracle layer)")


def test_bf16_attention_two_group_onto_cached_prefixes():
    """The two-group attention with cached prefixes (random keys that no k_norm of this call
    produced, so the running maximum is kept), ragged starts, one sequence with no prefix."""
    cfg = small_bf16_cfg(hq=16, hkv=4, hidden=256, inter=256)
    starts = [0, 300, 64, 511, 1, 700, 128, 33]
    b, t = len(starts), 1000
    cap = max(starts) + t
    log(f"bf16 prefill_at two-group attention B{b} T{t} starts {starts}")
    gl = GpuLayer.seeded(cfg, seed=44)
    kc, vc = _random_cache(cfg, starts, cap, seed=44)
    kd, vd = to_dev(kc, cfg), to_dev(vc, cfg)
    x = si.layer_input(cfg, b, t, seed=44)
    y, kd, vd, _ = gl.prefill(to_dev(x, cfg), cap=cap, caches=(kd, vd), starts=starts)
    ref, knew, _ = oracle.layer_prefill_cached(x, gl.w_np, cfg, kc, vc, starts)
    assert_bf16_parity(to_np(y), ref, "prefill_at y (two-group attention)")


def test_bf16_attention_two_group_large_gains():
    """q_norm / k_norm gains large enough that the score bound exceeds 2^60: the two-group
    attention keeps the running maximum on a plain prefill."""
    cfg = small_bf16_cfg(hq=16, hkv=4, hidden=256, inter=256)
    w = si.layer_weights(cfg, seed=45)
    w["q_norm"] = si.round_to_bf16(w["q_norm"] * 6.0)
    w["k_norm"] = si.round_to_bf16(w["k_norm"] * 6.0)
    gl = GpuLayer(cfg, w)
    b, t = 8, 1000
    log(f"bf16 two-group attention with 6x q/k gains, B{b} T{t}")
    x = si.layer_input(cfg, b, t, seed=45)
    y, kc, vc, ws = gl.prefill(to_dev(x, cfg))
    check_prefill_stages_full(gl, x, y, kc, vc, ws, "6x gains")


@pytest.mark.parametrize("shape", ["small", "8b"])
def test_bf16_single_token_attends_only_itself(shape):
    """The degenerate sequence of one token: a prefill of T = 1 and a decode step on empty caches
    (length 0).  The softmax over a single key is exactly 1, so the attention output must be that
    token's value row, bit for bit after the bf16 rounding (the normalisation divides p v by p);
    the layer outputs are compared with the oracle's prefill of the same token."""
    cfg = small_bf16_cfg(hq=8, hkv=2) if shape == "small" else si.WORKLOADS["qwen3-8b-layer-prefill"].cfg
    b = 3
    log(f"bf16 single token, {shape}, B{b}")
    gl = GpuLayer.seeded(cfg, seed=11)
    x = si.layer_input(cfg, b, 1, seed=12)
    ref = oracle.layer_prefill(x, gl.w_np, cfg)["y"]
    hq, hkv, d = cfg.num_attention_heads, cfg.num_key_value_heads, cfg.head_dim
    g = hq // hkv
    # prefill of T = 1
    y, kc, vc, ws = gl.prefill(to_dev(x, cfg), cap=4)
    it = gl.intermediates(ws, b, 1, 4)
    v0 = to_np(vc)[:, :, 0, :]                                   # [B, Hkv, D]
    want = np.repeat(v0, g, axis=1).reshape(b, 1, hq * d)        # head h reads KV head h // g
    assert np.array_equal(it["attn"], want), "prefill T=1: attention output is the value row"
    assert_bf16_parity(to_np(y), ref, "prefill T=1, y")
    # decode on empty caches: the token is written at slot 0 and attends only itself
    kc2, vc2 = gl.alloc_cache(b, 4)
    yd, wsd = gl.decode(to_dev(x, cfg), [0] * b, kc2, vc2)
    itd = gl.intermediates(wsd, b, 1, 4)
    assert np.array_equal(to_np(vc2)[:, :, 0, :], v0), "decode writes the same value row"
    assert np.array_equal(itd["attn"], want), "decode on empty caches: attention output is the value row"
    assert_bf16_parity(to_np(yd), ref, "decode on empty caches, y")


def test_bf16_causality_bit_exact():
    cfg = small_bf16_cfg()
    gl = GpuLayer.seeded(cfg, seed=9)
    t = 150
    x = si.layer_input(cfg, 1, t, seed=9)
    y0, *_ = gl.prefill(to_dev(x, cfg))
    y0 = y0.clone()
    for i in [0, 63, 64, 100, 148]:
        x2 = x.copy()
        x2[0, i + 1:] = si.round_to_bf16(np.random.default_rng(i).standard_normal(x2[0, i + 1:].shape)
                                         .astype(np.float32))
        y2, *_ = gl.prefill(to_dev(x2, cfg))
        assert torch.equal(y0[0, : i + 1], y2[0, : i + 1]), f"rows <= {i} changed"
        assert not torch.equal(y0[0, i + 1:], y2[0, i + 1:])
    log("  causality: rows up to i are bit-identical under changes after i")


def test_bf16_output_may_alias_input():
    cfg = small_bf16_cfg()
    gl = GpuLayer.seeded(cfg, seed=11)
    x = si.layer_input(cfg, 2, 40, seed=11)
    y, *_ = gl.prefill(to_dev(x, cfg))
    xd = to_dev(x, cfg)
    gl.prefill(xd, y_dev=xd)
    assert torch.equal(xd, y)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (8, 1), (8, 8)])
def test_bf16_decode_matches_oracle_ragged(hq, hkv):
    cfg = small_bf16_cfg(hq=hq, hkv=hkv)
    gl = GpuLayer.seeded(cfg, seed=13)
    lens = [0, 1, 511, 512, 513, 1500, 37]
    b = len(lens)
    cap = 1600
    log(f"bf16 decode Hq{hq} Hkv{hkv} lens {lens}")
    kc = np.zeros((b, hkv, cap, 128), np.float32)
    vc = np.zeros((b, hkv, cap, 128), np.float32)
    for i, n in enumerate(lens):
        for h in range(hkv):
            kc[i, h, :n] = si.cache_block(cfg, "k", i, h, n, seed=13)
            vc[i, h, :n] = si.cache_block(cfg, "v", i, h, n, seed=13)
    kd, vd = to_dev(kc, cfg), to_dev(vc, cfg)
    x = si.layer_input(cfg, b, 1, seed=13)
    y, ws = gl.decode(to_dev(x, cfg), lens, kd, vd)
    ref, _, _ = oracle.layer_decode(x, gl.w_np, cfg, kc, vc, lens)
    assert_bf16_parity(to_np(y), ref, "decode y")
    check_decode_steps(gl, ws, lens, kd, vd)


def test_bf16_decode_long_caches_merge_in_chunks():
    """Decode over caches longer than 64 splits of 1024 keys: the merge of the splits requests the
    partial outputs of 64 splits per chunk, so 70,000 and 131,072 cached keys (69 and 129 splits:
    two and three chunks) take its chunk loop; a third sequence with 32,768 (33 splits, one
    chunk) shares the call.  Every output row against the oracle decode.  (The layer is declared
    with a 256K-position context; the default 40,960 rejects these positions before any launch.)"""
    cfg = small_bf16_cfg(hq=4, hkv=2, max_position_embeddings=262144)
    gl = GpuLayer.seeded(cfg, seed=31)
    lens = [70000, 131072, 32768]
    b, hkv, d = len(lens), cfg.num_key_value_heads, cfg.head_dim
    cap = max(lens) + 1
    log(f"bf16 decode over long caches, lens {lens}")
    kd = torch.zeros((b, hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vd = torch.zeros_like(kd)
    kcs, vcs = [], []
    for i, n in enumerate(lens):
        kb = np.stack([si.cache_block(cfg, "k", i, h, n, seed=31) for h in range(hkv)])
        vb = np.stack([si.cache_block(cfg, "v", i, h, n, seed=31) for h in range(hkv)])
        kd[i, :, :n] = to_dev(kb, cfg)
        vd[i, :, :n] = to_dev(vb, cfg)
        kcs.append(kb)
        vcs.append(vb)
    x = si.layer_input(cfg, b, 1, seed=31)
    y, _ = gl.decode(to_dev(x, cfg), lens, kd, vd)
    ref, _, _ = oracle.layer_decode(x, gl.w_np, cfg, kcs, vcs, lens)
    assert_bf16_parity(to_np(y), ref, "decode y over 69, 129 and 33 splits")


@pytest.mark.parametrize("b", [1, 5, 16])
def test_bf16_decode_skinny_kernels(b):
    """Decode at widths where the skinny projections take their whole-line LDS-staged form (o and
    gate/up with K = 2048: one stage in flight per wave; down with K = 4096: two) and the QKV
    projection its split-K form whose slabs the QK-norm kernel adds (8 slices of 256): hidden 2048,
    intermediate 4096, 16 / 8 heads, with 1, 5 and 16 sequences (token rows past the batch in the
    16-row MFMA tiles read as zeros)."""
    cfg = small_bf16_cfg(hq=16, hkv=8, hidden=2048, inter=4096)
    gl = GpuLayer.seeded(cfg, seed=29)
    rng = np.random.default_rng(29 + b)
    lens = [int(v) for v in rng.integers(0, 700, size=b)]
    cap = 720
    log(f"bf16 decode hidden 2048, B{b}, lens {lens}")
    kc = np.zeros((b, 8, cap, 128), np.float32)
    vc = np.zeros((b, 8, cap, 128), np.float32)
    for i, n in enumerate(lens):
        for h in range(8):
            kc[i, h, :n] = si.cache_block(cfg, "k", i, h, n, seed=29)
            vc[i, h, :n] = si.cache_block(cfg, "v", i, h, n, seed=29)
    kd, vd = to_dev(kc, cfg), to_dev(vc, cfg)
    x = si.layer_input(cfg, b, 1, seed=29)
    y, ws = gl.decode(to_dev(x, cfg), lens, kd, vd)
    ref, _, _ = oracle.layer_decode(x, gl.w_np, cfg, kc, vc, lens)
    assert_bf16_parity(to_np(y), ref, "decode y")
    check_decode_steps(gl, ws, lens, kd, vd)


def test_bf16_decode_continues_prefill():
    cfg = small_bf16_cfg()
    gl = GpuLayer.seeded(cfg, seed=17)
    t = 300
    x = si.layer_input(cfg, 1, t, seed=17)
    yfull, *_ = gl.prefill(to_dev(x, cfg))
    cap = t + 8
    kc, vc = gl.alloc_cache(1, cap)
    gl.prefill(to_dev(x[:, : t - 1], cfg), caches=(kc, vc), cap=cap)
    y, _ = gl.decode(to_dev(x[:, t - 1: t], cfg), [t - 1], kc, vc)
    ref = oracle.layer_prefill_rows(x, gl.w_np, cfg, [(0, t - 1)])
    assert_bf16_parity(to_np(y)[0, 0], ref[0], "decode row vs oracle")
    assert_bf16_parity(to_np(y)[0, 0], to_np(yfull)[0, t - 1], "decode row vs prefill row")


def _random_cache(cfg, starts, cap, seed):
    b, hkv = len(starts), cfg.num_key_value_heads
    kc = np.zeros((b, hkv, cap, cfg.head_dim), np.float32)
    vc = np.zeros((b, hkv, cap, cfg.head_dim), np.float32)
    for i, n in enumerate(starts):
        for h in range(hkv):
            kc[i, h, :n] = si.cache_block(cfg, "k", i, h, n, seed=seed)
            vc[i, h, :n] = si.cache_block(cfg, "v", i, h, n, seed=seed)
    return kc, vc


@pytest.mark.parametrize("hq,hkv,t", [(4, 2, 77), (8, 1, 33), (8, 8, 130)])
def test_bf16_prefill_at_matches_oracle_ragged(hq, hkv, t):
    # prefill onto caches already holding 0, 1, 63, 64, 65, 200 and 511 keys
    cfg = small_bf16_cfg(hq=hq, hkv=hkv)
    gl = GpuLayer.seeded(cfg, seed=21)
    starts = [0, 1, 63, 64, 65, 200, 511]
    b = len(starts)
    cap = max(starts) + t + 5
    log(f"bf16 prefill_at Hq{hq} Hkv{hkv} T{t} starts {starts}")
    kc, vc = _random_cache(cfg, starts, cap, seed=21)
    kd, vd = to_dev(kc, cfg), to_dev(vc, cfg)
    x = si.layer_input(cfg, b, t, seed=21)
    y, kd, vd, _ = gl.prefill(to_dev(x, cfg), cap=cap, caches=(kd, vd), starts=starts)
    ref, knew, vnew = oracle.layer_prefill_cached(x, gl.w_np, cfg, kc, vc, starts)
    assert_bf16_parity(to_np(y), ref, "prefill_at y")
    kg, vg = to_np(kd), to_np(vd)
    for i, n in enumerate(starts):
        # slots before the start and after the new tokens are untouched
        assert np.array_equal(kg[i, :, :n], kc[i, :, :n]) and np.array_equal(vg[i, :, :n], vc[i, :, :n])
        assert not kg[i, :, n + t:].any() and not vg[i, :, n + t:].any()
        assert_bf16_parity(kg[i, :, n:n + t], knew[i], f"new keys of sequence {i}")
        assert_bf16_parity(vg[i, :, n:n + t], vnew[i], f"new values of sequence {i}")


def test_bf16_chunked_prefill_equals_one_shot():
    cfg = small_bf16_cfg()
    gl = GpuLayer.seeded(cfg, seed=22)
    t1, t2 = 150, 97
    x = si.layer_input(cfg, 2, t1 + t2, seed=22)
    log(f"bf16 chunked prefill {t1} + {t2}")
    yfull, *_ = gl.prefill(to_dev(x, cfg))
    cap = t1 + t2
    kc, vc = gl.alloc_cache(2, cap)
    y1, *_ = gl.prefill(to_dev(x[:, :t1], cfg), caches=(kc, vc), cap=cap)
    y2, *_ = gl.prefill(to_dev(x[:, t1:], cfg), caches=(kc, vc), cap=cap, starts=[t1, t1])
    got = np.concatenate([to_np(y1), to_np(y2)], axis=1)
    assert_bf16_parity(got, to_np(yfull), "chunked vs one-shot")
    rows = [(0, t1), (1, t1 + t2 - 1), (0, t1 + 40), (1, 3)]
    ref = oracle.layer_prefill_rows(x, gl.w_np, cfg, rows)
    for n, (b, r) in enumerate(rows):
        assert_bf16_parity(got[b, r], ref[n], f"chunked row {(b, r)} vs oracle")


def test_bf16_prefill_at_many_sequences_positions_in_workspace():
    # more than 64 sequences: the start positions go through the workspace
    cfg = small_bf16_cfg()
    gl = GpuLayer.seeded(cfg, seed=23)
    starts = [(5 * i) % 37 for i in range(66)]
    t = 3
    cap = max(starts) + t
    log(f"bf16 prefill_at {len(starts)} sequences")
    kc, vc = _random_cache(cfg, starts, cap, seed=23)
    kd, vd = to_dev(kc, cfg), to_dev(vc, cfg)
    x = si.layer_input(cfg, len(starts), t, seed=23)
    y, *_ = gl.prefill(to_dev(x, cfg), cap=cap, caches=(kd, vd), starts=starts)
    ref, _, _ = oracle.layer_prefill_cached(x, gl.w_np, cfg, kc, vc, starts)
    assert_bf16_parity(to_np(y), ref, "prefill_at y, 66 sequences")


def test_f32_prefill_at_matches_oracle():
    cfg = si.TINY_F32
    gl = GpuLayer.seeded(cfg, seed=24)
    starts = [0, 5, 16]
    t = 7
    cap = max(starts) + t
    log("f32 prefill_at")
    kc, vc = _random_cache(cfg, starts, cap, seed=24)
    x = si.layer_input(cfg, len(starts), t, seed=24)
    y, kd, vd, _ = gl.prefill(to_dev(x, cfg), cap=cap, caches=(to_dev(kc, cfg), to_dev(vc, cfg)), starts=starts)
    ref, knew, _ = oracle.layer_prefill_cached(x, gl.w_np, cfg, kc, vc, starts)
    assert_f32_parity(to_np(y), ref, "f32 prefill_at y")
    for i, n in enumerate(starts):
        assert_f32_parity(to_np(kd)[i, :, n:n + t], knew[i], f"f32 new keys {i}")


def test_profiling_reports_every_stage():
    cfg = small_bf16_cfg()
    gl = GpuLayer.seeded(cfg, seed=19)
    x = to_dev(si.layer_input(cfg, 1, 128, seed=19), cfg)
    gl.layer.set_profiling(True)
    for _ in range(3):
        gl.prefill(x)
    prof = gl.layer.read_profile()
    gl.layer.set_profiling(False)
    names = {"rmsnorm_input", "gemm_qkv", "qknorm_rope", "attention", "gemm_o_residual", "rmsnorm_post",
             "gemm_gate_up_swiglu", "gemm_down_residual"}
    assert names <= set(prof), prof
    for n in names:
        launches, ms = prof[n]
        assert launches == 3 and ms > 0
    assert gl.layer.read_profile() == {}


def test_mfma_probe_runs_and_repeats_exactly():
    """The matrix-core rate probe: finite per-lane sums, identical over two launches (the same
    MFMAs on the same register operands in the same order)."""
    import torch
    from transformer_decoder_layer_rmsnorm_amd import _native as nat
    log("mfma probe: 8 workgroups x 50 iterations, twice")
    a = torch.empty(8 * 256, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    nat.probe_mfma_rate(a, 8, 50)
    nat.probe_mfma_rate(b, 8, 50)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all()
    assert torch.equal(a, b)
    assert a.abs().max().item() > 0
