"""GPU parity of left-padded batches ("Transformer architectures: from BERT to diffusion,
lesson 6", section 8, batched generation): prompts padded on the left, padding attended by
nobody but itself, positions counted from each row's first real token, optionally after a
shared prefix, followed by decode steps that keep the padding unattended.  Every case runs
through the C ABI (qwen3_layer_prefill_padded / qwen3_layer_decode_padded) and is compared
with the oracle's layer_prefill_padded / layer_decode_padded."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_support import GpuLayer, assert_bf16_parity, assert_f32_parity, log, small_bf16_cfg, to_dev, to_np

pytestmark = pytest.mark.gpu


def _check_cache(kg, vg, knew, vnew, starts, t, what, f32=False):
    for i, n in enumerate(starts):
        if f32:
            assert_f32_parity(kg[i, :, n:n + t], knew[i], f"{what}: keys of sequence {i}")
            assert_f32_parity(vg[i, :, n:n + t], vnew[i], f"{what}: values of sequence {i}")
        else:
            assert_bf16_parity(kg[i, :, n:n + t], knew[i], f"{what}: keys of sequence {i}")
            assert_bf16_parity(vg[i, :, n:n + t], vnew[i], f"{what}: values of sequence {i}")


@pytest.mark.parametrize("hq,hkv,t", [(4, 2, 77), (8, 1, 33), (8, 8, 130)])
def test_bf16_padded_prefill_matches_oracle(hq, hkv, t):
    # pads from none to the whole row (a row of pure padding: every token sees only itself)
    cfg = small_bf16_cfg(hq=hq, hkv=hkv)
    gl = GpuLayer.seeded(cfg, seed=31)
    pads = sorted({0, 1, t // 3, min(64, t - 1), t - 1, t})
    b = len(pads)
    log(f"bf16 padded prefill Hq{hq} Hkv{hkv} T{t} pads {pads}")
    x = si.layer_input(cfg, b, t, seed=31)
    y, kd, vd, _ = gl.prefill(to_dev(x, cfg), pads=pads)
    zero = np.zeros((b, hkv, t, cfg.head_dim))
    ref, knew, vnew = oracle.layer_prefill_padded(x, gl.w_np, cfg, zero, zero, [0] * b, pads)
    assert_bf16_parity(to_np(y), ref, "padded prefill y (padding rows included)")
    for i, pad in enumerate(pads):
        if pad < t:
            assert_bf16_parity(to_np(y)[i, pad:], ref[i, pad:], f"real rows of sequence {i} (pad {pad})")
    _check_cache(to_np(kd), to_np(vd), knew, vnew, [0] * b, t, "padded prefill")


def test_bf16_padded_rows_equal_unpadded_rows():
    # the real rows of a padded row and the same tokens prefilled alone agree (the GPU against
    # itself, at the bf16 bar: the two runs tile the keys differently)
    cfg = small_bf16_cfg()
    gl = GpuLayer.seeded(cfg, seed=32)
    t, pads = 96, [0, 17, 70]
    x = si.layer_input(cfg, len(pads), t, seed=32)
    y, *_ = gl.prefill(to_dev(x, cfg), pads=pads)
    for i, pad in enumerate(pads):
        alone, *_ = gl.prefill(to_dev(x[i:i + 1, pad:], cfg))
        assert_bf16_parity(to_np(y)[i, pad:], to_np(alone)[0], f"sequence {i}: padded vs alone")


def test_bf16_prefix_padded_prefill_then_padded_decode():
    # shared prefix (a plain prefill), left-padded prompts after it, then three decode steps
    cfg = small_bf16_cfg(hq=8, hkv=2)
    gl = GpuLayer.seeded(cfg, seed=33)
    p0, t, steps = 70, 45, 3
    pads = [0, 9, 44, 30]
    b = len(pads)
    cap = p0 + t + steps
    log(f"bf16 prefix {p0} + padded {t} (pads {pads}) + {steps} decode steps")
    prefix = si.layer_input(cfg, 1, p0, seed=33)
    kd, vd = gl.alloc_cache(b, cap)
    xp = to_dev(np.repeat(prefix, b, axis=0), cfg)
    gl.prefill(xp, cap=cap, caches=(kd, vd))
    kc, vc = to_np(kd), to_np(vd)             # the oracle continues from the GPU's own prefix cache
    x = si.layer_input(cfg, b, t + steps, seed=34)
    y, kd, vd, _ = gl.prefill(to_dev(x[:, :t], cfg), cap=cap, caches=(kd, vd), starts=[p0] * b, pads=pads)
    ref, knew, vnew = oracle.layer_prefill_padded(x[:, :t], gl.w_np, cfg, kc, vc, [p0] * b, pads)
    assert_bf16_parity(to_np(y), ref, "prefix + padded prefill y")
    _check_cache(to_np(kd), to_np(vd), knew, vnew, [p0] * b, t, "prefix + padded prefill")
    for s in range(steps):
        n = p0 + t + s
        kc, vc = to_np(kd), to_np(vd)
        yd, _ = gl.decode(to_dev(x[:, t + s:t + s + 1], cfg), [n] * b, kd, vd, pad_starts=[p0] * b, pad_lens=pads)
        ref_d, kn, vn = oracle.layer_decode_padded(x[:, t + s:t + s + 1], gl.w_np, cfg, kc, vc, [n] * b,
                                                   [p0] * b, pads)
        assert_bf16_parity(to_np(yd), ref_d, f"padded decode step {s}")
        assert_bf16_parity(to_np(kd)[:, :, n], kn, f"decode step {s} new keys")


def test_bf16_padded_decode_masks_whole_splits():
    # a padding run longer than a 512-key split: whole splits of the decode kernel see no key
    cfg = small_bf16_cfg(hq=4, hkv=2)
    gl = GpuLayer.seeded(cfg, seed=35)
    n, cap = 1700, 1800
    pad_starts, pad_lens = [0, 100, 1], [1300, 1024, 0]
    b = len(pad_lens)
    log(f"bf16 padded decode over {n} cached keys, padding runs {list(zip(pad_starts, pad_lens))}")
    kc = np.zeros((b, 2, cap, 128), np.float32)
    vc = np.zeros((b, 2, cap, 128), np.float32)
    for i in range(b):
        for h in range(2):
            kc[i, h, :n] = si.cache_block(cfg, "k", i, h, n, seed=35)
            vc[i, h, :n] = si.cache_block(cfg, "v", i, h, n, seed=35)
    kd, vd = to_dev(kc, cfg), to_dev(vc, cfg)
    x = si.layer_input(cfg, b, 1, seed=35)
    y, _ = gl.decode(to_dev(x, cfg), [n] * b, kd, vd, pad_starts=pad_starts, pad_lens=pad_lens)
    kc16, vc16 = to_np(kd), to_np(vd)
    ref, _, _ = oracle.layer_decode_padded(x, gl.w_np, cfg, kc16, vc16, [n] * b, pad_starts, pad_lens)
    assert_bf16_parity(to_np(y), ref, "padded decode y")


def test_bf16_padded_many_sequences_values_in_workspace():
    # more than 64 sequences: starts and padding travel through the workspace
    cfg = small_bf16_cfg()
    gl = GpuLayer.seeded(cfg, seed=36)
    b, t = 67, 9
    pads = [(3 * i) % (t + 1) for i in range(b)]
    starts = [(7 * i) % 11 for i in range(b)]
    cap = max(starts) + t + 1
    kc = np.zeros((b, 2, cap, 128), np.float32)
    vc = np.zeros((b, 2, cap, 128), np.float32)
    for i, n in enumerate(starts):
        for h in range(2):
            kc[i, h, :n] = si.cache_block(cfg, "k", i, h, n, seed=36)
            vc[i, h, :n] = si.cache_block(cfg, "v", i, h, n, seed=36)
    kd, vd = to_dev(kc, cfg), to_dev(vc, cfg)
    kc16, vc16 = to_np(kd), to_np(vd)
    x = si.layer_input(cfg, b, t + 1, seed=36)
    y, kd, vd, _ = gl.prefill(to_dev(x[:, :t], cfg), cap=cap, caches=(kd, vd), starts=starts, pads=pads)
    ref, _, _ = oracle.layer_prefill_padded(x[:, :t], gl.w_np, cfg, kc16, vc16, starts, pads)
    assert_bf16_parity(to_np(y), ref, f"padded prefill y, {b} sequences")
    lens = [s + t for s in starts]
    kc16, vc16 = to_np(kd), to_np(vd)
    yd, _ = gl.decode(to_dev(x[:, t:], cfg), lens, kd, vd, pad_starts=starts, pad_lens=pads)
    ref_d, _, _ = oracle.layer_decode_padded(x[:, t:], gl.w_np, cfg, kc16, vc16, lens, starts, pads)
    assert_bf16_parity(to_np(yd), ref_d, f"padded decode y, {b} sequences")


def test_bf16_padded_many_sequences_ping_pong_qkv_epilogue():
    # 96 sequences x 32 tokens with Hq 16 / Hkv 8: the 3072 x 4096 QKV projection takes 256 x 256
    # ping-pong tiles with the QK-norm / RoPE / cache-write epilogue, which reads the starts and
    # the padding from the workspace arrays (more than 64 sequences)
    cfg = small_bf16_cfg(hq=16, hkv=8)
    gl = GpuLayer.seeded(cfg, seed=38)
    b, t = 96, 32
    pads = [(5 * i) % (t + 1) for i in range(b)]
    starts = [(13 * i) % 29 for i in range(b)]
    cap = max(starts) + t
    log(f"bf16 padded prefill, {b} sequences x T{t}, Hq16 Hkv8 (ping-pong QKV epilogue)")
    kc = np.zeros((b, 8, cap, 128), np.float32)
    vc = np.zeros((b, 8, cap, 128), np.float32)
    for i, n in enumerate(starts):
        for h in range(8):
            kc[i, h, :n] = si.cache_block(cfg, "k", i, h, n, seed=38)
            vc[i, h, :n] = si.cache_block(cfg, "v", i, h, n, seed=38)
    kd, vd = to_dev(kc, cfg), to_dev(vc, cfg)
    kc16, vc16 = to_np(kd), to_np(vd)
    x = si.layer_input(cfg, b, t, seed=38)
    y, kd, vd, _ = gl.prefill(to_dev(x, cfg), cap=cap, caches=(kd, vd), starts=starts, pads=pads)
    ref, knew, vnew = oracle.layer_prefill_padded(x, gl.w_np, cfg, kc16, vc16, starts, pads)
    assert_bf16_parity(to_np(y), ref, f"padded prefill y, {b} sequences")
    _check_cache(to_np(kd), to_np(vd), knew, vnew, starts, t, "padded prefill (ping-pong epilogue)")


def _padded_prefix_0p6b(b, t, starts, pads, seed, what):
    wl = si.WORKLOADS["qwen3-0.6b-layer-prefill"]
    cfg = wl.cfg
    gl = GpuLayer.seeded(cfg, seed=seed)
    hkv, d = cfg.num_key_value_heads, cfg.head_dim
    cap = max(starts) + t
    log(f"bf16 padded prefill on prefixes, 0.6B shapes, B{b} T{t} ({what})")
    kc = np.zeros((b, hkv, cap, d), np.float32)
    vc = np.zeros((b, hkv, cap, d), np.float32)
    for i, n in enumerate(starts):
        for h in range(hkv):
            kc[i, h, :n] = si.cache_block(cfg, "k", i, h, n, seed=seed)
            vc[i, h, :n] = si.cache_block(cfg, "v", i, h, n, seed=seed)
    kd, vd = to_dev(kc, cfg), to_dev(vc, cfg)
    kc16, vc16 = to_np(kd), to_np(vd)
    x = si.layer_input(cfg, b, t, seed=seed)
    y, kd, vd, _ = gl.prefill(to_dev(x, cfg), cap=cap, caches=(kd, vd), starts=starts, pads=pads)
    ref, knew, vnew = oracle.layer_prefill_padded(x, gl.w_np, cfg, kc16, vc16, starts, pads)
    assert_bf16_parity(to_np(y), ref, f"padded prefill y on prefixes (0.6B shapes, {what})")
    _check_cache(to_np(kd), to_np(vd), knew, vnew, starts, t, f"padded prefill ({what})")


def test_bf16_padded_prefix_0p6b_fused_qkv_epilogue():
    # 0.6B shapes, 2 sequences x 1024 tokens after prefixes of 100 and 37 keys, the second with
    # 300 tokens of left padding: the QKV projection (2048 x 4096) takes 256 x 128 ping-pong
    # tiles with the QK-norm / RoPE / cache-write epilogue, whose angles and slots come from the
    # table the input RMSNorm builds from the inline starts and padding
    _padded_prefix_0p6b(2, 1024, [100, 37], [0, 300], 39, "fused 256 x 128 ping-pong epilogue")


def test_bf16_padded_prefix_0p6b_fused_qkv_register_tiles():
    # one sequence of 1200 tokens after a 100-key prefix, 300 of them left padding: the QKV
    # projection (1200 x 4096) has too few 256-row tiles for the ping-pong forms and takes the
    # 128 x 128 register-tile kernel with the same epilogue, its last row tile partial (48 rows)
    _padded_prefix_0p6b(1, 1200, [100], [300], 40, "fused 128 x 128 epilogue")


def test_f32_padded_prefill_and_decode():
    cfg = si.TINY_F32
    gl = GpuLayer.seeded(cfg, seed=37)
    t, pads = 12, [0, 5, 11, 12]
    b = len(pads)
    cap = t + 1
    log("f32 padded prefill + decode")
    x = si.layer_input(cfg, b, t + 1, seed=37)
    kd, vd = gl.alloc_cache(b, cap)
    y, kd, vd, _ = gl.prefill(to_dev(x[:, :t], cfg), cap=cap, caches=(kd, vd), pads=pads)
    zero = np.zeros((b, cfg.num_key_value_heads, cap, cfg.head_dim))
    ref, knew, vnew = oracle.layer_prefill_padded(x[:, :t], gl.w_np, cfg, zero, zero, [0] * b, pads)
    assert_f32_parity(to_np(y), ref, "f32 padded prefill y")
    _check_cache(to_np(kd), to_np(vd), knew, vnew, [0] * b, t, "f32 padded prefill", f32=True)
    kc, vc = to_np(kd), to_np(vd)
    yd, _ = gl.decode(to_dev(x[:, t:], cfg), [t] * b, kd, vd, pad_starts=[0] * b, pad_lens=pads)
    ref_d, _, _ = oracle.layer_decode_padded(x[:, t:], gl.w_np, cfg, kc, vc, [t] * b, [0] * b, pads)
    assert_f32_parity(to_np(yd), ref_d, "f32 padded decode y")
