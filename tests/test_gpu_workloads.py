"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

  * 0.6B-shaped layer, B1 T2048: every output element against the oracle.
  * 8B-shaped layer, B1 T8192: every element of every stage, teacher-forced (each stage fed
    the GPU's own input for it), and every output element against the whole oracle layer.
  * 8B-shaped decode, 16 sequences on 32768 cached keys: every output row.
  * 0.6B-shaped 28-layer stack, B4 T4096: every output element of every layer against the
    oracle layer fed the GPU's bf16 input of that layer (teacher-forced), every stage of the
    first and last layers, and the final norm; the same stack in fp32 end to end at a small
    length; the bf16 end-to-end drift is reported.

Pass rule for bf16 outputs ("17. A modern architecture: Qwen3", section Why parity tests matter
now: random weights exercise every path, so a close match on them is the evidence): mean
relative error <= 5e-3 and max-abs <= 3e-2 * max(1, rms(ref)); the raw max-abs is logged beside
the scaled bar.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from gpu_support import (GpuLayer, assert_bf16_parity, assert_f32_parity, assert_rounded, bf16_metrics,
                         check_decode_steps, check_prefill_stages_full, log, oracle_layer_prefill_parallel, to_dev,
                         to_np)
from transformer_decoder_layer_rmsnorm_amd import _native as nat

pytestmark = pytest.mark.gpu


def test_qwen3_0p6b_layer_prefill_every_row():
    wl = si.WORKLOADS["qwen3-0.6b-layer-prefill"]
    cfg = wl.cfg
    log(f"{wl.name}: B{wl.batch} T{wl.seq_len}")
    gl = GpuLayer.seeded(cfg, seed=wl.seed)
    x = si.layer_input(cfg, wl.batch, wl.seq_len, seed=wl.seed)
    y, kc, vc, ws = gl.prefill(to_dev(x, cfg))
    ref = oracle.layer_prefill(x, gl.w_np, cfg)
    assert_bf16_parity(to_np(y), ref["y"], "y")
    it = gl.intermediates(ws, wl.batch, wl.seq_len)
    assert_bf16_parity(it["x1"], ref["x1"], "x1 (fp32 residual)")
    assert_bf16_parity(to_np(kc), ref["khat"], "k cache")


@pytest.mark.timeout(900)
def test_qwen3_8b_layer_prefill_every_element():
    """8B-shaped layer, B1 T8192: the QKV and gate/up projections on 256 x 256 ping-pong tiles
    (fused QK-norm / RoPE / cache epilogue; SwiGLU epilogue), o_proj and down on 256 x 256
    ping-pong tiles whose residual epilogues go through LDS, attention with 4 query heads per
    workgroup."""
    wl = si.WORKLOADS["qwen3-8b-layer-prefill"]
    cfg = wl.cfg
    log(f"{wl.name}: B{wl.batch} T{wl.seq_len}")
    gl = GpuLayer.seeded(cfg, seed=wl.seed)
    x = si.layer_input(cfg, wl.batch, wl.seq_len, seed=wl.seed)
    y, kc, vc, ws = gl.prefill(to_dev(x, cfg))
    log("  GPU done; teacher-forced stages")
    check_prefill_stages_full(gl, x, y, kc, vc, ws, "8B layer")
    log("  whole oracle layer")
    ref = oracle.layer_prefill(x, gl.w_np, cfg)
    assert_bf16_parity(to_np(y), ref["y"], "y, every element (whole oracle layer)")
    assert_bf16_parity(to_np(kc), ref["khat"], "k cache, every element")
    assert_bf16_parity(to_np(vc), ref["v"], "v cache, every element")


def test_qwen3_8b_layer_prefill_ragged_tail_rows():
    """8B shapes at T = 2600 (10 whole 256-row tiles plus a 40-row tail): the QKV and gate/up
    projections take the long-K ping-pong GEMM with a partial last row tile, o_proj and down
    the smaller tiles; rows in and around the tail are checked."""
    wl = si.WORKLOADS["qwen3-8b-layer-prefill"]
    cfg = wl.cfg
    t_len = 2600
    log(f"8B-shaped layer: B1 T{t_len}")
    gl = GpuLayer.seeded(cfg, seed=wl.seed)
    x = si.layer_input(cfg, 1, t_len, seed=wl.seed)
    y, kc, vc, ws = gl.prefill(to_dev(x, cfg))
    ts = [0, 255, 256, 1999, 2559, 2560, 2561, 2580, 2598, 2599]
    ref = oracle.layer_prefill_rows(x, gl.w_np, cfg, [(0, t) for t in ts])
    assert_bf16_parity(to_np(y)[0, ts], ref, f"y at {len(ts)} rows incl. the 40-row tail")


def test_qwen3_8b_layer_prefill_thin_every_element():
    """8B shapes at T = 300 (four whole 64-row tiles plus a 44-row tail, 160 tiles of 64 x 128):
    o_proj (K = 4096) and down (K = 12288, 96 stages of the ring) take the deep-ring GEMM with
    the residual in its epilogue; every element of y and of the caches against the oracle."""
    wl = si.WORKLOADS["qwen3-8b-layer-prefill"]
    cfg = wl.cfg
    t_len = 300
    log(f"8B-shaped layer: B1 T{t_len}")
    gl = GpuLayer.seeded(cfg, seed=wl.seed + 3)
    x = si.layer_input(cfg, 1, t_len, seed=wl.seed + 3)
    y, kc, vc, ws = gl.prefill(to_dev(x, cfg))
    ref = oracle.layer_prefill(x, gl.w_np, cfg)
    assert_bf16_parity(to_np(y), ref["y"], "y, every element")
    assert_bf16_parity(to_np(kc), ref["khat"], "k cache, every element")


def test_qwen3_0p6b_layer_prefill_ragged_tail_rows():
    """0.6B shapes at T = 2088 (32 whole 64-row tiles plus a 40-row tail): o_proj and down take
    the deep-ring 64 x 128 tiles with the residual in their epilogue, gate/up the 256 x 256
    ping-pong tiles, QKV the fused 256 x 128 ping-pong kernel, all with a partial last row tile;
    rows in and around the tail are checked."""
    wl = si.WORKLOADS["qwen3-0.6b-layer-prefill"]
    cfg = wl.cfg
    t_len = 2088
    log(f"0.6B-shaped layer: B1 T{t_len}")
    gl = GpuLayer.seeded(cfg, seed=wl.seed)
    x = si.layer_input(cfg, 1, t_len, seed=wl.seed)
    y, kc, vc, ws = gl.prefill(to_dev(x, cfg))
    ts = [0, 63, 64, 1000, 2047, 2048, 2049, 2070, 2086, 2087]
    ref = oracle.layer_prefill_rows(x, gl.w_np, cfg, [(0, t) for t in ts])
    assert_bf16_parity(to_np(y)[0, ts], ref, f"y at {len(ts)} rows incl. the 40-row tail")


def test_qwen3_8b_decode_32k_every_row():
    wl = si.WORKLOADS["qwen3-8b-layer-decode-32k"]
    cfg = wl.cfg
    b, n = wl.batch, wl.cached
    cap = n + 1
    log(f"{wl.name}: B{b}, {n} cached keys, capacity {cap}")
    gl = GpuLayer.seeded(cfg, seed=wl.seed)
    shape = (b, cfg.num_key_value_heads, cap, cfg.head_dim)
    kc = np.zeros(shape, np.float32)
    vc = np.zeros(shape, np.float32)

    def sink(i, h, kb, vb):
        kc[i, h, :n] = kb
        vc[i, h, :n] = vb

    si.fill_decode_cache(cfg, b, n, sink, seed=wl.seed)
    log("  cache generated")
    kd, vd = to_dev(kc, cfg), to_dev(vc, cfg)
    x = si.layer_input(cfg, b, 1, seed=wl.seed)
    y, ws = gl.decode(to_dev(x, cfg), [n] * b, kd, vd)
    ref, _, _ = oracle.layer_decode(x, gl.w_np, cfg, kc, vc, [n] * b)
    assert_bf16_parity(to_np(y), ref, "decode y (16 rows)")
    del kc, vc
    check_decode_steps(gl, ws, [n] * b, kd, vd)


@pytest.mark.timeout(900)
def test_qwen3_0p6b_stack28_teacher_forced():
    """28 layers on B4 T4096 (M = 16384): QKV and gate/up on 256 x 256 ping-pong tiles at
    K = 1024, o_proj and down on 256 x 256 ping-pong tiles with residual epilogues through LDS,
    attention with two query heads per workgroup and whole 64-key tiles per wave."""
    wl = si.WORKLOADS["qwen3-0.6b-stack28-prefill"]
    cfg = wl.cfg
    b, t = wl.batch, wl.seq_len
    log(f"{wl.name}: B{b} T{t}, {wl.layers} layers + final norm")
    x = si.layer_input(cfg, b, t, seed=wl.seed)
    cur = to_dev(x, cfg)
    kc = vc = ws = None
    worst = None
    for layer in range(wl.layers):
        gl = GpuLayer.seeded(cfg, layer=layer, seed=wl.seed)
        if kc is None:
            kc, vc = gl.alloc_cache(b, t)
            ws = gl.workspace(b, t, t)
        y, *_ = gl.prefill(cur, caches=(kc, vc), ws=ws)
        xin = to_np(cur)
        if layer in (0, wl.layers - 1):
            check_prefill_stages_full(gl, xin, y, kc, vc, ws, f"stack layer {layer}")
        ref = oracle_layer_prefill_parallel(xin, gl.w_np, cfg)
        m = assert_bf16_parity(to_np(y), ref["y"], f"layer {layer} y, every element (teacher-forced)")
        worst = m if worst is None or m["mean_rel"] > worst["mean_rel"] else worst
        cur = y
        del gl, ref
    gain = si.final_norm_gain(cfg, seed=wl.seed)
    gd = to_dev(gain, cfg)
    out = torch.empty_like(cur)
    nat.rmsnorm(cur, gd, out, cfg.rms_norm_eps)
    torch.cuda.synchronize()
    assert_rounded(to_np(out), oracle.rmsnorm(to_np(cur), gain, cfg.rms_norm_eps), "final norm (teacher-forced)")
    log(f"  worst layer mean_rel {worst['mean_rel']:.3g}, max_abs {worst['max_abs']:.3g} "
        f"(bar {worst['max_abs_bar']:.3g})")


def run_stack(cfg, x, layers, seed, gain):
    cur = to_dev(x, cfg)
    b, t, _ = x.shape
    kc = vc = ws = None
    for layer in range(layers):
        gl = GpuLayer.seeded(cfg, layer=layer, seed=seed)
        if kc is None:
            kc, vc = gl.alloc_cache(b, t)
            ws = gl.workspace(b, t, t)
        cur, *_ = gl.prefill(cur, caches=(kc, vc), ws=ws)
    out = torch.empty_like(cur)
    nat.rmsnorm(cur, to_dev(gain, cfg), out, cfg.rms_norm_eps)
    torch.cuda.synchronize()
    return to_np(out)


def test_stack28_fp32_end_to_end():
    cfg = si.with_dtype(si.QWEN3_0P6B, "f32")
    b, t, layers = 2, 48, 28
    log(f"fp32 stack of {layers} 0.6B-shaped layers, B{b} T{t}")
    x = si.layer_input(cfg, b, t, seed=4)
    gain = si.final_norm_gain(cfg, seed=4)
    got = run_stack(cfg, x, layers, 4, gain)
    ws = [si.layer_weights(cfg, layer=l, seed=4) for l in range(layers)]
    ref = oracle.stack_prefill(x, ws, gain, cfg)
    assert_f32_parity(got, ref, "final-normed output")


def test_stack28_bf16_end_to_end_drift_reported():
    cfg = si.QWEN3_0P6B
    b, t, layers = 1, 256, 28
    x = si.layer_input(cfg, b, t, seed=6)
    gain = si.final_norm_gain(cfg, seed=6)
    got = run_stack(cfg, x, layers, 6, gain)
    ws = [si.layer_weights(cfg, layer=l, seed=6) for l in range(layers)]
    ref = oracle.stack_prefill(x, ws, gain, cfg, round_between=si.round_to_bf16)
    m = bf16_metrics(got, ref)
    log(f"  bf16 28-layer end-to-end drift (reported, not gated): max_abs {m['max_abs']:.3g}, "
        f"mean_rel {m['mean_rel']:.3g}")
    assert np.all(np.isfinite(got))
    assert m["mean_rel"] < 0.05   # gross-error guard only
