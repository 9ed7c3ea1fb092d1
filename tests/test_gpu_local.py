"""GPU parity of local (sliding-window) layers ("Transformer architectures: from BERT to
diffusion, lesson 6", section 7): the banded prefill with attention sinks, decode under the
window on a full cache, and decode on a rolling buffer, through the C ABI
(qwen3_layer_prefill_window / qwen3_layer_decode_window), against the oracle's
layer_prefill_window / layer_decode_window / layer_decode_rolling; and the page's own check,
the banded prefill against a token-by-token run on a rolling buffer."""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from gpu_support import GpuLayer, assert_bf16_parity, assert_f32_parity, log, small_bf16_cfg, to_dev, to_np

pytestmark = pytest.mark.gpu


def prefill_window(gl, x_dev, window, sinks, cap=None, caches=None, starts=None):
    b, t, _ = x_dev.shape
    cap = cap or t
    kc, vc = caches or gl.alloc_cache(b, cap)
    ws = gl.workspace(b, t, cap)
    y = torch.empty_like(x_dev)
    gl.layer.prefill_window(x_dev, y, kc, vc, ws, window, sinks, start_positions=starts)
    torch.cuda.synchronize()
    return y, kc, vc


def decode_window(gl, x_dev, positions, kc, vc, window, sinks, rolling):
    b = x_dev.shape[0]
    ws = gl.workspace(b, 1, kc.shape[2])
    y = torch.empty_like(x_dev)
    gl.layer.decode_window(x_dev, y, positions, kc, vc, ws, window, sinks, rolling=rolling)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("hq,hkv,t,window,sinks", [
    (4, 2, 700, 100, 4),      # window inside two tiles, 4 sinks
    (4, 2, 700, 64, 0),       # window of exactly one tile, no sinks
    (8, 1, 333, 17, 70),      # narrow window, sinks spanning more than a tile (MQA)
    (8, 8, 257, 300, 2),      # window longer than the text: global plus nothing (MHA)
    (4, 2, 130, 1, 0),        # every token sees only itself
])
def test_bf16_banded_prefill_matches_oracle(hq, hkv, t, window, sinks):
    cfg = small_bf16_cfg(hq=hq, hkv=hkv)
    gl = GpuLayer.seeded(cfg, seed=51)
    log(f"bf16 banded prefill Hq{hq} Hkv{hkv} T{t} window {window} sinks {sinks}")
    x = si.layer_input(cfg, 2, t, seed=51)
    y, kd, vd = prefill_window(gl, to_dev(x, cfg), window, sinks)
    ref, kref, vref = oracle.layer_prefill_window(x, gl.w_np, cfg, window, sinks)
    assert_bf16_parity(to_np(y), ref, "banded prefill y")
    assert_bf16_parity(to_np(kd), kref, "cached keys")


def test_bf16_banded_chunked_prefill():
    # a banded prefill continued on a linear cache equals the one-shot banded prefill
    cfg = small_bf16_cfg()
    gl = GpuLayer.seeded(cfg, seed=52)
    t1, t2, window, sinks = 300, 200, 128, 4
    x = si.layer_input(cfg, 2, t1 + t2, seed=52)
    log(f"bf16 banded chunked prefill {t1} + {t2}, window {window}, sinks {sinks}")
    cap = t1 + t2
    kc, vc = gl.alloc_cache(2, cap)
    y1, *_ = prefill_window(gl, to_dev(x[:, :t1], cfg), window, sinks, cap=cap, caches=(kc, vc))
    y2, *_ = prefill_window(gl, to_dev(x[:, t1:], cfg), window, sinks, cap=cap, caches=(kc, vc), starts=[t1, t1])
    ref, _, _ = oracle.layer_prefill_window(x, gl.w_np, cfg, window, sinks)
    got = np.concatenate([to_np(y1), to_np(y2)], axis=1)
    assert_bf16_parity(got, ref, "chunked banded prefill y")


def test_bf16_window_decode_on_long_linear_cache():
    # 3000 cached keys, window 600 and 4 sinks: most 512-key splits are skipped
    cfg = small_bf16_cfg(hq=8, hkv=2)
    gl = GpuLayer.seeded(cfg, seed=53)
    n, window, sinks = 3000, 600, 4
    cap = n + 1
    b = 2
    log(f"bf16 window decode over {n} keys, window {window}, sinks {sinks}")
    kc = np.zeros((b, 2, cap, 128), np.float32)
    vc = np.zeros((b, 2, cap, 128), np.float32)
    for i in range(b):
        for h in range(2):
            kc[i, h, :n] = si.cache_block(cfg, "k", i, h, n, seed=53)
            vc[i, h, :n] = si.cache_block(cfg, "v", i, h, n, seed=53)
    kd, vd = to_dev(kc, cfg), to_dev(vc, cfg)
    x = si.layer_input(cfg, b, 1, seed=53)
    y = decode_window(gl, to_dev(x, cfg), [n, n - 7], kd, vd, window, sinks, rolling=False)
    ref, _, _ = oracle.layer_decode_window(x, gl.w_np, cfg, to_np(kd), to_np(vd), [n, n - 7], window, sinks)
    assert_bf16_parity(to_np(y), ref, "window decode y")


@pytest.mark.parametrize("window,sinks", [(16, 0), (24, 4), (64, 2)])
def test_bf16_rolling_buffer_equals_banded_prefill(window, sinks):
    # the page's check: a token-by-token run on a rolling buffer of sinks + window slots (no mask)
    # against the banded prefill; the run wraps the buffer several times
    cfg = small_bf16_cfg(hq=4, hkv=2)
    gl = GpuLayer.seeded(cfg, seed=54)
    t = 3 * (window + sinks) + 5
    b = 2
    log(f"bf16 rolling buffer window {window} sinks {sinks}: {t} decode steps")
    x = si.layer_input(cfg, b, t, seed=54)
    banded, _, _ = prefill_window(gl, to_dev(x, cfg), window, sinks)
    kd, vd = gl.alloc_cache(b, sinks + window)
    steps = []
    for i in range(t):
        steps.append(to_np(decode_window(gl, to_dev(x[:, i:i + 1], cfg), [i] * b, kd, vd, window, sinks,
                                         rolling=True)))
    got = np.concatenate(steps, axis=1)
    ref, _, _ = oracle.layer_prefill_window(x, gl.w_np, cfg, window, sinks)
    assert_bf16_parity(got, ref, "rolling decode vs oracle banded prefill")
    assert_bf16_parity(got, to_np(banded), "rolling decode vs GPU banded prefill")


def test_f32_local_layers():
    cfg = si.TINY_F32
    gl = GpuLayer.seeded(cfg, seed=55)
    t, window, sinks = 21, 5, 2
    log("f32 banded prefill, window decode and rolling decode")
    x = si.layer_input(cfg, 2, t, seed=55)
    ref, _, _ = oracle.layer_prefill_window(x, gl.w_np, cfg, window, sinks)
    y, kd, vd = prefill_window(gl, to_dev(x, cfg), window, sinks)
    assert_f32_parity(to_np(y), ref, "f32 banded prefill y")
    kd2, vd2 = gl.alloc_cache(2, sinks + window)
    steps = [to_np(decode_window(gl, to_dev(x[:, i:i + 1], cfg), [i, i], kd2, vd2, window, sinks, rolling=True))
             for i in range(t)]
    assert_f32_parity(np.concatenate(steps, axis=1), ref, "f32 rolling decode")
    kl, vl = gl.alloc_cache(2, t)
    prefill_window(gl, to_dev(x[:, :t - 1], cfg), window, sinks, cap=t, caches=(kl, vl))
    yl = decode_window(gl, to_dev(x[:, t - 1:], cfg), [t - 1, t - 1], kl, vl, window, sinks, rolling=False)
    assert_f32_parity(to_np(yl)[:, 0], ref[:, t - 1], "f32 window decode on a linear cache")
