"""GPU parity over a seeded sweep of layer shapes, each a prefill followed by one decode step,
every output element against the oracle.

The shapes are drawn (fixed seed) from head groupings g = 1, 2, 4, 8 over 1-8 KV heads, hidden and
intermediate widths that are odd multiples of 128, 1-5 sequences and lengths from 1 token to
past a thousand, so that between them they land on both sides of the kernel choices: 256 x 256
ping-pong, 128 x 128, deep-ring and small-tile projections (with and without a partial last row
tile), the two-group and the 4-wave attention (split tiles or whole tiles, 1, 2 or 4 heads per
wave), and every decode attention grouping.  The layer runs on a cache one slot longer than the
prompt; the prompt's last token is then decoded onto it, so one oracle prefill over T + 1 tokens
gives the expected prefill rows (causality) and the decode row.  Pass rule as everywhere for bf16
outputs ("17. A modern architecture: Qwen3", section Why parity tests matter now): mean relative
error <= 5e-3 and max-abs <= 3e-2 * max(1, rms(ref)).
"""
import numpy as np
import pytest

import seeded_inputs as si
from gpu_support import (GpuLayer, assert_bf16_parity, log, oracle_layer_prefill_parallel, small_bf16_cfg, to_dev,
                         to_np)

pytestmark = pytest.mark.gpu


def _cases(n=12, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        g = int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.choice([1, 2, 4, 8]))
        if g * hkv > 32:
            continue
        hidden = 128 * int(rng.choice([1, 2, 3, 5, 8, 9]))
        inter = 128 * int(rng.choice([1, 3, 6, 11]))
        b = int(rng.choice([1, 2, 3, 5]))
        t = int(rng.choice([1, 2, 63, 64, 65, 255, 257, 700, 1000, 1200, 2049]))
        # keep the float64 oracle within seconds: attention work ~ B Hq T^2
        if b * g * hkv * t * t > 3e8:
            continue
        cases.append((g * hkv, hkv, hidden, inter, b, t))
    # two shapes long enough for the two-group attention (>= 512 workgroups) and 256 x 256 ping-pong
    # projections: 8 heads per KV head (4 per wave) with the fused QKV on ping-pong tiles; one head per
    # KV head with every projection on ping-pong tiles and a partial last row tile (M = 16376)
    cases += [(32, 4, 512, 640, 4, 1100), (8, 8, 1024, 1536, 8, 2047)]
    return cases


@pytest.mark.parametrize("hq,hkv,hidden,inter,b,t", _cases())
def test_bf16_layer_sweep_prefill_then_decode(hq, hkv, hidden, inter, b, t):
    cfg = small_bf16_cfg(hq=hq, hkv=hkv, hidden=hidden, inter=inter)
    seed = hq * 7 + hidden + inter + b * 13 + t
    log(f"sweep: Hq{hq} Hkv{hkv} hidden {hidden} inter {inter} B{b} T{t} (+1 decoded)")
    gl = GpuLayer.seeded(cfg, seed=seed)
    x = si.layer_input(cfg, b, t + 1, seed=seed)
    cap = t + 1
    kc, vc = gl.alloc_cache(b, cap)
    y, kc, vc, _ = gl.prefill(to_dev(x[:, :t], cfg), cap=cap, caches=(kc, vc))
    ref = oracle_layer_prefill_parallel(x, gl.w_np, cfg)
    assert_bf16_parity(to_np(y), ref["y"][:, :t], "prefill y, every element")
    kn = to_np(kc)
    assert_bf16_parity(kn[:, :, :t], ref["khat"][:, :, :t], "k cache after prefill")
    assert not np.any(kn[:, :, t:]), "prefill left the slot past the prompt untouched"
    yd, _ = gl.decode(to_dev(x[:, t:], cfg), [t] * b, kc, vc)
    assert_bf16_parity(to_np(yd)[:, 0], ref["y"][:, t], f"decode row at position {t}")
    assert_bf16_parity(to_np(vc)[:, :, t], ref["v"][:, :, t], "decode wrote the new value row")
