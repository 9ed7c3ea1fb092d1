"""GPU parity of the RoPE and RMSNorm variants of "17. A modern architecture: Qwen3"
(sections RMSNorm and Rotary position embeddings, and its exercises): partial RoPE (only the
first rotary_dim features rotated), adjacent-pair RoPE, linear RoPE position scaling, and
zero-centred RMSNorm gains (1 + g), each through the C ABI against the oracle, in prefill and
decode, bf16 and fp32."""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from gpu_support import GpuLayer, assert_bf16_parity, assert_f32_parity, log, small_bf16_cfg, to_dev, to_np
from transformer_decoder_layer_rmsnorm_amd import _native as nat

pytestmark = pytest.mark.gpu

VARIANTS = [
    dict(rotary_dim=64),
    dict(rope_adjacent_pairs=True),
    dict(rotary_dim=32, rope_adjacent_pairs=True),
    dict(rope_position_scale=0.25),
    dict(norm_unit_offset=True),
    dict(rotary_dim=96, rope_position_scale=0.5, norm_unit_offset=True),
]


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: "-".join(f"{k}={v[k]}" for k in v))
def test_bf16_variant_prefill_and_decode(variant):
    base = small_bf16_cfg(hq=4, hkv=2)
    cfg = si.LayerConfig(**{**base.__dict__, **variant})
    gl = GpuLayer.seeded(cfg, seed=71)
    t, b = 150, 2
    log(f"bf16 variant {variant}: prefill T{t}, then one decode step")
    x = si.layer_input(cfg, b, t + 1, seed=71)
    cap = t + 1
    kd, vd = gl.alloc_cache(b, cap)
    y, kd, vd, _ = gl.prefill(to_dev(x[:, :t], cfg), cap=cap, caches=(kd, vd))
    ref = oracle.layer_prefill(x[:, :t], gl.w_np, cfg)
    assert_bf16_parity(to_np(y), ref["y"], "prefill y")
    assert_bf16_parity(to_np(kd)[:, :, :t], ref["khat"], "cached keys")
    kc, vc = to_np(kd), to_np(vd)
    yd, _ = gl.decode(to_dev(x[:, t:], cfg), [t] * b, kd, vd)
    ref_d, kn, _ = oracle.layer_decode(x[:, t:], gl.w_np, cfg, kc, vc, [t] * b)
    assert_bf16_parity(to_np(yd), ref_d, "decode y")
    assert_bf16_parity(to_np(kd)[:, :, t], kn, "decode new key")


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: "-".join(f"{k}={v[k]}" for k in v))
def test_f32_variant_prefill(variant):
    v = dict(variant)
    if v.get("rotary_dim", 0) > 32:
        v["rotary_dim"] = 16
    cfg = si.LayerConfig(**{**si.TINY_F32.__dict__, **v})
    gl = GpuLayer.seeded(cfg, seed=72)
    x = si.layer_input(cfg, 2, 16, seed=72)
    y, kd, _, _ = gl.prefill(to_dev(x, cfg))
    ref = oracle.layer_prefill(x, gl.w_np, cfg)
    assert_f32_parity(to_np(y), ref["y"], f"f32 variant {v} y")
    assert_f32_parity(to_np(kd), ref["khat"], f"f32 variant {v} keys")


def test_zero_centred_final_norm():
    cfg = si.LayerConfig(**{**small_bf16_cfg().__dict__, "norm_unit_offset": True})
    gain = si.final_norm_gain(cfg, seed=73)
    x = si.layer_input(cfg, 3, 37, seed=73)
    xd, gd = to_dev(x, cfg), to_dev(gain, cfg)
    yd = torch.empty_like(xd)
    nat.rmsnorm(xd, gd, yd, cfg.rms_norm_eps, gain_offset=1.0)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(x, 1.0 + gain.astype(np.float64), cfg.rms_norm_eps)
    assert_bf16_parity(to_np(yd), ref, "zero-centred final norm")
