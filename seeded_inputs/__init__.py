"""Seeded synthetic inputs for the Qwen3-style decoder layer.

This module is shared by the float64 oracle side (tests, CPU baseline) and by the
HIP side (tests, bench).  It holds the workload shapes and the random draws only:
none of the layer's arithmetic lives here.

Recipe (the pages print no seeds, weights or data for this path):
  * every tensor is drawn from numpy's PCG64 seeded with
    ``SeedSequence([seed, layer, tensor_id])``; float32 standard normals, scaled,
  * projection matrices are N(0, 0.02^2), in the ``nn.Linear`` layout [out, in]
    (Qwen3 page, Qwen3Attention and SwiGLU classes),
  * every RMSNorm gain (input, post-attention, q_norm, k_norm, final) is
    1 + N(0, 0.1^2), so that no gain makes a sub-layer vanish (for zero-centred
    norms, which apply 1 + g, the stored g is N(0, 0.1^2)),
  * layer inputs are N(0, 1); a decode-time KV cache holds N(0, 1) keys and values,
  * bf16 workloads round each float32 draw to bf16 (round to nearest even), and
    both sides consume exactly those values.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

# Order of the per-layer tensors; also the ``tensor_id`` of each draw.
TENSOR_NAMES = (
    "input_layernorm", "q_proj", "k_proj", "v_proj", "q_norm", "k_norm",
    "o_proj", "post_attention_layernorm", "gate_proj", "up_proj", "down_proj",
)
GAIN_NAMES = frozenset({"input_layernorm", "q_norm", "k_norm", "post_attention_layernorm"})

INPUT_STREAM = 1000       # SeedSequence key of the layer input x
FINAL_GAIN_STREAM = 999   # key of the final RMSNorm gain of a stack
K_CACHE_STREAM = 2000     # keys already in a decode cache
V_CACHE_STREAM = 2001     # values already in a decode cache


@dataclass(frozen=True)
class LayerConfig:
    """The per-layer subset of a Qwen3 config.json (field names as in config.json)."""
    hidden_size: int
    num_attention_heads: int
    num_key_value_heads: int
    head_dim: int
    intermediate_size: int
    rope_theta: float = 1.0e6
    rms_norm_eps: float = 1.0e-6
    max_position_embeddings: int = 40960
    dtype: str = "bf16"           # "bf16" or "f32": storage type of weights and activations
    # RoPE / RMSNorm variants (the Qwen3 defaults leave all four off)
    rotary_dim: int = 0           # features rotated per head; 0 = all of head_dim (partial RoPE)
    rope_adjacent_pairs: bool = False   # pair (2i, 2i+1) instead of (i, i + rotary_dim/2)
    rope_position_scale: float = 1.0    # linear RoPE scaling: angles use position * scale
    norm_unit_offset: bool = False      # zero-centred RMSNorm gains: (1 + g)


@dataclass(frozen=True)
class Workload:
    name: str
    cfg: LayerConfig
    batch: int
    seq_len: int                  # new tokens per sequence (1 for decode)
    layers: int = 1
    cached: int = 0               # keys already in the cache (decode)
    final_norm: bool = False
    seed: int = 0


QWEN3_0P6B = LayerConfig(hidden_size=1024, num_attention_heads=16, num_key_value_heads=8,
                         head_dim=128, intermediate_size=3072)
QWEN3_8B = LayerConfig(hidden_size=4096, num_attention_heads=32, num_key_value_heads=8,
                       head_dim=128, intermediate_size=12288)
TINY_F32 = LayerConfig(hidden_size=64, num_attention_heads=4, num_key_value_heads=2,
                       head_dim=32, intermediate_size=192, dtype="f32")

WORKLOADS = {
    "tiny-f32-layer": Workload("tiny-f32-layer", TINY_F32, batch=1, seq_len=16),
    "qwen3-0.6b-layer-prefill": Workload("qwen3-0.6b-layer-prefill", QWEN3_0P6B, batch=1, seq_len=2048),
    "qwen3-0.6b-stack28-prefill": Workload("qwen3-0.6b-stack28-prefill", QWEN3_0P6B, batch=4,
                                           seq_len=4096, layers=28, final_norm=True),
    "qwen3-8b-layer-prefill": Workload("qwen3-8b-layer-prefill", QWEN3_8B, batch=1, seq_len=8192),
    "qwen3-8b-layer-decode-32k": Workload("qwen3-8b-layer-decode-32k", QWEN3_8B, batch=16,
                                          seq_len=1, cached=32768),
}


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32.  Finite inputs."""
    u = np.array(a, dtype=np.float32, copy=True).view(np.uint32)
    lsb = u >> 16
    lsb &= 1
    u += lsb
    u += 0x7FFF
    u &= 0xFFFF0000
    return u.view(np.float32)


def _rng(seed: int, *keys: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *keys])))


def _finish(a: np.ndarray, dtype: str) -> np.ndarray:
    a = a.astype(np.float32, copy=False)
    return round_to_bf16(a) if dtype == "bf16" else a


def weight_shapes(cfg: LayerConfig) -> dict:
    h, d, hq, hkv, i = (cfg.hidden_size, cfg.head_dim, cfg.num_attention_heads,
                        cfg.num_key_value_heads, cfg.intermediate_size)
    return {
        "input_layernorm": (h,), "q_proj": (hq * d, h), "k_proj": (hkv * d, h),
        "v_proj": (hkv * d, h), "q_norm": (d,), "k_norm": (d,), "o_proj": (h, hq * d),
        "post_attention_layernorm": (h,), "gate_proj": (i, h), "up_proj": (i, h),
        "down_proj": (h, i),
    }


def layer_weights(cfg: LayerConfig, layer: int = 0, seed: int = 0,
                  weight_std: float = 0.02, gain_std: float = 0.1) -> dict:
    """All tensors of one layer as float32 arrays holding exactly representable values."""
    out = {}
    for tid, (name, shape) in enumerate(weight_shapes(cfg).items()):
        g = _rng(seed, layer, tid)
        z = g.standard_normal(shape, dtype=np.float32)
        centre = 0.0 if cfg.norm_unit_offset else 1.0      # zero-centred gains are stored as g
        a = centre + gain_std * z if name in GAIN_NAMES else weight_std * z
        out[name] = _finish(a, cfg.dtype)
    return out


def final_norm_gain(cfg: LayerConfig, seed: int = 0, gain_std: float = 0.1) -> np.ndarray:
    z = _rng(seed, FINAL_GAIN_STREAM).standard_normal((cfg.hidden_size,), dtype=np.float32)
    return _finish(1.0 + gain_std * z, cfg.dtype)


def layer_input(cfg: LayerConfig, batch: int, seq_len: int, seed: int = 0,
                stream: int = INPUT_STREAM) -> np.ndarray:
    z = _rng(seed, stream).standard_normal((batch, seq_len, cfg.hidden_size), dtype=np.float32)
    return _finish(z, cfg.dtype)


def cache_block(cfg: LayerConfig, which: str, b: int, kv_head: int, n: int,
                seed: int = 0) -> np.ndarray:
    """Keys (which='k') or values ('v') already held in a decode cache for
    sequence b, KV head kv_head, positions 0..n-1: [n, head_dim], N(0, 1)."""
    stream = K_CACHE_STREAM if which == "k" else V_CACHE_STREAM
    z = _rng(seed, stream, b, kv_head).standard_normal((n, cfg.head_dim), dtype=np.float32)
    return _finish(z, cfg.dtype)


def with_dtype(cfg: LayerConfig, dtype: str) -> LayerConfig:
    return replace(cfg, dtype=dtype)


def fill_decode_cache(cfg: LayerConfig, batch: int, cached, sink, seed: int = 0, threads: int = 8) -> None:
    """Draw the cached keys and values of every (sequence, KV head) in parallel and hand
    each block to ``sink(b, kv_head, k_block, v_block)`` ([n, head_dim] arrays).
    ``cached`` is one length for all sequences or a list of per-sequence lengths."""
    import concurrent.futures

    lens = [cached] * batch if np.isscalar(cached) else list(cached)

    def one(item):
        b, h = item
        n = int(lens[b])
        sink(b, h, cache_block(cfg, "k", b, h, n, seed), cache_block(cfg, "v", b, h, n, seed))

    items = [(b, h) for b in range(batch) for h in range(cfg.num_key_value_heads)]
    with concurrent.futures.ThreadPoolExecutor(max(1, threads)) as pool:
        for _ in pool.map(one, items):
            pass
