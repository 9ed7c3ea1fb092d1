"""Float64 CPU oracle for the Qwen3-style pre-norm decoder layer (prefill and decode).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares no
code with the HIP path (it imports nothing from the package, and the package
imports nothing from here).

Every function is the plain mathematical definition the pages give, in numpy
float64, applied to the exact stored values of inputs and weights, with no
intermediate rounding (the pages' bf16/fp32 cast points are deliberately not
reproduced: the GPU path is judged against the exact result).  Sources:

  [Q17]  "17. A modern architecture: Qwen3" (inference.shantanugoel.com), sections
         RMSNorm, Rotary position embeddings, Attention with grouped KV heads and
         Q/K normalization, SwiGLU, The whole model.
  [L6]   "Transformer architectures: from BERT to diffusion, lesson 6"
         (xmarva.github.io), sections 3 Grouped-query attention, 4 Training
         stability (QK-norm formula), 5 Qwen3 in PyTorch, 7 (sliding-window
         attention, rolling buffer, attention sinks), 8 (prefix caching;
         batched generation of left-padded prompts).
  [CHK]  "Understand modern AI from the inside out" (Qwen3 layer checklist page),
         items on pre-norm order, q_norm/k_norm placement, rotate-half, scaling,
         GQA, causality, SwiGLU and the float32 RMSNorm.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rmsnorm", "rope_inv_freq", "rope_rotate", "silu", "swiglu_mlp",
    "gqa_causal_attention", "qk_norm_rope", "layer_prefill", "layer_prefill_rows",
    "layer_decode", "layer_prefill_cached", "stack_prefill",
    "padded_positions", "masked_attention", "layer_prefill_padded", "layer_decode_padded",
    "window_mask", "layer_prefill_window", "RollingCache", "layer_decode_rolling", "layer_decode_window",
    "rope_rotate_pairs",
]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------- primitives

def rmsnorm(x, gain, eps):
    """[Q17 RMSNorm]: gain_i * x_i / sqrt(mean_j x_j^2 + eps) over the last axis.

    No mean subtraction, no bias, eps inside the square root ([CHK] float32 RMSNorm
    item; [L6 section 5] RMSNorm class)."""
    x = _f64(x)
    mean_square = np.mean(x * x, axis=-1, keepdims=True)
    return _f64(gain) * (x / np.sqrt(mean_square + eps))


def rope_inv_freq(rotary_dim, theta):
    """[Q17 Rotary position embeddings]: omega_i = theta^(-2i/d), i = 0 .. d/2-1."""
    if rotary_dim % 2:
        raise ValueError("RoPE needs an even number of rotated dimensions")
    i = np.arange(rotary_dim // 2, dtype=np.float64)
    return float(theta) ** (-2.0 * i / rotary_dim)


def rope_rotate(a, positions, omega):
    """Rotate-half RoPE [Q17 Rotary position embeddings; CHK rotate-half item].

    Feature i is paired with feature i + d/2, and the pair (a_i, a_{i+d/2}) of a
    token at position p is turned by the angle p * omega_i:
        out_i       = a_i cos(p w_i) - a_{i+d/2} sin(p w_i)
        out_{i+d/2} = a_{i+d/2} cos(p w_i) + a_i sin(p w_i)
    a: [..., T, d]; positions: [T]; omega: [d/2] (explicit, so d = 2 can be tested)."""
    a = _f64(a)
    half = a.shape[-1] // 2
    angle = _f64(positions)[:, None] * _f64(omega)[None, :]        # [T, d/2]
    c, s = np.cos(angle), np.sin(angle)
    a1, a2 = a[..., :half], a[..., half:]
    return np.concatenate([a1 * c - a2 * s, a2 * c + a1 * s], axis=-1)


def rope_rotate_pairs(a, positions, omega, rotary_dim=None, adjacent=False):
    """RoPE with the pairing and extent as parameters [Q17 Rotary position
    embeddings: "The pairing convention is part of the contract"; apply_rope's
    partial rotation].  Only the first rotary_dim features are rotated (the rest
    pass through unchanged); pair i of them is (i, i + rotary_dim/2) (split-half,
    Qwen/Llama) or (2i, 2i+1) (adjacent, the original paper), each turned by
    p * omega_i exactly as in rope_rotate."""
    a = _f64(a)
    r = a.shape[-1] if not rotary_dim else rotary_dim
    rot, rest = a[..., :r], a[..., r:]
    if adjacent:
        angle = _f64(positions)[:, None] * _f64(omega)[None, :]
        c, s = np.cos(angle), np.sin(angle)
        x1, x2 = rot[..., 0::2], rot[..., 1::2]
        out = np.empty_like(rot)
        out[..., 0::2] = x1 * c - x2 * s
        out[..., 1::2] = x2 * c + x1 * s
    else:
        out = rope_rotate(rot, positions, omega)
    return np.concatenate([out, rest], axis=-1)


def silu(z):
    """[Q17 SwiGLU]: SiLU(z) = z * sigmoid(z)."""
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def swiglu_mlp(h, w_gate, w_up, w_down):
    """[Q17 SwiGLU]: down( silu(gate h) * up h ), nn.Linear weights [out, in], no bias."""
    h = _f64(h)
    gate = h @ _f64(w_gate).T
    up = h @ _f64(w_up).T
    return (silu(gate) * up) @ _f64(w_down).T


def gqa_causal_attention(q, k, v, q_pos, k_pos):
    """Scaled causal softmax attention with grouped KV heads.

    [L6 section 3]: query head h reads KV head floor(h / g), g = Hq / Hkv;
    scores q.k / sqrt(d_h); [CHK] attention is causal.  A key is visible to a query
    iff key_position <= query_position (positions, not indices, so the same code
    serves prefill rows, sampled rows and decode).
    q: [Hq, Tq, D]; k, v: [Hkv, Tk, D]; q_pos: [Tq]; k_pos: [Tk] -> [Hq, Tq, D]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    hq, _, d = q.shape
    hkv = k.shape[0]
    if hq % hkv:
        raise ValueError("Query heads must be a multiple of KV heads")
    group = hq // hkv
    visible = _f64(k_pos)[None, :] <= _f64(q_pos)[:, None]           # [Tq, Tk]
    out = np.empty_like(q)
    for h in range(hq):
        kv = h // group
        scores = (q[h] @ k[kv].T) / np.sqrt(d)
        scores = np.where(visible, scores, -np.inf)
        scores = scores - scores.max(axis=-1, keepdims=True)
        weights = np.exp(scores)
        weights = weights / weights.sum(axis=-1, keepdims=True)
        out[h] = weights @ v[kv]
    return out


# ----------------------------------------------------------------------------- layer steps

def _dims(cfg):
    return (cfg.hidden_size, cfg.num_attention_heads, cfg.num_key_value_heads, cfg.head_dim)


def _rope_variant(cfg):
    """(rotary_dim, adjacent pairs, position scale) of a config; the Qwen3 defaults are
    (head_dim, False, 1): every feature rotated, split-half pairs, positions as they are.
    [Q17 Rotary position embeddings: partial RoPE rotates only the first rotary_dim
    features, frequencies theta^(-2i/rotary_dim); the pairing convention; exercise 3:
    linear RoPE scaling multiplies the positions by a factor.]"""
    r = getattr(cfg, "rotary_dim", 0) or cfg.head_dim
    return r, bool(getattr(cfg, "rope_adjacent_pairs", False)), float(getattr(cfg, "rope_position_scale", 1.0))


def _gain(cfg, g):
    """[Q17 RMSNorm, parity detail 2]: zero-centred norms (Gemma, Qwen3.5) apply 1 + g."""
    return (1.0 + _f64(g)) if getattr(cfg, "norm_unit_offset", False) else _f64(g)


def qk_norm_rope(h, w, cfg, positions, with_q=True, with_kv=True):
    """Projections, per-head Q/K RMSNorm, then RoPE, for the tokens of one sequence.

    [Q17 Attention with grouped KV heads and Q/K normalization]: q, k, v are
    separate bias-free projections of widths Hq*D, Hkv*D, Hkv*D; q_norm/k_norm are
    RMSNorms over each head's D features with one gain shared by the heads, applied
    after the reshape to heads and before RoPE; V is neither normalised nor
    rotated ([CHK] items).  h: [T, H] -> qhat [Hq, T, D], khat [Hkv, T, D],
    v [Hkv, T, D] (None for a part not asked for)."""
    _, hq, hkv, d = _dims(cfg)
    h = _f64(h)
    t = h.shape[0]
    r, adjacent, pscale = _rope_variant(cfg)
    omega = rope_inv_freq(r, cfg.rope_theta)
    ppos = _f64(positions) * pscale
    qhat = khat = v = None
    if with_q:
        q = (h @ _f64(w["q_proj"]).T).reshape(t, hq, d).transpose(1, 0, 2)
        qhat = rope_rotate_pairs(rmsnorm(q, _gain(cfg, w["q_norm"]), cfg.rms_norm_eps), ppos, omega, r, adjacent)
    if with_kv:
        k = (h @ _f64(w["k_proj"]).T).reshape(t, hkv, d).transpose(1, 0, 2)
        v = (h @ _f64(w["v_proj"]).T).reshape(t, hkv, d).transpose(1, 0, 2)
        khat = rope_rotate_pairs(rmsnorm(k, _gain(cfg, w["k_norm"]), cfg.rms_norm_eps), ppos, omega, r, adjacent)
    return qhat, khat, v


def _layer_sequence(x, w, cfg, rows=None):
    """One sequence x [T, H] through the layer; optionally only output rows `rows`.

    [Q17 The whole model, Qwen3Layer]: x1 = x + attn(input_layernorm(x));
    y = x1 + mlp(post_attention_layernorm(x1))  ([CHK] pre-norm items).
    Keys and values are needed for every token; queries, attention, o_proj and
    the MLP only for the requested rows (all rows when `rows` is None)."""
    _, hq, _, d = _dims(cfg)
    x = _f64(x)
    t = x.shape[0]
    positions = np.arange(t, dtype=np.float64)
    rows = np.arange(t) if rows is None else np.asarray(rows, dtype=np.int64)
    h = rmsnorm(x, _gain(cfg, w["input_layernorm"]), cfg.rms_norm_eps)
    _, khat, v = qk_norm_rope(h, w, cfg, positions, with_q=False)
    qhat, _, _ = qk_norm_rope(h[rows], w, cfg, positions[rows], with_kv=False)
    attn = gqa_causal_attention(qhat, khat, v, positions[rows], positions)   # [Hq, R, D]
    attn_flat = attn.transpose(1, 0, 2).reshape(rows.size, hq * d)
    x1 = x[rows] + attn_flat @ _f64(w["o_proj"]).T
    h2 = rmsnorm(x1, _gain(cfg, w["post_attention_layernorm"]), cfg.rms_norm_eps)
    gate = h2 @ _f64(w["gate_proj"]).T
    up = h2 @ _f64(w["up_proj"]).T
    act = silu(gate) * up
    y = x1 + act @ _f64(w["down_proj"]).T
    return dict(h=h[rows], qhat=qhat, khat=khat, v=v, attn=attn_flat, x1=x1, h2=h2,
                act=act, y=y)


def layer_prefill(x, w, cfg):
    """Prefill of a batch x [B, T, H] at positions 0..T-1 with an empty cache.

    Returns a dict of float64 arrays: y [B,T,H] and the intermediates
    h, qhat [B,Hq,T,D], khat/v [B,Hkv,T,D] (what the cache holds), attn [B,T,Hq*D],
    x1, h2, act."""
    x = _f64(x)
    parts = [_layer_sequence(x[b], w, cfg) for b in range(x.shape[0])]
    return {key: np.stack([p[key] for p in parts]) for key in parts[0]}


def layer_prefill_rows(x, w, cfg, rows):
    """y for selected (b, t) rows of a prefill of x [B, T, H]: the same definition
    as layer_prefill, evaluated only where asked.  rows: list of (b, t)."""
    x = _f64(x)
    out = np.empty((len(rows), x.shape[2]))
    by_seq = {}
    for n, (b, t) in enumerate(rows):
        by_seq.setdefault(int(b), []).append((n, int(t)))
    for b, items in by_seq.items():
        ts = np.array([t for _, t in items])
        res = _layer_sequence(x[b], w, cfg, rows=ts)
        for j, (n, _) in enumerate(items):
            out[n] = res["y"][j]
    return out


def layer_decode(x, w, cfg, k_cache, v_cache, cache_lens):
    """One new token per sequence on top of a cache of already rotated keys.

    [Q17 Rotary position embeddings, last paragraph]: keys are cached after
    rotation and never rotated again; the new token rotates its own q and k at its
    own position.  [Q17 The whole model]: the position is the cache length.
    The new key/value go to slot cache_lens[b] and the token attends keys
    0..cache_lens[b] of its own sequence.
    x: [B, 1, H]; k_cache, v_cache: per sequence [Hkv, >= len, D] arrays (or a
    [B, Hkv, cap, D] array); cache_lens: [B] ints.  Returns y [B,1,H], khat_new
    [B,Hkv,D], v_new [B,Hkv,D]."""
    hsize, hq, hkv, d = _dims(cfg)
    x = _f64(x)
    bsz = x.shape[0]
    y = np.empty_like(x)
    khat_new = np.empty((bsz, hkv, d))
    v_new = np.empty((bsz, hkv, d))
    for b in range(bsz):
        p = int(cache_lens[b])
        pos = np.array([float(p)])
        h = rmsnorm(x[b], _gain(cfg, w["input_layernorm"]), cfg.rms_norm_eps)          # [1, H]
        qhat, khat, v = qk_norm_rope(h, w, cfg, pos)                         # [*, 1, D]
        keys = np.concatenate([_f64(k_cache[b])[:, :p], khat], axis=1)     # [Hkv, p+1, D]
        vals = np.concatenate([_f64(v_cache[b])[:, :p], v], axis=1)
        attn = gqa_causal_attention(qhat, keys, vals, pos, np.arange(p + 1, dtype=np.float64))
        x1 = x[b] + attn.transpose(1, 0, 2).reshape(1, hq * d) @ _f64(w["o_proj"]).T
        h2 = rmsnorm(x1, _gain(cfg, w["post_attention_layernorm"]), cfg.rms_norm_eps)
        y[b] = x1 + swiglu_mlp(h2, w["gate_proj"], w["up_proj"], w["down_proj"])
        khat_new[b], v_new[b] = khat[:, 0], v[:, 0]
    return y, khat_new, v_new


def layer_prefill_cached(x, w, cfg, k_cache, v_cache, starts):
    """Prefill of T new tokens per sequence on top of a cache of rotated keys.

    [Q17 The whole model, Qwen3.forward]: without explicit positions the new
    tokens sit at positions start .. start+T-1, start being the cache length.
    [Q17 Rotary position embeddings, last paragraph]: cached keys are already
    rotated and are used as they are; the new tokens rotate their own q and k.
    [L6 section 8, prefix caching]: a shared prefix's keys and values are
    computed once and every continuation starts from them.
    Token t of sequence b (position p = starts[b] + t) attends the cached keys
    0..starts[b]-1 and the new keys at positions <= p (causal rule).
    x: [B, T, H]; k_cache, v_cache: per sequence [Hkv, >= start, D] arrays (or a
    [B, Hkv, cap, D] array); starts: [B] ints.  Returns y [B,T,H], khat_new
    [B,Hkv,T,D] and v_new [B,Hkv,T,D] (what goes to slots start..start+T-1)."""
    hsize, hq, hkv, d = _dims(cfg)
    x = _f64(x)
    bsz, t = x.shape[0], x.shape[1]
    y = np.empty_like(x)
    khat_new = np.empty((bsz, hkv, t, d))
    v_new = np.empty((bsz, hkv, t, d))
    for b in range(bsz):
        p0 = int(starts[b])
        pos = np.arange(p0, p0 + t, dtype=np.float64)
        h = rmsnorm(x[b], _gain(cfg, w["input_layernorm"]), cfg.rms_norm_eps)          # [T, H]
        qhat, khat, v = qk_norm_rope(h, w, cfg, pos)                         # [*, T, D]
        keys = np.concatenate([_f64(k_cache[b])[:, :p0], khat], axis=1)    # [Hkv, p0+T, D]
        vals = np.concatenate([_f64(v_cache[b])[:, :p0], v], axis=1)
        attn = gqa_causal_attention(qhat, keys, vals, pos, np.arange(p0 + t, dtype=np.float64))
        x1 = x[b] + attn.transpose(1, 0, 2).reshape(t, hq * d) @ _f64(w["o_proj"]).T
        h2 = rmsnorm(x1, _gain(cfg, w["post_attention_layernorm"]), cfg.rms_norm_eps)
        y[b] = x1 + swiglu_mlp(h2, w["gate_proj"], w["up_proj"], w["down_proj"])
        khat_new[b], v_new[b] = khat, v
    return y, khat_new, v_new


def stack_prefill(x, layer_weights, final_gain, cfg, round_between=None):
    """[Q17 The whole model, Qwen3.forward]: the layers in order, then the final
    RMSNorm (model.norm) after the last one.  round_between, if given, maps each
    layer's output to the storage type between layers (the layer I/O dtype)."""
    h = _f64(x)
    for w in layer_weights:
        h = layer_prefill(h, w, cfg)["y"]
        if round_between is not None:
            h = _f64(round_between(h))
    return rmsnorm(h, _gain(cfg, final_gain), cfg.rms_norm_eps)


# ----------------------------------------------------------------------------- left padding

def padded_positions(real):
    """[L6 section 8, batched generation]: positions are counted from each row's
    first real token: position = (number of real tokens up to and including this
    column) - 1, clamped at 0 (so padding columns before any real token sit at 0).
    real: [..., S] booleans -> int positions of the same shape."""
    real = np.asarray(real, dtype=bool)
    return np.maximum(np.cumsum(real, axis=-1) - 1, 0)


def masked_attention(q, k, v, visible):
    """Scaled softmax attention over an explicit visibility matrix, grouped KV heads
    as in gqa_causal_attention ([L6 section 3]).  visible: [Tq, Tk] booleans (every
    row must see at least one key).  q: [Hq, Tq, D]; k, v: [Hkv, Tk, D]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    hq, _, d = q.shape
    group = hq // k.shape[0]
    out = np.empty_like(q)
    for h in range(hq):
        kv = h // group
        scores = np.where(visible, (q[h] @ k[kv].T) / np.sqrt(d), -np.inf)
        scores = scores - scores.max(axis=-1, keepdims=True)
        weights = np.exp(scores)
        weights = weights / weights.sum(axis=-1, keepdims=True)
        out[h] = weights @ v[kv]
    return out


def _padded_real(start, pad, length):
    """Slots 0..length-1 of one sequence: real except the padding run [start, start+pad)."""
    slots = np.arange(length)
    return ~((slots >= start) & (slots < start + pad))


def layer_prefill_padded(x, w, cfg, k_cache, v_cache, starts, pads):
    """Prefill of rows padded on the left, on top of an optional shared prefix.

    [L6 section 8, batched generation]: prompts of different lengths are padded
    on the left so every row ends in the same column; padding gets no attention;
    positions count from each row's first real token; every token may see itself,
    so a row of pure padding never attends to nothing.  The mask is
    (causal & real_key) | itself.  With a prefix (keys and values of a shared start
    computed once), the prefix columns are real and come first.
    Sequence b holds starts[b] cached (rotated) prefix keys in slots 0..starts[b]-1;
    its T new tokens go to slots starts[b]+t, and the first pads[b] of them are
    padding.  x: [B, T, H]; k_cache, v_cache: per sequence [Hkv, >= start, D]
    (or [B, Hkv, cap, D]).  Returns y [B,T,H], khat_new [B,Hkv,T,D], v_new
    [B,Hkv,T,D] (what goes to slots starts[b]..starts[b]+T-1, padding included)."""
    hsize, hq, hkv, d = _dims(cfg)
    x = _f64(x)
    bsz, t = x.shape[0], x.shape[1]
    y = np.empty_like(x)
    khat_new = np.empty((bsz, hkv, t, d))
    v_new = np.empty((bsz, hkv, t, d))
    for b in range(bsz):
        p0, pad = int(starts[b]), int(pads[b])
        real = _padded_real(p0, pad, p0 + t)                                  # [p0+T] slots
        pos_all = padded_positions(real).astype(np.float64)
        pos = pos_all[p0:]
        h = rmsnorm(x[b], _gain(cfg, w["input_layernorm"]), cfg.rms_norm_eps)
        qhat, khat, v = qk_norm_rope(h, w, cfg, pos)
        keys = np.concatenate([_f64(k_cache[b])[:, :p0], khat], axis=1)
        vals = np.concatenate([_f64(v_cache[b])[:, :p0], v], axis=1)
        qslot = np.arange(p0, p0 + t)[:, None]
        kslot = np.arange(p0 + t)[None, :]
        visible = ((kslot <= qslot) & real[None, :]) | (kslot == qslot)
        attn = masked_attention(qhat, keys, vals, visible)
        x1 = x[b] + attn.transpose(1, 0, 2).reshape(t, hq * d) @ _f64(w["o_proj"]).T
        h2 = rmsnorm(x1, _gain(cfg, w["post_attention_layernorm"]), cfg.rms_norm_eps)
        y[b] = x1 + swiglu_mlp(h2, w["gate_proj"], w["up_proj"], w["down_proj"])
        khat_new[b], v_new[b] = khat, v
    return y, khat_new, v_new


def layer_decode_padded(x, w, cfg, k_cache, v_cache, cache_lens, pad_starts, pad_lens):
    """One new token per sequence after a padded prefill ([L6 section 8, batched
    generation]: each step appends a real column, the mask stays the row's real
    columns, and the position advances by one from the last prompt position).
    The new token of sequence b goes to slot cache_lens[b], sits at position
    (real slots before it) = cache_lens[b] - pad_lens[b], and attends the real
    cached keys (slots outside [pad_starts[b], pad_starts[b] + pad_lens[b])) and
    itself.  Returns y [B,1,H], khat_new [B,Hkv,D], v_new [B,Hkv,D]."""
    hsize, hq, hkv, d = _dims(cfg)
    x = _f64(x)
    bsz = x.shape[0]
    y = np.empty_like(x)
    khat_new = np.empty((bsz, hkv, d))
    v_new = np.empty((bsz, hkv, d))
    for b in range(bsz):
        n = int(cache_lens[b])
        real = np.append(_padded_real(int(pad_starts[b]), int(pad_lens[b]), n), True)   # [n+1]
        pos = np.array([float(padded_positions(real)[-1])])
        h = rmsnorm(x[b], _gain(cfg, w["input_layernorm"]), cfg.rms_norm_eps)
        qhat, khat, v = qk_norm_rope(h, w, cfg, pos)
        keys = np.concatenate([_f64(k_cache[b])[:, :n], khat], axis=1)
        vals = np.concatenate([_f64(v_cache[b])[:, :n], v], axis=1)
        attn = masked_attention(qhat, keys, vals, real[None, :])
        x1 = x[b] + attn.transpose(1, 0, 2).reshape(1, hq * d) @ _f64(w["o_proj"]).T
        h2 = rmsnorm(x1, _gain(cfg, w["post_attention_layernorm"]), cfg.rms_norm_eps)
        y[b] = x1 + swiglu_mlp(h2, w["gate_proj"], w["up_proj"], w["down_proj"])
        khat_new[b], v_new[b] = khat[:, 0], v[:, 0]
    return y, khat_new, v_new


# ----------------------------------------------------------------------------- local attention

def window_mask(q_pos, k_pos, window, sinks=0):
    """[L6 section 7]: in a local layer token i sees token j iff i - W < j <= i
    (itself included); with attention sinks the first `sinks` tokens stay visible
    to every later token (mask | (causal & j < sinks)).  window = 0 means global
    (plain causal).  q_pos: [Tq], k_pos: [Tk] -> [Tq, Tk] booleans."""
    qp = np.asarray(q_pos)[:, None]
    kp = np.asarray(k_pos)[None, :]
    causal = kp <= qp
    if window <= 0:
        return causal
    return (causal & (qp - kp < window)) | (causal & (kp < sinks))


def layer_prefill_window(x, w, cfg, window, sinks=0):
    """Prefill at positions 0..T-1 with the banded mask of window_mask (the page's
    "full causal cache and a banded mask").  x: [B, T, H] -> y [B, T, H],
    khat [B, Hkv, T, D], v [B, Hkv, T, D] (the whole causal cache)."""
    hsize, hq, hkv, d = _dims(cfg)
    x = _f64(x)
    bsz, t = x.shape[0], x.shape[1]
    pos = np.arange(t, dtype=np.float64)
    vis = window_mask(np.arange(t), np.arange(t), window, sinks)
    y = np.empty_like(x)
    khat_all = np.empty((bsz, hkv, t, d))
    v_all = np.empty((bsz, hkv, t, d))
    for b in range(bsz):
        h = rmsnorm(x[b], _gain(cfg, w["input_layernorm"]), cfg.rms_norm_eps)
        qhat, khat, v = qk_norm_rope(h, w, cfg, pos)
        attn = masked_attention(qhat, khat, v, vis)
        x1 = x[b] + attn.transpose(1, 0, 2).reshape(t, hq * d) @ _f64(w["o_proj"]).T
        h2 = rmsnorm(x1, _gain(cfg, w["post_attention_layernorm"]), cfg.rms_norm_eps)
        y[b] = x1 + swiglu_mlp(h2, w["gate_proj"], w["up_proj"], w["down_proj"])
        khat_all[b], v_all[b] = khat, v
    return y, khat_all, v_all


class RollingCache:
    """[L6 section 7]: a rolling buffer of a local layer keeps at most W keys and
    values and writes token i over the token that has just left the window (slot
    i mod W); order does not matter, since each key carries its position in its
    rotation.  With sinks, the first `sinks` tokens keep slots 0..sinks-1 and the
    ring of W slots after them holds the other tokens (token i >= sinks goes to
    slot sinks + (i - sinks) mod W), so the buffer always holds exactly the keys
    window_mask lets the newest token see.  Per sequence: k, v [Hkv, sinks + W, D]."""

    def __init__(self, hkv, d, window, sinks=0):
        self.window, self.sinks = window, sinks
        self.k = np.zeros((hkv, sinks + window, d))
        self.v = np.zeros((hkv, sinks + window, d))
        self.seen = 0

    def slot(self, i):
        return i if i < self.sinks else self.sinks + (i - self.sinks) % self.window

    def add(self, k, v):
        s = self.slot(self.seen)
        self.k[:, s], self.v[:, s] = k, v
        self.seen += 1
        return min(self.seen, self.sinks + self.window)          # slots holding tokens


def layer_decode_rolling(x, w, cfg, caches):
    """One decode step per sequence on its RollingCache (the page's token-by-token
    run "with a rolling buffer ... and no mask at all"): the new token sits at
    position caches[b].seen, its key/value enter the buffer first, then it attends
    every filled slot.  x: [B, 1, H]; caches: list of RollingCache (updated).
    Returns y [B, 1, H]."""
    hsize, hq, hkv, d = _dims(cfg)
    x = _f64(x)
    y = np.empty_like(x)
    for b, cache in enumerate(caches):
        pos = np.array([float(cache.seen)])
        h = rmsnorm(x[b], _gain(cfg, w["input_layernorm"]), cfg.rms_norm_eps)
        qhat, khat, v = qk_norm_rope(h, w, cfg, pos)
        n = cache.add(khat[:, 0], v[:, 0])
        attn = masked_attention(qhat, cache.k[:, :n], cache.v[:, :n], np.ones((1, n), dtype=bool))
        x1 = x[b] + attn.transpose(1, 0, 2).reshape(1, hq * d) @ _f64(w["o_proj"]).T
        h2 = rmsnorm(x1, _gain(cfg, w["post_attention_layernorm"]), cfg.rms_norm_eps)
        y[b] = x1 + swiglu_mlp(h2, w["gate_proj"], w["up_proj"], w["down_proj"])
    return y


def layer_decode_window(x, w, cfg, k_cache, v_cache, cache_lens, window, sinks=0):
    """One decode step per sequence on a full (linear) cache under the window mask:
    the new token at position cache_lens[b] (slot cache_lens[b]) attends the cached
    keys window_mask allows and itself.  Returns y [B,1,H], khat_new, v_new [B,Hkv,D]."""
    hsize, hq, hkv, d = _dims(cfg)
    x = _f64(x)
    bsz = x.shape[0]
    y = np.empty_like(x)
    khat_new = np.empty((bsz, hkv, d))
    v_new = np.empty((bsz, hkv, d))
    for b in range(bsz):
        p = int(cache_lens[b])
        pos = np.array([float(p)])
        h = rmsnorm(x[b], _gain(cfg, w["input_layernorm"]), cfg.rms_norm_eps)
        qhat, khat, v = qk_norm_rope(h, w, cfg, pos)
        keys = np.concatenate([_f64(k_cache[b])[:, :p], khat], axis=1)
        vals = np.concatenate([_f64(v_cache[b])[:, :p], v], axis=1)
        vis = window_mask([p], np.arange(p + 1), window, sinks)
        attn = masked_attention(qhat, keys, vals, vis)
        x1 = x[b] + attn.transpose(1, 0, 2).reshape(1, hq * d) @ _f64(w["o_proj"]).T
        h2 = rmsnorm(x1, _gain(cfg, w["post_attention_layernorm"]), cfg.rms_norm_eps)
        y[b] = x1 + swiglu_mlp(h2, w["gate_proj"], w["up_proj"], w["down_proj"])
        khat_new[b], v_new[b] = khat[:, 0], v[:, 0]
    return y, khat_new, v_new
