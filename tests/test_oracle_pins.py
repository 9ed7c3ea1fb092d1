"""Pins of the float64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a value the
pages print (fixtures under tests/golden/, each citing its page and section), a
closed form, an invariant, or a special case that reduces to a library routine.
Together they are chosen so that a plausible slip in the oracle (a dropped term,
a sign, an index, a transposed operand, a wrong pairing or head mapping) fails
at least one of them.  All CPU-only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import seeded_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def half_unit(decimals):
    return 0.5 * 10.0 ** (-decimals) + 1e-12


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_worked_example():
    g = golden("rmsnorm_worked_example.json")
    x = np.array(g["x"])
    out = oracle.rmsnorm(x, np.ones(2), 1e-6)
    np.testing.assert_allclose(out, g["output"], atol=half_unit(g["printed_decimals"]))
    assert np.mean(x * x) == g["mean_square"]
    assert abs(math.sqrt(np.mean(x * x)) - g["rms"]) < half_unit(4)
    # the normalised vector keeps its direction and has RMS 1
    assert abs(math.sqrt(np.mean(out * out)) - 1.0) < 1e-6
    assert abs(out[0] / out[1] - 0.75) < 1e-12


def test_rmsnorm_eps_inside_root_closed_form():
    # a constant vector c*1 normalises to c / sqrt(c^2 + eps): eps inside the root
    for c, eps in [(1e-3, 1e-6), (2.0, 1e-6), (1e-4, 1e-6)]:
        out = oracle.rmsnorm(np.full(8, c), np.ones(8), eps)
        np.testing.assert_allclose(out, c / math.sqrt(c * c + eps), rtol=1e-14)
    # with c = 1e-3 the eps term matters: eps outside the root would give ~0.999
    assert abs(oracle.rmsnorm(np.full(4, 1e-3), np.ones(4), 1e-6)[0] - 1 / math.sqrt(2)) < 1e-12


def test_rmsnorm_matches_torch_library_routine():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 5, 96))
    gain = 1 + 0.1 * rng.standard_normal(96)
    ref = F.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(gain), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rmsnorm(x, gain, 1e-6), ref, rtol=1e-13, atol=1e-14)


def test_rmsnorm_reduces_over_last_axis_only():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 32))
    x[1] *= 100.0                     # one row much larger: other rows must not change
    out = oracle.rmsnorm(x, np.ones(32), 1e-6)
    np.testing.assert_allclose(np.sqrt(np.mean(out ** 2, axis=-1)), 1.0, rtol=1e-6)


# ---------------------------------------------------------------- RoPE

def test_rope_relativity_worked_example():
    g = golden("rope_relativity.json")
    q, k = np.array(g["q"])[None, :], np.array(g["k"])[None, :]
    omega = np.array([g["omega"]])
    for p, s in g["position_pairs"]:
        rq = oracle.rope_rotate(q, np.array([p]), omega)
        rk = oracle.rope_rotate(k, np.array([s]), omega)
        score = float(rq[0] @ rk[0])
        assert abs(score - g["score"]) < half_unit(g["printed_decimals"])
        assert abs(score - math.cos(0.7)) < 1e-14


def test_rope_frequency_range():
    g = golden("rope_frequency_range.json")
    omega = oracle.rope_inv_freq(g["head_dim"], g["theta"])
    assert omega.shape == (g["head_dim"] // 2,)
    assert omega[0] == g["fastest_rad_per_token"]
    assert abs(omega[-1] - g["slowest_rad_per_token_about"]) < 0.05e-6      # "about 1.2e-6"
    wavelength = 2 * math.pi / omega[-1]
    assert abs(wavelength / g["slowest_wavelength_tokens_about"] - 1) < 0.05  # "about 5 million"
    assert np.all(np.diff(omega) < 0)


def test_rope_pairs_are_page_rotation_matrix():
    # Each pair (a_i, a_{i+d/2}) is multiplied by R(phi) = [[cos, -sin], [sin, cos]]
    # with phi = p * omega_i (textbook 2-D rotation; split-half pairing).
    rng = np.random.default_rng(3)
    d = 16
    a = rng.standard_normal((5, d))
    pos = np.array([0, 1, 7, 100, 32768])
    omega = oracle.rope_inv_freq(d, 1e6)
    out = oracle.rope_rotate(a, pos, omega)
    for t in range(5):
        for i in range(d // 2):
            phi = pos[t] * omega[i]
            r = np.array([[math.cos(phi), -math.sin(phi)], [math.sin(phi), math.cos(phi)]])
            want = r @ np.array([a[t, i], a[t, i + d // 2]])
            np.testing.assert_allclose([out[t, i], out[t, i + d // 2]], want, atol=1e-12)


def test_rope_is_complex_multiplication():
    # Split-half RoPE is z_i * exp(j p w_i) with z_i = a_i + j a_{i+d/2}.
    rng = np.random.default_rng(4)
    d = 128
    a = rng.standard_normal((3, 7, d))
    pos = np.arange(7) * 1000 + 5
    omega = oracle.rope_inv_freq(d, 1e6)
    z = a[..., : d // 2] + 1j * a[..., d // 2:]
    zr = z * np.exp(1j * pos[:, None] * omega[None, :])
    out = oracle.rope_rotate(a, pos, omega)
    np.testing.assert_allclose(out, np.concatenate([zr.real, zr.imag], axis=-1), atol=1e-12)


def test_rope_invariants():
    rng = np.random.default_rng(5)
    d = 64
    omega = oracle.rope_inv_freq(d, 1e6)
    q, k = rng.standard_normal((1, d)), rng.standard_normal((1, d))
    # norm preservation
    for p in [0, 3, 9999]:
        r = oracle.rope_rotate(q, np.array([p]), omega)
        assert abs(np.linalg.norm(r) - np.linalg.norm(q)) < 1e-12
    # distance 0 score equals the unrotated dot product
    for p in [0, 17, 4096]:
        rq = oracle.rope_rotate(q, np.array([p]), omega)
        rk = oracle.rope_rotate(k, np.array([p]), omega)
        assert abs(float(rq[0] @ rk[0]) - float(q[0] @ k[0])) < 1e-12
    # a shared shift of 10 leaves the score unchanged
    s1 = oracle.rope_rotate(q, np.array([3]), omega)[0] @ oracle.rope_rotate(k, np.array([8]), omega)[0]
    s2 = oracle.rope_rotate(q, np.array([13]), omega)[0] @ oracle.rope_rotate(k, np.array([18]), omega)[0]
    assert abs(s1 - s2) < 1e-12


# ---------------------------------------------------------------- SiLU / SwiGLU

def test_silu_values_and_swiglu():
    g = golden("silu_values.json")
    for z, want in g["silu"]:
        assert abs(float(oracle.silu(z)) - want) < half_unit(g["printed_decimals"])
    # an MLP whose gate pre-activation is 2 and up value is 3, down = identity
    h = np.array([[1.0, 0.0]])
    wg = np.array([[2.0, 0.0]])
    wu = np.array([[3.0, 0.0]])
    wd = np.array([[1.0], [0.0]])
    out = oracle.swiglu_mlp(h, wg, wu, wd)
    assert abs(out[0, 0] - g["passed"]) < half_unit(g["printed_decimals"])
    assert out[0, 1] == 0.0
    rng = np.random.default_rng(6)
    z = rng.standard_normal(50) * 4
    np.testing.assert_allclose(oracle.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-14)


# ---------------------------------------------------------------- attention

def test_gqa_matches_torch_sdpa_page_shapes():
    g = golden("gqa_vs_sdpa.json")
    rng = np.random.default_rng(7)
    q = rng.standard_normal(g["q_shape"])
    k = rng.standard_normal(g["kv_shape"])
    v = rng.standard_normal(g["kv_shape"])
    t = g["q_shape"][2]
    pos = np.arange(t)
    ours = oracle.gqa_causal_attention(q[0], k[0], v[0], pos, pos)
    mask = torch.ones(t, t, dtype=torch.bool).tril()
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                         attn_mask=mask, enable_gqa=True)[0].numpy()
    assert np.abs(ours - ref).max() < 1e-12


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (6, 3), (8, 1)])
def test_gqa_mapping_against_library(hq, hkv):
    rng = np.random.default_rng(8 + hq + hkv)
    t, d = 9, 8
    q = rng.standard_normal((hq, t, d))
    k = rng.standard_normal((hkv, t, d))
    v = rng.standard_normal((hkv, t, d))
    pos = np.arange(t)
    ours = oracle.gqa_causal_attention(q, k, v, pos, pos)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None], torch.from_numpy(k)[None],
                                         torch.from_numpy(v)[None], is_causal=True,
                                         enable_gqa=True)[0].numpy()
    assert np.abs(ours - ref).max() < 1e-12
    if hq == hkv:   # groups = 1 is plain multi-head attention, head by head
        for h in range(hq):
            one = oracle.gqa_causal_attention(q[h:h + 1], k[h:h + 1], v[h:h + 1], pos, pos)
            np.testing.assert_allclose(ours[h], one[0], atol=1e-15)


def test_attention_closed_forms():
    rng = np.random.default_rng(9)
    hq, hkv, t, d = 4, 2, 6, 8
    k = rng.standard_normal((hkv, t, d))
    v = rng.standard_normal((hkv, t, d))
    pos = np.arange(t)
    # query 0 sees only key 0: its output is exactly v_0 of its KV head (h // 2)
    q = rng.standard_normal((hq, t, d))
    out = oracle.gqa_causal_attention(q, k, v, pos, pos)
    for h in range(hq):
        np.testing.assert_allclose(out[h, 0], v[h // 2, 0], atol=1e-15)
    # all-zero queries: equal scores, so each output is the causal running mean
    out0 = oracle.gqa_causal_attention(np.zeros((hq, t, d)), k, v, pos, pos)
    for h in range(hq):
        running = np.cumsum(v[h // 2], axis=0) / np.arange(1, t + 1)[:, None]
        np.testing.assert_allclose(out0[h], running, atol=1e-14)


# ---------------------------------------------------------------- the layer

def tiny_cfg(**kw):
    return si.LayerConfig(**{**dict(hidden_size=64, num_attention_heads=4, num_key_value_heads=2,
                                    head_dim=32, intermediate_size=192, dtype="f32"), **kw})


def test_qk_norm_is_per_head_before_rope():
    # the identity |qhat| = sqrt(D) before the gain is exact for eps = 0
    cfg = tiny_cfg(rms_norm_eps=0.0)
    w = si.layer_weights(cfg, seed=11)
    w["q_norm"] = np.ones(32, np.float32)
    w["k_norm"] = np.ones(32, np.float32)
    h = si.layer_input(cfg, 1, 5, seed=11)[0]
    qhat, khat, v = oracle.qk_norm_rope(h, w, cfg, np.arange(5))
    # with unit gain every head vector has norm sqrt(D) (rotation keeps the norm)
    np.testing.assert_allclose(np.linalg.norm(qhat, axis=-1), math.sqrt(32), rtol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(khat, axis=-1), math.sqrt(32), rtol=1e-12)
    # V is the plain projection: neither normalised nor rotated
    np.testing.assert_allclose(v, (h.astype(np.float64) @ w["v_proj"].T.astype(np.float64))
                               .reshape(5, 2, 32).transpose(1, 0, 2), rtol=1e-14)


def torch_layer_from_library(x, w, cfg):
    """The layer assembled from torch library routines in float64 (F.rms_norm,
    F.linear, F.scaled_dot_product_attention with enable_gqa, F.silu) and the
    complex-exponential form of RoPE, following the class structure of the
    Qwen3 pages.  Independent of the oracle's own primitives."""
    t64 = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    hs, hq, hkv, d = cfg.hidden_size, cfg.num_attention_heads, cfg.num_key_value_heads, cfg.head_dim
    eps = cfg.rms_norm_eps
    X = t64(x)
    b, t, _ = X.shape
    H = F.rms_norm(X, (hs,), t64(w["input_layernorm"]), eps)
    q = F.linear(H, t64(w["q_proj"])).view(b, t, hq, d)
    k = F.linear(H, t64(w["k_proj"])).view(b, t, hkv, d)
    v = F.linear(H, t64(w["v_proj"])).view(b, t, hkv, d).transpose(1, 2)
    q = F.rms_norm(q, (d,), t64(w["q_norm"]), eps).transpose(1, 2)
    k = F.rms_norm(k, (d,), t64(w["k_norm"]), eps).transpose(1, 2)
    inv = torch.tensor([cfg.rope_theta ** (-2.0 * i / d) for i in range(d // 2)], dtype=torch.float64)
    rot = torch.polar(torch.ones(t, d // 2, dtype=torch.float64),
                      torch.arange(t, dtype=torch.float64)[:, None] * inv[None, :])

    def rope(a):
        z = torch.complex(a[..., : d // 2], a[..., d // 2:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    o = F.scaled_dot_product_attention(rope(q), rope(k), v, is_causal=True, enable_gqa=True)
    X1 = X + F.linear(o.transpose(1, 2).reshape(b, t, hq * d), t64(w["o_proj"]))
    H2 = F.rms_norm(X1, (hs,), t64(w["post_attention_layernorm"]), eps)
    mlp = F.linear(F.silu(F.linear(H2, t64(w["gate_proj"]))) * F.linear(H2, t64(w["up_proj"])),
                   t64(w["down_proj"]))
    return (X1 + mlp).numpy()


@pytest.mark.parametrize("cfg,b,t", [
    (tiny_cfg(), 1, 16),
    (tiny_cfg(num_attention_heads=4, num_key_value_heads=4), 2, 7),
    (si.LayerConfig(hidden_size=128, num_attention_heads=8, num_key_value_heads=2, head_dim=64,
                    intermediate_size=256, dtype="f32"), 2, 33),
])
def test_layer_matches_library_assembly(cfg, b, t):
    w = si.layer_weights(cfg, seed=12)
    x = si.layer_input(cfg, b, t, seed=12)
    ours = oracle.layer_prefill(x, w, cfg)["y"]
    ref = torch_layer_from_library(x, w, cfg)
    assert np.abs(ours - ref).max() < 1e-11


def test_layer_causality_future_tokens_do_not_matter():
    cfg = tiny_cfg()
    w = si.layer_weights(cfg, seed=13)
    x = si.layer_input(cfg, 1, 12, seed=13)
    y = oracle.layer_prefill(x, w, cfg)["y"]
    for i in [0, 5, 10]:
        x2 = x.copy()
        x2[0, i + 1:] = np.random.default_rng(i).standard_normal(x2[0, i + 1:].shape)
        y2 = oracle.layer_prefill(x2, w, cfg)["y"]
        assert np.array_equal(y[0, : i + 1], y2[0, : i + 1])
        assert not np.allclose(y[0, i + 1:], y2[0, i + 1:])


def test_layer_zero_weights_special_cases():
    cfg = tiny_cfg()
    w = si.layer_weights(cfg, seed=14)
    x = si.layer_input(cfg, 1, 6, seed=14)
    wz = {**w, "o_proj": np.zeros_like(w["o_proj"]), "down_proj": np.zeros_like(w["down_proj"])}
    assert np.array_equal(oracle.layer_prefill(x, wz, cfg)["y"], x.astype(np.float64))
    wd = {**w, "down_proj": np.zeros_like(w["down_proj"])}
    res = oracle.layer_prefill(x, wd, cfg)
    assert np.array_equal(res["y"], res["x1"])
    assert not np.allclose(res["x1"], x)


def test_sampled_rows_equal_full_layer():
    cfg = si.LayerConfig(hidden_size=128, num_attention_heads=8, num_key_value_heads=2, head_dim=64,
                         intermediate_size=256, dtype="bf16")
    w = si.layer_weights(cfg, seed=15)
    x = si.layer_input(cfg, 2, 40, seed=15)
    full = oracle.layer_prefill(x, w, cfg)["y"]
    rows = [(0, 0), (1, 39), (0, 17), (1, 3)]
    part = oracle.layer_prefill_rows(x, w, cfg, rows)
    for n, (b, t) in enumerate(rows):
        np.testing.assert_allclose(part[n], full[b, t], atol=1e-12)


def test_decode_continues_prefill():
    # prefill(T) row T-1 == prefill(T-1) then one decode step at position T-1
    cfg = tiny_cfg()
    w = si.layer_weights(cfg, seed=16)
    x = si.layer_input(cfg, 3, 10, seed=16)
    full = oracle.layer_prefill(x, w, cfg)
    lens = [9, 5, 1]
    cap = 12
    kc = np.zeros((3, 2, cap, 32))
    vc = np.zeros((3, 2, cap, 32))
    for b, n in enumerate(lens):
        pre = oracle.layer_prefill(x[b:b + 1, :n], w, cfg)
        kc[b, :, :n] = pre["khat"][0]
        vc[b, :, :n] = pre["v"][0]
    xin = np.stack([x[b, n] for b, n in enumerate(lens)])[:, None, :]
    y, knew, vnew = oracle.layer_decode(xin, w, cfg, kc, vc, lens)
    for b, n in enumerate(lens):
        np.testing.assert_allclose(y[b, 0], full["y"][b, n], atol=1e-12)
        np.testing.assert_allclose(knew[b], full["khat"][b, :, n], atol=1e-12)
        np.testing.assert_allclose(vnew[b], full["v"][b, :, n], atol=1e-12)


def test_cached_prefill_continues_prefill():
    # prefill(n) then the remaining tokens as a prefill onto that cache == the rows n.. of
    # prefill(n + T) (causal rule + positions continuing from the cache length), ragged n
    cfg = tiny_cfg()
    w = si.layer_weights(cfg, seed=18)
    x = si.layer_input(cfg, 3, 13, seed=18)
    t_new = 5
    starts = [8, 0, 3]
    cap = 16
    kc = np.zeros((3, 2, cap, 32))
    vc = np.zeros((3, 2, cap, 32))
    xin = np.zeros((3, t_new, 64), dtype=x.dtype)
    for b, n in enumerate(starts):
        if n:
            pre = oracle.layer_prefill(x[b:b + 1, :n], w, cfg)
            kc[b, :, :n] = pre["khat"][0]
            vc[b, :, :n] = pre["v"][0]
        xin[b] = x[b, n:n + t_new]
    y, knew, vnew = oracle.layer_prefill_cached(xin, w, cfg, kc, vc, starts)
    for b, n in enumerate(starts):
        full = oracle.layer_prefill(x[b:b + 1, :n + t_new], w, cfg)
        np.testing.assert_allclose(y[b], full["y"][0, n:], atol=1e-12)
        np.testing.assert_allclose(knew[b], full["khat"][0, :, n:], atol=1e-12)
        np.testing.assert_allclose(vnew[b], full["v"][0, :, n:], atol=1e-12)


def test_cached_prefill_matches_library_assembly_on_given_cache():
    # arbitrary cached keys/values (not produced by this layer) are used as they are; the new
    # tokens rotate at positions start.. and see the cache plus their own causal prefix
    cfg = tiny_cfg()
    hs, hq, hkv, d, eps = 64, 4, 2, 32, cfg.rms_norm_eps
    w = si.layer_weights(cfg, seed=19)
    x = si.layer_input(cfg, 1, 6, seed=19)
    p0 = 9
    rng = np.random.default_rng(19)
    kc = rng.standard_normal((1, hkv, 20, d))
    vc = rng.standard_normal((1, hkv, 20, d))
    y, _, _ = oracle.layer_prefill_cached(x, w, cfg, kc, vc, [p0])

    t64 = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    X = t64(x)
    t = X.shape[1]
    H = F.rms_norm(X, (hs,), t64(w["input_layernorm"]), eps)
    q = F.rms_norm(F.linear(H, t64(w["q_proj"])).view(1, t, hq, d), (d,), t64(w["q_norm"]), eps).transpose(1, 2)
    k = F.rms_norm(F.linear(H, t64(w["k_proj"])).view(1, t, hkv, d), (d,), t64(w["k_norm"]), eps).transpose(1, 2)
    v = F.linear(H, t64(w["v_proj"])).view(1, t, hkv, d).transpose(1, 2)
    inv = torch.tensor([cfg.rope_theta ** (-2.0 * i / d) for i in range(d // 2)], dtype=torch.float64)
    pos = torch.arange(p0, p0 + t, dtype=torch.float64)
    rot = torch.polar(torch.ones(t, d // 2, dtype=torch.float64), pos[:, None] * inv[None, :])

    def rope(a):
        z = torch.complex(a[..., : d // 2], a[..., d // 2:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    keys = torch.cat([t64(kc[:, :, :p0]), rope(k)], dim=2)
    vals = torch.cat([t64(vc[:, :, :p0]), v], dim=2)
    mask = torch.arange(p0 + t)[None, :] <= pos.long()[:, None]
    o = F.scaled_dot_product_attention(rope(q), keys, vals, attn_mask=mask, enable_gqa=True)
    X1 = X + F.linear(o.transpose(1, 2).reshape(1, t, hq * d), t64(w["o_proj"]))
    H2 = F.rms_norm(X1, (hs,), t64(w["post_attention_layernorm"]), eps)
    ref = X1 + F.linear(F.silu(F.linear(H2, t64(w["gate_proj"]))) * F.linear(H2, t64(w["up_proj"])),
                        t64(w["down_proj"]))
    assert np.abs(y - ref.numpy()).max() < 1e-11



# ---------------------------------------------------------------- left padding (lesson 6, section 8)

def test_padded_positions_page_rule():
    g = golden("left_padding_positions.json")
    for case in g["cases"]:
        assert oracle.padded_positions(case["real"]).tolist() == case["positions"]


def test_padded_prefill_real_rows_equal_unpadded_prefill():
    # padding gets no attention and positions count from the first real token: the real rows
    # of a left-padded row equal the plain prefill of its real tokens, and their keys/values
    # equal that prefill's cache
    cfg = tiny_cfg()
    w = si.layer_weights(cfg, seed=21)
    t = 11
    pads = [0, 4, 10]
    x = si.layer_input(cfg, 3, t, seed=21)
    kc = np.zeros((3, 2, t, 32))
    y, knew, vnew = oracle.layer_prefill_padded(x, w, cfg, kc, kc, [0, 0, 0], pads)
    for b, pad in enumerate(pads):
        ref = oracle.layer_prefill(x[b:b + 1, pad:], w, cfg)
        np.testing.assert_allclose(y[b, pad:], ref["y"][0], atol=1e-12)
        np.testing.assert_allclose(knew[b, :, pad:], ref["khat"][0], atol=1e-12)
        np.testing.assert_allclose(vnew[b, :, pad:], ref["v"][0], atol=1e-12)


def test_padded_prefill_padding_query_sees_only_itself():
    # every token sees itself, and a padding token (no real token before it) sees nothing
    # else: its attention output is its own value vector, so its row is the layer applied to
    # a one-token sequence at position 0
    cfg = tiny_cfg()
    w = si.layer_weights(cfg, seed=22)
    x = si.layer_input(cfg, 1, 6, seed=22)
    kc = np.zeros((1, 2, 6, 32))
    y, _, _ = oracle.layer_prefill_padded(x, w, cfg, kc, kc, [0], [3])
    for t in range(3):
        ref = oracle.layer_prefill(x[:, t:t + 1], w, cfg)["y"][0, 0]
        np.testing.assert_allclose(y[0, t], ref, atol=1e-12)


def test_padded_prefill_with_prefix_equals_cached_prefill():
    # a shared prefix followed by left-padded rows: the real rows equal a prefill onto the
    # prefix cache of the real tokens alone (positions continue from the prefix length)
    cfg = tiny_cfg()
    w = si.layer_weights(cfg, seed=23)
    p0, t = 5, 8
    prefix = si.layer_input(cfg, 1, p0, seed=23)
    pre = oracle.layer_prefill(prefix, w, cfg)
    kc = np.repeat(pre["khat"], 2, axis=0)
    vc = np.repeat(pre["v"], 2, axis=0)
    x = si.layer_input(cfg, 2, t, seed=24)
    pads = [0, 3]
    y, knew, vnew = oracle.layer_prefill_padded(x, w, cfg, kc, vc, [p0, p0], pads)
    for b, pad in enumerate(pads):
        ref_y, ref_k, ref_v = oracle.layer_prefill_cached(x[b:b + 1, pad:], w, cfg, kc[b:b + 1], vc[b:b + 1], [p0])
        np.testing.assert_allclose(y[b, pad:], ref_y[0], atol=1e-12)
        np.testing.assert_allclose(knew[b, :, pad:], ref_k[0], atol=1e-12)


def test_padded_decode_equals_unpadded_decode():
    # after a left-padded prefill, a decode step attends the real keys and itself at position
    # (real tokens so far): equal to decoding the unpadded sequence
    cfg = tiny_cfg()
    w = si.layer_weights(cfg, seed=25)
    t = 9
    pads = [2, 0, 6]
    x = si.layer_input(cfg, 3, t + 1, seed=25)
    cap = t + 1
    kc = np.zeros((3, 2, cap, 32))
    vc = np.zeros((3, 2, cap, 32))
    _, knew, vnew = oracle.layer_prefill_padded(x[:, :t], w, cfg, kc, vc, [0, 0, 0], pads)
    kc[:, :, :t], vc[:, :, :t] = knew, vnew
    y, kd, vd = oracle.layer_decode_padded(x[:, t:], w, cfg, kc, vc, [t] * 3, [0, 0, 0], pads)
    for b, pad in enumerate(pads):
        real = t - pad
        kr = kc[b:b + 1, :, pad:t]
        vr = vc[b:b + 1, :, pad:t]
        ref, rk, rv = oracle.layer_decode(x[b:b + 1, t:], w, cfg, kr, vr, [real])
        np.testing.assert_allclose(y[b], ref[0], atol=1e-12)
        np.testing.assert_allclose(kd[b], rk[0], atol=1e-12)
        np.testing.assert_allclose(vd[b], rv[0], atol=1e-12)


def test_masked_attention_reduces_to_causal():
    # with the causal mask and no padding, the explicit-mask attention is the causal one
    rng = np.random.default_rng(26)
    q = rng.standard_normal((4, 7, 16))
    k = rng.standard_normal((2, 7, 16))
    v = rng.standard_normal((2, 7, 16))
    pos = np.arange(7)
    causal = pos[None, :] <= pos[:, None]
    np.testing.assert_allclose(oracle.masked_attention(q, k, v, causal),
                               oracle.gqa_causal_attention(q, k, v, pos, pos), atol=1e-13)



# ---------------------------------------------------------------- local layers (lesson 6, section 7)

def test_window_mask_page_rule():
    g = golden("sliding_window_mask.json")
    for case in g["cases"]:
        m = oracle.window_mask(np.arange(6), np.arange(6), case["window"], case["sinks"])
        assert m.astype(int).tolist() == case["mask"], case


@pytest.mark.parametrize("window,sinks", [(4, 0), (5, 2), (1, 0), (3, 3)])
def test_banded_prefill_equals_rolling_buffer_decode(window, sinks):
    # the page's check: the full causal cache with a banded mask and a token-by-token run with a
    # rolling buffer (no mask at all) compute the same thing; here in float64 the two agree to
    # rounding, and the buffer never holds more than sinks + window slots
    cfg = tiny_cfg()
    w = si.layer_weights(cfg, seed=41)
    t = 13
    x = si.layer_input(cfg, 2, t, seed=41)
    banded, _, _ = oracle.layer_prefill_window(x, w, cfg, window, sinks)
    caches = [oracle.RollingCache(2, 32, window, sinks) for _ in range(2)]
    steps = np.concatenate([oracle.layer_decode_rolling(x[:, i:i + 1], w, cfg, caches) for i in range(t)], axis=1)
    np.testing.assert_allclose(steps, banded, atol=1e-12)
    assert caches[0].k.shape[1] == sinks + window and caches[0].seen == t


def test_window_special_cases():
    cfg = tiny_cfg()
    w = si.layer_weights(cfg, seed=42)
    x = si.layer_input(cfg, 1, 9, seed=42)
    full = oracle.layer_prefill(x, w, cfg)["y"]
    # a window as long as the text is global attention; window 0 means global
    np.testing.assert_allclose(oracle.layer_prefill_window(x, w, cfg, 9)[0], full, atol=1e-12)
    np.testing.assert_allclose(oracle.layer_prefill_window(x, w, cfg, 0)[0], full, atol=1e-12)
    # window 1: every token sees only itself, so its attention output is its own value and the
    # row is the layer on that token alone
    y1 = oracle.layer_prefill_window(x, w, cfg, 1)[0]
    for t in range(9):
        np.testing.assert_allclose(y1[0, t], oracle.layer_prefill(x[:, t:t + 1], w, cfg)["y"][0, 0], atol=1e-12)
    # the banded prefill leaves keys and values untouched (only the mask changes)
    _, kb, vb = oracle.layer_prefill_window(x, w, cfg, 3, 1)
    ref = oracle.layer_prefill(x, w, cfg)
    np.testing.assert_allclose(kb, ref["khat"], atol=1e-12)
    np.testing.assert_allclose(vb, ref["v"], atol=1e-12)


def test_window_decode_on_full_cache_equals_banded_rows():
    # decode with the window mask over a full cache continues the banded prefill
    cfg = tiny_cfg()
    w = si.layer_weights(cfg, seed=43)
    t, window, sinks = 11, 4, 2
    x = si.layer_input(cfg, 2, t, seed=43)
    banded, kb, vb = oracle.layer_prefill_window(x, w, cfg, window, sinks)
    _, kp, vp = oracle.layer_prefill_window(x[:, :t - 1], w, cfg, window, sinks)
    y, kn, vn = oracle.layer_decode_window(x[:, t - 1:], w, cfg, kp, vp, [t - 1, t - 1], window, sinks)
    np.testing.assert_allclose(y[:, 0], banded[:, t - 1], atol=1e-12)
    np.testing.assert_allclose(kn, kb[:, :, t - 1], atol=1e-12)



# ---------------------------------------------------------------- RoPE / RMSNorm variants (Qwen3 page)

def test_rope_pairs_full_split_half_is_rope_rotate():
    rng = np.random.default_rng(61)
    a = rng.standard_normal((3, 7, 16))
    pos = rng.integers(0, 5000, 7).astype(np.float64)
    omega = oracle.rope_inv_freq(16, 1e6)
    np.testing.assert_array_equal(oracle.rope_rotate_pairs(a, pos, omega), oracle.rope_rotate(a, pos, omega))


def test_rope_adjacent_pairs_against_complex_library_routine():
    # adjacent pairs (2i, 2i+1) are the natural complex pairing: torch.view_as_complex
    rng = np.random.default_rng(62)
    d, r = 32, 32
    a = rng.standard_normal((2, 9, d))
    pos = np.arange(9, dtype=np.float64) * 37.0
    omega = oracle.rope_inv_freq(r, 1e4)
    got = oracle.rope_rotate_pairs(a, pos, omega, r, adjacent=True)
    z = torch.view_as_complex(torch.from_numpy(a.reshape(2, 9, d // 2, 2)).contiguous())
    rot = torch.polar(torch.ones(9, d // 2, dtype=torch.float64),
                      torch.from_numpy(pos)[:, None] * torch.from_numpy(omega)[None, :])
    ref = torch.view_as_real(z * rot).reshape(2, 9, d).numpy()
    np.testing.assert_allclose(got, ref, atol=1e-12)
    # the two conventions differ (the page: a model is trained with exactly one), but are the same
    # rotation up to the permutation that takes (2i, 2i+1) to (i, i + d/2)
    split = oracle.rope_rotate_pairs(a, pos, omega, r)
    assert np.abs(split - got).max() > 0.1
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    np.testing.assert_allclose(oracle.rope_rotate_pairs(a[..., perm], pos, omega, r)[..., np.argsort(perm)], got,
                               atol=1e-12)


def test_partial_rope_against_page_apply_rope():
    # apply_rope rotates the first rotary_dim features (split-half within them, frequencies
    # theta^(-2i/rotary_dim)) and passes the rest through; written here with torch.cat /
    # rotate_half the way the page's function is described, in float64
    rng = np.random.default_rng(63)
    d, r = 256, 64
    a = rng.standard_normal((2, 5, d))
    pos = np.array([0, 1, 17, 1000, 40000], dtype=np.float64)
    omega = oracle.rope_inv_freq(r, 1e6)
    got = oracle.rope_rotate_pairs(a, pos, omega, r)
    A = torch.from_numpy(a)
    ang = torch.from_numpy(pos)[:, None] * torch.from_numpy(omega)[None, :]
    ang = torch.cat((ang, ang), dim=-1)
    x_rot, x_pass = A[..., :r], A[..., r:]
    h1, h2 = x_rot.chunk(2, dim=-1)
    ref = torch.cat((x_rot * ang.cos() + torch.cat((-h2, h1), dim=-1) * ang.sin(), x_pass), dim=-1).numpy()
    np.testing.assert_allclose(got, ref, atol=1e-12)
    np.testing.assert_array_equal(got[..., r:], a[..., r:])


def test_linear_rope_scaling_rescales_positions():
    # linear scaling multiplies the positions by a factor: with factor 1/4, position 4p turns every
    # pair exactly as position p does unscaled, i.e. every wavelength is 4x longer
    cfg = tiny_cfg()
    w = si.layer_weights(cfg, seed=64)
    h = si.layer_input(cfg, 1, 6, seed=64)[0]
    p = np.arange(6, dtype=np.float64) * 3
    scaled = si.LayerConfig(**{**cfg.__dict__, "rope_position_scale": 0.25})
    q1, k1, _ = oracle.qk_norm_rope(h, w, scaled, 4 * p)
    q0, k0, _ = oracle.qk_norm_rope(h, w, cfg, p)
    np.testing.assert_allclose(q1, q0, atol=1e-12)
    np.testing.assert_allclose(k1, k0, atol=1e-12)


def test_zero_centred_norm_is_the_standard_norm_with_shifted_gains():
    # (1 + g) with g = gamma - 1 is gamma: the zero-centred layer with every gain shifted by -1
    # equals the standard layer, for all four norms of the layer and the final norm
    cfg = tiny_cfg()
    zc = si.LayerConfig(**{**cfg.__dict__, "norm_unit_offset": True})
    w = si.layer_weights(cfg, seed=65)
    wz = {k: (v - 1.0 if k in si.GAIN_NAMES else v) for k, v in w.items()}
    x = si.layer_input(cfg, 2, 7, seed=65)
    np.testing.assert_allclose(oracle.layer_prefill(x, wz, zc)["y"], oracle.layer_prefill(x, w, cfg)["y"],
                               atol=1e-12)
    gain = si.final_norm_gain(cfg, seed=65)
    np.testing.assert_allclose(oracle.stack_prefill(x, [wz], gain - 1.0, zc),
                               oracle.stack_prefill(x, [w], gain, cfg), atol=1e-12)
    # and the seeded draw of a zero-centred layer is centred on 0
    assert abs(float(np.mean(si.layer_weights(zc, seed=65)["input_layernorm"]))) < 0.05


def test_stack_applies_final_norm_after_last_layer():
    cfg = tiny_cfg()
    ws = [si.layer_weights(cfg, layer=l, seed=17) for l in range(3)]
    gain = si.final_norm_gain(cfg, seed=17)
    x = si.layer_input(cfg, 1, 8, seed=17)
    h = x.astype(np.float64)
    for w in ws:
        h = oracle.layer_prefill(h, w, cfg)["y"]
    want = F.rms_norm(torch.from_numpy(h), (64,), torch.from_numpy(gain.astype(np.float64)), 1e-6).numpy()
    np.testing.assert_allclose(oracle.stack_prefill(x, ws, gain, cfg), want, atol=1e-12)


# ---------------------------------------------------------------- shapes of the workloads

def test_parameter_counts_match_pages():
    g = golden("qwen3_parameter_counts.json")
    small = g["qwen3_0p6b"]
    cfg = si.QWEN3_0P6B
    for key in ["hidden_size", "num_attention_heads", "num_key_value_heads", "head_dim",
                "intermediate_size"]:
        assert getattr(cfg, key) == small[key]
    assert cfg.rope_theta == small["rope_theta"] and cfg.rms_norm_eps == small["rms_norm_eps"]
    sizes = {k: int(np.prod(s)) for k, s in si.weight_shapes(cfg).items()}
    n = small["num_hidden_layers"]
    attention = sum(sizes[k] for k in ["q_proj", "k_proj", "v_proj", "o_proj"])
    assert n * attention == small["attention"]
    assert n * (sizes["q_norm"] + sizes["k_norm"]) == small["qk_norm"]
    assert n * (sizes["gate_proj"] + sizes["up_proj"] + sizes["down_proj"]) == small["feed_forward"]
    assert n * (sizes["input_layernorm"] + sizes["post_attention_layernorm"]) + cfg.hidden_size \
        == small["other_norms"]
    per_layer = sum(sizes.values())
    assert per_layer == 15730944 and abs(per_layer / 1e6 - small["layer_millions_about"]) < 0.05
    big = g["qwen3_8b_card"]
    cfg8 = si.QWEN3_8B
    assert (cfg8.hidden_size, cfg8.num_attention_heads, cfg8.num_key_value_heads, cfg8.head_dim) == \
        (big["hidden_size"], big["num_attention_heads"], big["num_key_value_heads"], big["head_dim"])
    per8 = sum(int(np.prod(s)) for s in si.weight_shapes(cfg8).values())
    non_embedding = big["num_hidden_layers"] * per8 + cfg8.hidden_size
    assert round(non_embedding / 1e9, 2) == big["non_embedding_billions"]


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.00390625, 1.01171875, 1.0 + 2 ** -9, -3.14159, 65504.0], np.float32)
    got = si.round_to_bf16(vals)
    want = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got, want)
