"""Helpers for the GPU parity tests: upload seeded inputs, run the layer through the C ABI
(Python binding), read intermediates back from the workspace, and compare with the oracle.

Tolerances (written here, used by every GPU test):
  * fp32 storage: max |gpu - oracle| <= 1e-4.
  * bf16 storage, layer output: mean relative error sum|d| / sum|ref| <= 5e-3 and
    max |d| <= 3e-2 * max(1, rms(ref)) (the 3e-2 bar scaled by the output RMS, since a
    bf16 output of magnitude >= 8 already has a half-ulp of 3.1e-2).
  * teacher-forced single kernels (the oracle step fed the GPU's own bf16 input) are held
    to what one bf16 rounding of the output allows, see `assert_rounded`.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import seeded_inputs as si
from transformer_decoder_layer_rmsnorm_amd import _native as nat

F32_MAX_ABS = 1e-4
BF16_MEAN_REL = 5e-3
BF16_MAX_ABS = 3e-2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def to_dev(a, cfg):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(torch_dtype(cfg))


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


class GpuLayer:
    """A layer's seeded weights on the device plus its native handle."""

    def __init__(self, cfg, weights_np):
        self.cfg = cfg
        self.w_np = weights_np
        self.w_dev = {k: to_dev(v, cfg) for k, v in weights_np.items()}
        self.layer = nat.Layer(cfg, self.w_dev)

    @classmethod
    def seeded(cls, cfg, layer=0, seed=0):
        return cls(cfg, si.layer_weights(cfg, layer=layer, seed=seed))

    def alloc_cache(self, batch, cap):
        c = self.cfg
        shape = (batch, c.num_key_value_heads, cap, c.head_dim)
        return (torch.zeros(shape, dtype=torch_dtype(c), device="cuda"),
                torch.zeros(shape, dtype=torch_dtype(c), device="cuda"))

    def workspace(self, batch, seq_len, cap):
        n = self.layer.workspace_size(batch, seq_len, cap)
        return torch.empty(n, dtype=torch.uint8, device="cuda")

    def prefill(self, x_dev, cap=None, caches=None, ws=None, y_dev=None, starts=None, pads=None):
        b, t, _ = x_dev.shape
        cap = cap or t
        kc, vc = caches or self.alloc_cache(b, cap)
        ws = ws if ws is not None else self.workspace(b, t, cap)
        y = y_dev if y_dev is not None else torch.empty_like(x_dev)
        self.layer.prefill(x_dev, y, kc, vc, ws, start_positions=starts, pad_lens=pads)
        torch.cuda.synchronize()
        return y, kc, vc, ws

    def decode(self, x_dev, lens, kc, vc, ws=None, y_dev=None, pad_starts=None, pad_lens=None):
        b = x_dev.shape[0]
        cap = kc.shape[2]
        ws = ws if ws is not None else self.workspace(b, 1, cap)
        y = y_dev if y_dev is not None else torch.empty_like(x_dev)
        self.layer.decode(x_dev, y, lens, kc, vc, ws, pad_starts=pad_starts, pad_lens=pad_lens)
        torch.cuda.synchronize()
        return y, ws

    def intermediates(self, ws, batch, seq_len, cap=0):
        """Views of the workspace regions as float64 arrays."""
        c = self.cfg
        lay = self.layer.workspace_layout(batch, seq_len, cap)
        m = batch * seq_len
        h, d, hq, hkv, i = c.hidden_size, c.head_dim, c.num_attention_heads, c.num_key_value_heads, c.intermediate_size
        td = torch_dtype(c)
        es = 2 if c.dtype == "bf16" else 4

        def region(off, shape, dtype=td, size=None):
            n = int(np.prod(shape))
            b = size or (2 if dtype == torch.bfloat16 else 4)
            return to_np(ws[off: off + n * b].view(dtype).view(shape))

        return dict(
            h=region(lay.h, (batch, seq_len, h)),
            qkv=region(lay.qkv, (batch, seq_len, (hq + 2 * hkv) * d)),
            qhat=region(lay.qhat, (batch, hq, seq_len, d)),
            attn=region(lay.attn, (batch, seq_len, hq * d)),
            x1=region(lay.x1, (batch, seq_len, h), torch.float32),
            h2=region(lay.h2, (batch, seq_len, h)),
            act=region(lay.act, (batch, seq_len, i)),
        )


def bf16_metrics(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    rms = math.sqrt(float(np.mean(ref * ref)))
    return dict(max_abs=float(d.max()), mean_rel=float(d.sum() / max(np.abs(ref).sum(), 1e-300)),
                rms=rms, max_abs_bar=BF16_MAX_ABS * max(1.0, rms))


def assert_bf16_parity(got, ref, what=""):
    m = bf16_metrics(got, ref)
    log(f"  {what}: max_abs {m['max_abs']:.4g} (bar {m['max_abs_bar']:.4g}), "
        f"mean_rel {m['mean_rel']:.3g} (bar {BF16_MEAN_REL}), rms(ref) {m['rms']:.3g}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert m["mean_rel"] <= BF16_MEAN_REL, f"{what}: {m}"
    assert m["max_abs"] <= m["max_abs_bar"], f"{what}: {m}"
    return m


def assert_f32_parity(got, ref, what="", bar=F32_MAX_ABS):
    d = float(np.abs(np.asarray(got) - np.asarray(ref)).max())
    log(f"  {what}: max_abs {d:.3g} (bar {bar})")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert d <= bar, f"{what}: max abs {d}"
    return d


def assert_rounded(got, ref, what="", rel=2.0 ** -8, abs_frac=1e-3):
    """Elementwise: |got - ref| <= rel*|ref| + abs_frac*rms(ref): one bf16 rounding of the
    result (half-ulp = 2^-9 relative) plus fp32 accumulation-order noise."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = math.sqrt(float(np.mean(ref * ref))) or 1.0
    bound = rel * np.abs(ref) + abs_frac * rms
    excess = np.abs(got - ref) - bound
    worst = float(excess.max())
    log(f"  {what}: worst excess over rounding bound {worst:.3g} (max_abs {np.abs(got - ref).max():.3g})")
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    assert worst <= 0, f"{what}: exceeds rounding bound by {worst}"


def small_bf16_cfg(hq=4, hkv=2, hidden=256, inter=384, **kw):
    return si.LayerConfig(hidden_size=hidden, num_attention_heads=hq, num_key_value_heads=hkv, head_dim=128,
                          intermediate_size=inter, dtype="bf16", **kw)


def oracle_qk_from_proj(qkv, w, cfg, positions):
    """Oracle step 3 fed the GPU's projections: per-head Q/K RMSNorm then RoPE."""
    t = qkv.shape[0]
    hq, hkv, d = cfg.num_attention_heads, cfg.num_key_value_heads, cfg.head_dim
    q = qkv[:, : hq * d].reshape(t, hq, d).transpose(1, 0, 2)
    k = qkv[:, hq * d: (hq + hkv) * d].reshape(t, hkv, d).transpose(1, 0, 2)
    v = qkv[:, (hq + hkv) * d:].reshape(t, hkv, d).transpose(1, 0, 2)
    omega = oracle.rope_inv_freq(d, cfg.rope_theta)
    qhat = oracle.rope_rotate(oracle.rmsnorm(q, w["q_norm"], cfg.rms_norm_eps), positions, omega)
    khat = oracle.rope_rotate(oracle.rmsnorm(k, w["k_norm"], cfg.rms_norm_eps), positions, omega)
    return qhat, khat, v


def check_decode_steps(gl, ws, lens, kd, vd):
    """Teacher-forced decode kernels: the new token's qk-norm/RoPE at position lens[b] (and
    its cache slot), then attention over slots 0..lens[b] of the GPU's own cache."""
    cfg = gl.cfg
    b, cap = len(lens), kd.shape[2]
    it = gl.intermediates(ws, b, 1, cap)
    kdn, vdn = to_np(kd), to_np(vd)
    hq, d = cfg.num_attention_heads, cfg.head_dim
    for i, n in enumerate(lens):
        qhat, khat, v = oracle_qk_from_proj(it["qkv"][i], gl.w_np, cfg, np.array([n]))
        assert_rounded(it["qhat"][i], qhat, f"decode qknorm_rope q at position {n}")
        assert_rounded(kdn[i, :, n], khat[:, 0], f"decode new key at slot {n}")
        assert np.array_equal(vdn[i, :, n], v[:, 0]), "new value copied unchanged"
        if n + 1 < cap:
            assert not np.any(kdn[i, :, n + 1:]), "slots past the new token untouched"
        att = oracle.gqa_causal_attention(it["qhat"][i], kdn[i, :, : n + 1], vdn[i, :, : n + 1],
                                          np.array([n]), np.arange(n + 1))
        assert_bf16_parity(it["attn"][i], att.transpose(1, 0, 2).reshape(1, hq * d), f"decode attention, {n + 1} keys")


# ---------------------------------------------------------------- full-tensor checks at full size

def _pool_map(fn, items, workers=8):
    """Map fn over items on a thread pool (numpy releases the GIL in its array work)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=max(1, min(workers, len(items)))) as pool:
        return list(pool.map(fn, items))


def oracle_attention_per_head(qhat, kc, vc, q_pos, k_pos, workers=8):
    """oracle.gqa_causal_attention evaluated head by head on a thread pool (the same
    definition; each call sees one query head and the KV head it reads).
    qhat [Hq, T, D], kc / vc [Hkv, S, D] -> [Hq, T, D]."""
    hq, hkv = qhat.shape[0], kc.shape[0]
    g = hq // hkv
    outs = _pool_map(lambda h: oracle.gqa_causal_attention(qhat[h:h + 1], kc[h // g: h // g + 1],
                                                           vc[h // g: h // g + 1], q_pos, k_pos)[0],
                     list(range(hq)), workers)
    return np.stack(outs)


def oracle_layer_prefill_parallel(x, w, cfg, workers=4):
    """oracle.layer_prefill with its sequences evaluated on a thread pool (the oracle treats
    sequences independently, so this is the same result)."""
    parts = _pool_map(lambda b: oracle.layer_prefill(x[b:b + 1], w, cfg), list(range(x.shape[0])), workers)
    return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}


def check_prefill_stages_full(gl, x, y_dev, kc_dev, vc_dev, ws, what):
    """Every element of every stage of a prefill on an empty cache (positions 0..T-1), each
    stage fed the GPU's own input for it (teacher forcing) from the workspace:
      h = rmsnorm(x);  qhat, khat, v from h through the projections, QK-norm and RoPE (the
      fused QKV epilogue never stores the raw projections, so this step starts at h);
      attn from the GPU's qhat and cache;  x1 = x + attn Wo^T (fp32);  h2 = rmsnorm(x1);
      act = silu(h2 Wg^T) * (h2 Wu^T);  y = x1 + act Wd^T.
    Returns the stage metrics (raw max-abs included)."""
    cfg, w = gl.cfg, gl.w_np
    b, t, _ = x.shape
    hq, hkv, d = cfg.num_attention_heads, cfg.num_key_value_heads, cfg.head_dim
    eps = cfg.rms_norm_eps
    it = gl.intermediates(ws, b, t)
    y = to_np(y_dev)
    kcn, vcn = to_np(kc_dev), to_np(vc_dev)
    pos = np.arange(t)
    f64 = lambda a: np.asarray(a, np.float64)
    wqkv = np.concatenate([w["q_proj"], w["k_proj"], w["v_proj"]]).astype(np.float64)
    stats = {}
    for s in range(b):
        tag = f"{what} seq {s}"
        assert_rounded(it["h"][s], oracle.rmsnorm(x[s], w["input_layernorm"], eps), f"{tag}: rmsnorm_input")
        qhat, khat, v = oracle_qk_from_proj(it["h"][s] @ wqkv.T, w, cfg, pos)
        assert_rounded(it["qhat"][s], qhat, f"{tag}: q (QKV + QK-norm + RoPE)")
        assert_rounded(kcn[s, :, :t], khat, f"{tag}: k cache (QKV + QK-norm + RoPE)")
        assert_rounded(vcn[s, :, :t], v, f"{tag}: v cache (QKV)")
        del qhat, khat, v
        log(f"  {tag}: attention, {hq} heads")
        att = oracle_attention_per_head(it["qhat"][s], kcn[s, :, :t], vcn[s, :, :t], pos, pos)
        stats[f"attn{s}"] = assert_bf16_parity(it["attn"][s], att.transpose(1, 0, 2).reshape(t, hq * d),
                                               f"{tag}: attention")
        del att
        x1 = x[s] + it["attn"][s] @ f64(w["o_proj"]).T
        d1 = np.abs(it["x1"][s] - x1)
        log(f"  {tag}: x1 (fp32) max_abs {d1.max():.3g}")
        np.testing.assert_allclose(it["x1"][s], x1, rtol=1e-5, atol=2e-5)
        del x1, d1
        assert_rounded(it["h2"][s], oracle.rmsnorm(it["x1"][s], w["post_attention_layernorm"], eps),
                       f"{tag}: rmsnorm_post")
        h2 = it["h2"][s]
        act = oracle.silu(h2 @ f64(w["gate_proj"]).T) * (h2 @ f64(w["up_proj"]).T)
        assert_rounded(it["act"][s], act, f"{tag}: gate/up + SwiGLU")
        del act
        assert_rounded(y[s], it["x1"][s] + it["act"][s] @ f64(w["down_proj"]).T, f"{tag}: down + residual")
    return stats
