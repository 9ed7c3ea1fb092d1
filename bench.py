"""Benchmark of the Qwen3-style decoder layer on one MI355X.

A step is one full layer prefill (RMSNorm, QKV projection, QK-norm + RoPE + cache write, GQA
causal attention, o_proj + residual, RMSNorm, gate/up + SwiGLU, down + residual) of the
8B-shaped layer (hidden 4096, 32 / 8 heads of 128, intermediate 12288) on one batch of B1 x T8192
synthetic tokens, inputs resident in HBM: the largest of the workloads that fits one GPU.

Each workload first runs untimed for --settle seconds (the board's clocks and power state
settle under load), then --warmup untimed steps, then the timed steps between two HIP events on
the launch stream (the mean), then as many again with an event between consecutive steps (the
median).  A further untimed pass with the library's per-launch events gives the per-kernel
durations from which the roofline fraction of the dominant kernel is taken.

Prints ONE JSON line: tokens/s of the headline step and the roofline of its dominant kernel;
under "workloads" the same record for the 0.6B-shaped layer prefill (B1 T2048), the 28-layer
0.6B-shaped stack with its final norm (B4 T4096), the 8B-shaped decode step on a 32768-key cache
(B16; decode attention and whole-layer bytes against HBM peak) and the tiny fp32 layer; and the
float64 CPU oracle timed on bounded samples of the same workloads, with the parity of the GPU
result against it on identical inputs.

`--summarize-rocprof DB` (no GPU needed) prints a markdown summary of a rocprofv3 database of
this benchmark: per-kernel durations, or FETCH_SIZE / WRITE_SIZE, or MFMA utilisation and clock.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E peak
METRIC = "Qwen3-layer prefill tokens/s & % MFMA peak; 32K decode attn % HBM BW"
CU_COUNT = 256
XCD_COUNT = 8

SHORT = {"c1": "tiny-f32-layer", "c2": "qwen3-0.6b-layer-prefill", "c3": "qwen3-0.6b-stack28-prefill",
         "c4": "qwen3-8b-layer-prefill", "c5": "qwen3-8b-layer-decode-32k"}
HEADLINE = "qwen3-8b-layer-prefill"

# parity bars: fp32 max-abs; bf16 mean relative error and max-abs scaled by the output RMS
F32_MAX_ABS = 1e-4
BF16_MEAN_REL = 5e-3
BF16_MAX_ABS = 3e-2


# ------------------------------------------------------------------------------ work counts

def layer_flops(cfg, b, t):
    """Algorithmic FLOPs per launch of each prefill stage (2*M*N*K for projections; causal
    attention counts 4*D*Hq*sum_t(t+1) over visible keys only)."""
    m = b * t
    h, d, hq, hkv, i = cfg.hidden_size, cfg.head_dim, cfg.num_attention_heads, cfg.num_key_value_heads, \
        cfg.intermediate_size
    return {
        "gemm_qkv": 2.0 * m * (hq + 2 * hkv) * d * h,
        "attention": 4.0 * d * hq * b * t * (t + 1) / 2,
        "gemm_o_residual": 2.0 * m * h * hq * d,
        "gemm_gate_up_swiglu": 2.0 * m * 2 * i * h,
        "gemm_down_residual": 2.0 * m * h * i,
    }


def decode_attention_bytes(cfg, b, cached):
    """Keys and values read once per decode step (each KV head read once for its g query
    heads): 2 * B * Hkv * (cached + 1) * D * 2 bytes."""
    return 2.0 * b * cfg.num_key_value_heads * (cached + 1) * cfg.head_dim * 2


def decode_weight_bytes(cfg):
    """bf16 weight bytes one decode step streams: q, k, v, o, gate, up, down (+ the gains)."""
    h, d, hq, hkv, i = cfg.hidden_size, cfg.head_dim, cfg.num_attention_heads, cfg.num_key_value_heads, \
        cfg.intermediate_size
    return 2.0 * (h * (hq + 2 * hkv) * d + hq * d * h + 3 * h * i + 2 * h + 2 * d)


def decode_skinny_bytes(cfg):
    """Weight bytes of each skinny projection stage of a decode step."""
    h, d, hq, hkv, i = cfg.hidden_size, cfg.head_dim, cfg.num_attention_heads, cfg.num_key_value_heads, \
        cfg.intermediate_size
    return {"gemm_qkv": 2.0 * h * (hq + 2 * hkv) * d, "gemm_o_residual": 2.0 * hq * d * h,
            "gemm_gate_up_swiglu": 4.0 * h * i, "gemm_down_residual": 2.0 * h * i}


# stages that run a GEMM of the table above with more work fused into its epilogue
FUSED_ALIASES = {"gemm_qkv_qknorm_rope": "gemm_qkv"}


def stage_work(work, stage):
    return work.get(stage, work.get(FUSED_ALIASES.get(stage, ""), None))


# ------------------------------------------------------------------------------ timing

SETTLE_S = 0.25
settle_seconds = SETTLE_S    # set from --settle


def settle(torch, fn, seconds):
    """Run fn until `seconds` of wall time have passed (untimed)."""
    t0 = time.perf_counter()
    while seconds > 0:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break


def time_steps(torch, fn, steps, warmup):
    """ms per step over exactly `steps` timed steps between two events on the launch stream
    (synchronised before and after), and the median step from a second run of `steps` with an
    event between consecutive steps."""
    settle(torch, fn, settle_seconds)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    mean = t0.elapsed_time(t1) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return mean, statistics.median(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))


def profile_steps(torch, layers, fn, steps):
    """Average ms per launch of every stage, from the library's events around each launch."""
    for layer in layers:
        layer.set_profiling(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    tot = {}
    for layer in layers:
        for k, (n, ms) in layer.read_profile().items():
            c = tot.setdefault(k, [0, 0.0])
            c[0] += n
            c[1] += ms
        layer.set_profiling(False)
    return {k: v[1] / v[0] for k, v in tot.items()}


def kernel_table(avg_ms, flops=None, byts=None):
    out = {}
    for k, ms in avg_ms.items():
        e = {"avg_ms": round(ms, 5)}
        f = stage_work(flops, k) if flops else None
        if f is not None:
            tf = f / (ms * 1e-3) / 1e12
            e.update(tflops=round(tf, 1), frac_of_bf16_peak=round(tf / PEAK_BF16_TFLOPS, 4))
        b = stage_work(byts, k) if byts else None
        if b is not None:
            gbs = b / (ms * 1e-3) / 1e9
            e.update(gbs=round(gbs, 1), frac_of_hbm_peak=round(gbs / PEAK_HBM_GBS, 4))
        out[k] = e
    return out


def measured_traffic(kernel, workload):
    """HBM traffic per launch recorded by the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (profiles/roofline_traffic.json, counters scaled by the copy calibration), or None when the
    kernel's source has changed since the counters were taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(here, "profiles", "roofline_traffic.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    for e in rec.get("entries", []):
        if e.get("kernel") == kernel and e.get("workload") == workload:
            try:
                with open(os.path.join(here, e["source"]), "rb") as f:
                    sha = hashlib.sha256(f.read()).hexdigest()
            except OSError:
                return None
            return e["traffic_bytes"] if sha == e.get("source_sha256") else None
    return None


def mfma_roofline(stage, ms, flops, workload):
    tf = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": stage, "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(stage, workload),
            "avg_ms": round(ms, 5), "flops_per_launch": flops}


# ------------------------------------------------------------------------------ device inputs

def dev(torch, a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(dtype)


def device_weights(torch, si, cfg, w_np=None, gen=None):
    """The layer's weights on the device: the seeded numpy draws when given (so the oracle sees
    identical values), else drawn on the device with the same distributions."""
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    if w_np is not None:
        return {k: dev(torch, v, dt) for k, v in w_np.items()}
    w = {}
    for name, shape in si.weight_shapes(cfg).items():
        z = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
        w[name] = ((1 + 0.1 * z) if name in si.GAIN_NAMES else 0.02 * z).to(dt)
    return w


class Prefill:
    """One layer, its cache and workspace, set up for repeated prefill steps."""

    def __init__(self, torch, nat, cfg, w_dev, x_dev, cap):
        self.layer = nat.Layer(cfg, w_dev)
        self.w = w_dev
        self.x = x_dev
        self.y = torch.empty_like(x_dev)
        b = x_dev.shape[0]
        shape = (b, cfg.num_key_value_heads, cap, cfg.head_dim)
        self.kc = torch.zeros(shape, dtype=x_dev.dtype, device="cuda")
        self.vc = torch.zeros_like(self.kc)
        self.ws = torch.empty(self.layer.workspace_size(b, x_dev.shape[1], cap), dtype=torch.uint8, device="cuda")

    def __call__(self):
        self.layer.prefill(self.x, self.y, self.kc, self.vc, self.ws)


# ------------------------------------------------------------------------------ workloads

def bench_prefill(torch, si, nat, wl, steps, warmup, w_np=None, x_np=None):
    cfg = wl.cfg
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    gen = torch.Generator(device="cuda").manual_seed(wl.seed)
    w = device_weights(torch, si, cfg, w_np, gen)
    x = dev(torch, x_np, dt) if x_np is not None else \
        torch.randn((wl.batch, wl.seq_len, cfg.hidden_size), generator=gen, device="cuda").to(dt)
    run = Prefill(torch, nat, cfg, w, x, wl.seq_len)
    ms, med = time_steps(torch, run, steps, warmup)
    avg = profile_steps(torch, [run.layer], run, steps)
    flops = layer_flops(cfg, wl.batch, wl.seq_len)
    total = sum(flops.values())
    res = {"ms_per_step": round(ms, 5), "median_ms_per_step": round(med, 5),
           "tokens_per_s": round(wl.batch * wl.seq_len / (ms * 1e-3), 1),
           "layer_tflops": round(total / (ms * 1e-3) / 1e12, 1),
           "layer_frac_of_bf16_peak": round(total / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "steps": steps, "warmup": warmup}
    if cfg.dtype == "bf16":
        dom = max((k for k in avg if stage_work(flops, k) is not None), key=lambda k: avg[k])
        res["roofline"] = mfma_roofline(dom, avg[dom], stage_work(flops, dom), wl.name)
        res["kernels"] = kernel_table(avg, flops)
    else:
        res["kernels"] = kernel_table(avg)
    y = run.y.float().cpu().numpy()
    run.layer.close()
    return res, y


def bench_stack(torch, si, nat, wl, steps, warmup):
    """The layer stack with its final RMSNorm: one step runs every layer's prefill in turn, each
    with its own random-init weights and K/V cache, then the final norm (one shared workspace,
    one stream)."""
    cfg = wl.cfg
    dt = torch.bfloat16
    gen = torch.Generator(device="cuda").manual_seed(wl.seed)
    layers, caches = [], []
    for _ in range(wl.layers):
        w = device_weights(torch, si, cfg, None, gen)
        layers.append((nat.Layer(cfg, w), w))
        kc = torch.zeros((wl.batch, cfg.num_key_value_heads, wl.seq_len, cfg.head_dim), dtype=dt, device="cuda")
        caches.append((kc, torch.zeros_like(kc)))
    gain = (1 + 0.1 * torch.randn(cfg.hidden_size, generator=gen, device="cuda")).to(dt)
    x = torch.randn((wl.batch, wl.seq_len, cfg.hidden_size), generator=gen, device="cuda").to(dt)
    bufs = (torch.empty_like(x), torch.empty_like(x))
    out = torch.empty_like(x)
    ws = torch.empty(layers[0][0].workspace_size(wl.batch, wl.seq_len, wl.seq_len), dtype=torch.uint8, device="cuda")

    def run():
        cur = x
        for i, ((layer, _), (kc, vc)) in enumerate(zip(layers, caches)):
            nxt = bufs[i & 1]
            layer.prefill(cur, nxt, kc, vc, ws)
            cur = nxt
        nat.rmsnorm(cur, gain, out, cfg.rms_norm_eps)

    ms, med = time_steps(torch, run, steps, warmup)
    avg = profile_steps(torch, [l for l, _ in layers], run, max(1, steps // 2))
    flops = layer_flops(cfg, wl.batch, wl.seq_len)
    total = sum(flops.values()) * wl.layers
    dom = max((k for k in avg if stage_work(flops, k) is not None), key=lambda k: avg[k])
    for layer, _ in layers:
        layer.close()
    return {"ms_per_step": round(ms, 5), "median_ms_per_step": round(med, 5),
            "tokens_per_s": round(wl.batch * wl.seq_len / (ms * 1e-3), 1),
            "ms_per_layer": round(ms / wl.layers, 5),
            "stack_tflops": round(total / (ms * 1e-3) / 1e12, 1),
            "stack_frac_of_bf16_peak": round(total / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "steps": steps, "warmup": warmup,
            "roofline": mfma_roofline(dom, avg[dom], stage_work(flops, dom), wl.name),
            "kernels": kernel_table(avg, flops)}


def mfma_ceiling(torch, nat, launches=3, workgroups=1024, iterations=20000):
    """Rate of the matrix-core probe (qwen3_probe_mfma_rate): back-to-back bf16 32x32x16 MFMAs on
    register operands, no memory traffic.  The GEMMs' achieved rate is also given as a fraction of
    this measured ceiling beside the published peak."""
    out = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
    nat.probe_mfma_rate(out, workgroups, iterations)   # warm-up launch
    flops = workgroups * 4 * iterations * 16 * 32768   # 32 x 32 x 16 multiply-adds per MFMA
    best = None
    for _ in range(launches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        nat.probe_mfma_rate(out, workgroups, iterations)
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    if not torch.isfinite(out).all():
        raise RuntimeError("matrix-core probe produced non-finite sums")
    tf = flops / (best * 1e-3) / 1e12
    return {"probe": "qwen3_probe_mfma_rate (bf16 32x32x16 MFMAs on register operands)",
            "workgroups": workgroups, "iterations": iterations, "ms": round(best, 4), "tflops": round(tf, 1),
            "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def plain_read_reference(torch, tensors, steps, warmup):
    """A same-box reference for the decode attention's bandwidth: one plain streaming read of
    the same bytes, torch.sum over rows of 4096 bf16 values into fp32 (one small output per row),
    timed like a step.  Returns ms per pass over all the tensors."""
    views = [t.view(-1, 4096 if t.numel() % 4096 == 0 else t.shape[-1]) for t in tensors]

    def run():
        for v in views:
            torch.sum(v, dim=1, dtype=torch.float32)

    ms, _ = time_steps(torch, run, steps, warmup)
    return ms


def bench_decode(torch, si, nat, wl, steps, warmup, w_np=None):
    cfg = wl.cfg
    dt = torch.bfloat16
    gen = torch.Generator(device="cuda").manual_seed(wl.seed)
    w = device_weights(torch, si, cfg, w_np, gen)
    n = wl.cached
    cap = n + 1
    x = torch.randn((wl.batch, 1, cfg.hidden_size), generator=gen, device="cuda").to(dt)
    run = Prefill(torch, nat, cfg, w, x, cap)
    for c in (run.kc, run.vc):
        for b in range(wl.batch):
            c[b, :, :n].copy_(torch.randn(c[b, :, :n].shape, generator=gen, device="cuda").to(dt))
    lens = [n] * wl.batch
    step = lambda: run.layer.decode(run.x, run.y, lens, run.kc, run.vc, run.ws)
    ms, med = time_steps(torch, step, steps, warmup)
    avg = profile_steps(torch, [run.layer], step, steps)
    read_ms = plain_read_reference(torch, [run.kc, run.vc], steps, warmup)
    run.layer.close()
    kv = decode_attention_bytes(cfg, wl.batch, n)
    read_gbs = kv / (read_ms * 1e-3) / 1e9
    attn_ms = avg["attention_decode_split"] + avg["attention_decode_combine"]
    gbs = kv / (attn_ms * 1e-3) / 1e9
    split_gbs = kv / (avg["attention_decode_split"] * 1e-3) / 1e9
    layer_bytes = kv + decode_weight_bytes(cfg)
    return {"ms_per_step": round(ms, 5), "median_ms_per_step": round(med, 5),
            "tokens_per_s": round(wl.batch / (ms * 1e-3), 1), "steps": steps, "warmup": warmup,
            "roofline": {"bound": "hbm", "kernel": "attention_decode_split + attention_decode_combine",
                         "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("attention_decode_split + attention_decode_combine", wl.name),
                         "avg_ms": round(attn_ms, 5), "bytes_per_launch": kv,
                         "split_kernel_only": {"avg_ms": round(avg["attention_decode_split"], 5),
                                               "achieved": round(split_gbs, 1),
                                               "frac": round(split_gbs / PEAK_HBM_GBS, 4)},
                         # the same K/V bytes read by a plain streaming reduction on this machine:
                         # what the memory system delivers to a simple read, for context
                         "plain_read_reference": {"op": "torch.sum(cache.view(-1, 4096), dim=1, dtype=float32) "
                                                        "over the K and V caches",
                                                  "ms": round(read_ms, 5), "gbs": round(read_gbs, 1),
                                                  "frac_of_peak": round(read_gbs / PEAK_HBM_GBS, 4),
                                                  "attention_frac_of_reference": round(gbs / read_gbs, 4)}},
            "layer_bytes": layer_bytes,
            "layer_gbs": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
            "layer_frac_of_hbm_peak": round(layer_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "kernels": kernel_table(avg, byts=decode_skinny_bytes(cfg))}


def library_gemm(torch, cfg, m, steps, warmup, ours):
    """Context for the projections (--library-gemm): torch.matmul, which is hipBLASLt on this
    image, on the same M x N x K shapes in bf16 - plain products with a bf16 output, none of the
    fused epilogues (residual in fp32, SwiGLU, QK-norm + RoPE + cache write) - beside this
    library's stage time."""
    h, d, i = cfg.hidden_size, cfg.head_dim, cfg.intermediate_size
    hq, hkv = cfg.num_attention_heads, cfg.num_key_value_heads
    shapes = {"gemm_qkv_qknorm_rope": ((hq + 2 * hkv) * d, h), "gemm_o_residual": (h, hq * d),
              "gemm_gate_up_swiglu": (2 * i, h), "gemm_down_residual": (h, i)}
    gen = torch.Generator(device="cuda").manual_seed(1234)
    out = {}
    for stage, (n, k) in shapes.items():
        a = torch.randn((m, k), generator=gen, device="cuda").to(torch.bfloat16)
        w = (0.02 * torch.randn((n, k), generator=gen, device="cuda")).to(torch.bfloat16)
        ms, _ = time_steps(torch, lambda: torch.matmul(a, w.t()), steps, warmup)
        rec = {"M": m, "N": n, "K": k, "avg_ms": round(ms, 5), "tflops": round(2 * m * n * k / (ms * 1e-3) / 1e12, 1)}
        if stage in ours:
            rec["this_library_ms"] = ours[stage]["avg_ms"]
        out[stage] = rec
        del a, w
    torch.cuda.empty_cache()
    return {"kind": "torch.matmul (hipBLASLt), plain bf16 products without the fused epilogues",
            "stages": out}


# ------------------------------------------------------------------------------ CPU baseline

def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = None
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)), "blas_threads": blas}


def parity(got, ref, fp32=False):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    rms = math.sqrt(float(np.mean(ref * ref)))
    out = {"max_abs": float(d.max()), "mean_rel": float(d.sum() / max(np.abs(ref).sum(), 1e-300)),
           "rms_ref": round(rms, 4), "elements": int(d.size)}
    if fp32:
        out.update(max_abs_bar=F32_MAX_ABS, ok=bool(out["max_abs"] <= F32_MAX_ABS))
    else:
        bar = BF16_MAX_ABS * max(1.0, rms)
        out.update(max_abs_bar=round(bar, 5), mean_rel_bar=BF16_MEAN_REL,
                   ok=bool(out["max_abs"] <= bar and out["mean_rel"] <= BF16_MEAN_REL))
    return out


def oracle_prefill_baseline(oracle, wl, w, x, y_gpu, min_s=0.0, note=""):
    """Full float64 oracle prefills of the workload's input, repeated until min_s have passed."""
    t0 = time.perf_counter()
    runs = 0
    while True:
        ref = oracle.layer_prefill(x, w, wl.cfg)
        runs += 1
        el = time.perf_counter() - t0
        if el >= min_s:
            break
    tok = runs * wl.batch * wl.seq_len
    return {"value": round(tok / el, 2), "unit": "tokens/s", "seconds": round(el, 3),
            "sample": f"{runs} full float64 oracle prefill(s) of {wl.name} (B{wl.batch} x T{wl.seq_len}){note}",
            "parity_vs_gpu": parity(y_gpu, ref["y"], fp32=wl.cfg.dtype == "f32")}


def run_cpu_baselines(torch, si, nat, wls, gpu_y, inputs):
    """The oracle as it stands (plain float64 numpy), on the host cores of the GPU machine, on the
    same inputs the GPU consumed: each workload's sample is stated in its record."""
    import oracle
    out = {}
    if "c4" in wls:
        wl = wls["c4"]
        w, x = inputs["c4"]
        print(f"[bench] cpu baseline: {wl.name}", file=sys.stderr, flush=True)
        out[wl.name] = oracle_prefill_baseline(oracle, wl, w, x, gpu_y["c4"])
    if "c2" in wls:
        wl = wls["c2"]
        w, x = inputs["c2"]
        print(f"[bench] cpu baseline: {wl.name}", file=sys.stderr, flush=True)
        out[wl.name] = oracle_prefill_baseline(oracle, wl, w, x, gpu_y["c2"], min_s=3.0)
    if "c1" in wls:
        wl = wls["c1"]
        w, x = inputs["c1"]
        out[wl.name] = oracle_prefill_baseline(oracle, wl, w, x, gpu_y["c1"], min_s=1.0)
    if "c3" in wls:
        # one layer of the stack (layer 0's seeded weights on the stack's B4 x T4096 input),
        # its time scaled by the 28 layers; the final norm's time is negligible beside it
        wl = wls["c3"]
        print(f"[bench] cpu baseline: {wl.name} (layer 0)", file=sys.stderr, flush=True)
        w, x = inputs["c3"]
        t0 = time.perf_counter()
        ref = oracle.layer_prefill(x, w, wl.cfg)
        el = time.perf_counter() - t0
        out[wl.name] = {"value": round(wl.batch * wl.seq_len / (el * wl.layers), 2), "unit": "tokens/s",
                        "seconds": round(el, 3), "scaled_seconds": round(el * wl.layers, 3),
                        "sample": f"one float64 oracle layer (layer 0 of the stack, B{wl.batch} x T{wl.seq_len}) "
                                  f"timed once, its time multiplied by {wl.layers} layers",
                        "parity_vs_gpu": parity(gpu_y["c3"], ref["y"])}
    if "c5" in wls:
        # two of the sixteen sequences, each with its own seeded 32768-key cache; tokens/s from
        # their time (the oracle treats sequences independently)
        wl = wls["c5"]
        print(f"[bench] cpu baseline: {wl.name} (2 sequences)", file=sys.stderr, flush=True)
        w, x, kc, vc, lens, y = inputs["c5"]
        t0 = time.perf_counter()
        ref, _, _ = oracle.layer_decode(x, w, wl.cfg, kc, vc, lens)
        el = time.perf_counter() - t0
        out[wl.name] = {"value": round(len(lens) / el, 3), "unit": "tokens/s", "seconds": round(el, 3),
                        "sample": f"float64 oracle decode of {len(lens)} of the {wl.batch} sequences, "
                                  f"each over {wl.cached} cached keys plus the new one",
                        "parity_vs_gpu": parity(y, ref)}
    return out


def decode_parity_inputs(torch, si, nat, wl, w_np, nseq=2):
    """A decode call on `nseq` sequences with seeded caches of the workload's length (same
    kernels and launch shapes per sequence as the timed batch), for the oracle to check."""
    cfg = wl.cfg
    n = wl.cached
    cap = n + 1
    hkv, d = cfg.num_key_value_heads, cfg.head_dim
    kc = np.zeros((nseq, hkv, cap, d), np.float32)
    vc = np.zeros((nseq, hkv, cap, d), np.float32)

    def sink(b, h, kb, vb):
        kc[b, h, :n] = kb
        vc[b, h, :n] = vb

    si.fill_decode_cache(cfg, nseq, n, sink, seed=wl.seed)
    x = si.layer_input(cfg, nseq, 1, seed=wl.seed)
    dt = torch.bfloat16
    w = device_weights(torch, si, cfg, w_np)
    layer = nat.Layer(cfg, w)
    kd, vd = dev(torch, kc, dt), dev(torch, vc, dt)
    xd = dev(torch, x, dt)
    yd = torch.empty_like(xd)
    ws = torch.empty(layer.workspace_size(nseq, 1, cap), dtype=torch.uint8, device="cuda")
    layer.decode(xd, yd, [n] * nseq, kd, vd, ws)
    torch.cuda.synchronize()
    y = yd.float().cpu().numpy()
    layer.close()
    del kd, vd
    return w_np, x, kc, vc, [n] * nseq, y


# ------------------------------------------------------------------------------ rocprof summaries

def _short(name):
    import re
    if name.startswith("_Z"):
        import subprocess
        try:
            name = subprocess.run(["c++filt", name], capture_output=True, text=True).stdout.strip() or name
        except OSError:
            pass
    name = re.sub(r"\(anonymous namespace\)::|q3::", "", name)
    name = name.replace("bool _Accum", "bf16").replace("__bf16", "bf16")
    return re.sub(r"^void ", "", name)


def _ours(name):
    """Kernels of this library (torch's setup kernels and runtime copies are left out)."""
    return not (name.startswith("at::") or name.startswith("void at::") or "rocclr" in name)


# Copy calibration of the byte counters (a plain 256 MiB device copy in the same runs):
# FETCH_SIZE reads half the bytes read, WRITE_SIZE the bytes written.
FETCH_FACTOR = 2.0
WRITE_FACTOR = 1.0
# The dominant kernel of each workload's step, as the rocprofv3 database names it: (kernel name
# prefix, grid in workgroups) -> (stage, workload, source file).
ROOFLINE_KERNELS = {
    ("gemm_bf16_pp_kernel<(Epilogue)2, 256>", (3072, 1, 1)): ("gemm_gate_up_swiglu", "qwen3-8b-layer-prefill",
                                                            "transformer_decoder_layer_rmsnorm_amd/csrc/gemm_bf16.hip"),
    ("flash_prefill_kernel<2, 2, false>", (512, 1, 1)): ("attention", "qwen3-0.6b-layer-prefill",
                                                        "transformer_decoder_layer_rmsnorm_amd/csrc/attention_prefill.hip"),
    ("flash_prefill_pp_kernel<2>", (1024, 1, 1)): ("attention", "qwen3-0.6b-stack28-prefill",
                                                  "transformer_decoder_layer_rmsnorm_amd/csrc/attention_prefill.hip"),
    ("flash_prefill_pp_kernel<4>", (1024, 1, 1)): ("attention", "qwen3-8b-layer-prefill",
                                                  "transformer_decoder_layer_rmsnorm_amd/csrc/attention_prefill.hip"),
}
DECODE_KERNELS = (("decode_split_kernel<4>", (33, 8, 16)), ("decode_combine_kernel", (32, 16, 1)))


def _traffic(dbs, mode):
    """Per-kernel FETCH_SIZE / WRITE_SIZE (KiB per dispatch) from the databases of the two
    counter runs, and the calibrated HBM bytes per dispatch."""
    import collections
    import hashlib
    import sqlite3
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for db in dbs:
        c = sqlite3.connect(db).cursor()
        for n, gx, gy, gz, wx, cn, v in c.execute(
                "select kernel_name, grid_size_x, grid_size_y, grid_size_z, workgroup_size_x, counter_name, value "
                "from counters_collection").fetchall():
            if _ours(n) and cn in ("FETCH_SIZE", "WRITE_SIZE"):
                agg[(_short(n), (gx // max(wx, 1), gy, gz))][cn].append(v)
    avg = lambda v: sum(v) / len(v) if v else float("nan")
    byts = lambda a: 1024 * (FETCH_FACTOR * avg(a["FETCH_SIZE"]) + WRITE_FACTOR * avg(a["WRITE_SIZE"]))
    if mode == "traffic":
        lines = ["| kernel | grid (workgroups) | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes |",
                 "|---|---|---|---|---|---|"]
        for k in sorted(agg, key=lambda k: -avg(agg[k]["FETCH_SIZE"])):
            a = agg[k]
            lines.append(f"| `{k[0]}` | {k[1]} | {len(a['FETCH_SIZE'])} | {avg(a['FETCH_SIZE']):.1f} | "
                         f"{avg(a['WRITE_SIZE']):.1f} | {byts(a):.4g} |")
        return "\n".join(lines)
    here = os.path.dirname(os.path.abspath(__file__))
    sha = lambda p: hashlib.sha256(open(os.path.join(here, p), "rb").read()).hexdigest()
    entries = []
    for (prefix, grid), (stage, wl, source) in ROOFLINE_KERNELS.items():
        for (name, g), a in agg.items():
            if name.startswith(prefix) and g == grid:
                entries.append({"kernel": stage, "workload": wl, "grid": list(grid),
                                "fetch_kib": round(avg(a["FETCH_SIZE"]), 1), "write_kib": round(avg(a["WRITE_SIZE"]), 1),
                                "traffic_bytes": int(byts(a)), "source": source, "source_sha256": sha(source)})
    dec = [a for (name, g), a in agg.items() for p, gg in DECODE_KERNELS if name.startswith(p) and g == gg]
    if len(dec) == 2:
        src = "transformer_decoder_layer_rmsnorm_amd/csrc/attention_decode.hip"
        entries.append({"kernel": "attention_decode_split + attention_decode_combine",
                        "workload": "qwen3-8b-layer-decode-32k", "grid": [list(g) for _, g in DECODE_KERNELS],
                        "traffic_bytes": int(sum(byts(a) for a in dec)), "source": src, "source_sha256": sha(src)})
    return json.dumps({"fetch_factor": FETCH_FACTOR, "write_factor": WRITE_FACTOR, "entries": entries}, indent=1)


def summarize_rocprof(db, mode):
    """Markdown table from a rocprofv3 database of this benchmark: 'trace' (durations per
    kernel and grid), 'traffic' (FETCH_SIZE / WRITE_SIZE per dispatch), 'issue' (instruction mix
    and co-issue of the MFMA kernels), or 'mfma' (MFMA
    utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs * 256 CUs * one XCD's GRBM_GUI_ACTIVE), the
    share of SIMD cycles whose matrix pipe was busy, and the clock = one XCD's GRBM_GUI_ACTIVE /
    the dispatch's duration, meaningful for dispatches far longer than the counter overhead)."""
    import collections
    import sqlite3
    if mode in ("traffic", "traffic-json"):
        return _traffic(db.split(","), mode)
    c = sqlite3.connect(db).cursor()
    lines = []
    if mode == "trace":
        rows = c.execute("select name, grid_x, grid_y, grid_z, workgroup_x, start, end from kernels").fetchall()
        agg = collections.defaultdict(list)
        for n, gx, gy, gz, wx, s, e in rows:
            if _ours(n):
                agg[(_short(n), gx // max(wx, 1), gy, gz)].append((e - s) / 1e3)
        lines.append("| kernel | grid (workgroups) | calls | avg us | median us |")
        lines.append("|---|---|---|---|---|")
        for (n, gx, gy, gz), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
            v = sorted(v)
            lines.append(f"| `{n}` | ({gx}, {gy}, {gz}) | {len(v)} | {sum(v) / len(v):.2f} | {v[len(v) // 2]:.2f} |")
        return "\n".join(lines)
    rows = c.execute("select dispatch_id, kernel_name, grid_size_x, grid_size_y, grid_size_z, workgroup_size_x, "
                     "counter_name, value, duration from counters_collection").fetchall()
    disp = collections.defaultdict(lambda: collections.defaultdict(float))
    key, dur = {}, {}
    for di, n, gx, gy, gz, wx, cn, v, du in rows:
        if not _ours(n):
            continue
        disp[di][cn] += v
        key[di] = (_short(n), gx // max(wx, 1), gy, gz)
        dur[di] = du
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for di, cs in disp.items():
        for cn, v in cs.items():
            agg[key[di]][cn].append(v)
        if dur.get(di, 0) > 0:
            agg[key[di]]["_us"].append(dur[di] / 1e3)
            if "GRBM_GUI_ACTIVE" in cs:
                # the database sums GRBM_GUI_ACTIVE over the 8 XCDs; one XCD's count is the
                # kernel's busy cycles (rocprofv3's derived metrics take the max over XCDs)
                agg[key[di]]["_mhz"].append(cs["GRBM_GUI_ACTIVE"] / XCD_COUNT / dur[di] * 1e3)
    avg = lambda v: sum(v) / len(v) if v else float("nan")
    if mode == "issue":
        # instruction mix of the kernels that use the matrix cores: VALU, transcendental and LDS
        # instructions per MFMA instruction, MFMA busy share (as in 'mfma') and the share of
        # MFMA-busy cycles in which the VALU also issued (SQ_VALU_MFMA_COEXEC_CYCLES)
        lines.append("| kernel | grid (workgroups) | dispatches | avg us | VALU / MFMA | TRANS / MFMA | "
                     "LDS / MFMA | MFMA busy % | VALU co-issue % of MFMA busy |")
        lines.append("|---|---|---|---|---|---|---|---|---|")
        for k in sorted(agg, key=lambda k: -avg(agg[k].get("_us", [0])) * len(agg[k].get("_us", [0]))):
            a = agg[k]
            mf = avg(a.get("SQ_INSTS_MFMA", []))
            if not mf or mf != mf:
                continue
            gui = avg(a.get("GRBM_GUI_ACTIVE", [])) / XCD_COUNT
            busy = avg(a.get("SQ_VALU_MFMA_BUSY_CYCLES", []))
            util = 100.0 * busy / (4 * CU_COUNT * gui) if gui else float("nan")
            co = 100.0 * avg(a.get("SQ_VALU_MFMA_COEXEC_CYCLES", [])) / busy if busy else float("nan")
            lines.append(f"| `{k[0]}` | {k[1:]} | {len(a.get('GRBM_GUI_ACTIVE', []))} | {avg(a.get('_us', [])):.2f} | "
                         f"{avg(a.get('SQ_INSTS_VALU', [])) / mf:.2f} | {avg(a.get('SQ_INSTS_VALU_TRANS_F32', [])) / mf:.2f} | "
                         f"{avg(a.get('SQ_INSTS_LDS', [])) / mf:.2f} | {util:.1f} | {co:.1f} |")
        return "\n".join(lines)
    if mode == "lds":
        # LDS use of each kernel: SQ_LDS_IDX_ACTIVE and SQ_LDS_BANK_CONFLICT are cycles summed over
        # the CUs, so divided by 256 CUs x one XCD's GRBM_GUI_ACTIVE they are the share of CU
        # cycles the LDS was busy or stalled on bank conflicts; the *_BANDWIDTH counters count 64-byte
        # units moved; SQ_WAIT_INST_LDS counts wave-cycles (units of 4) waiting to issue an LDS
        # instruction, given here per wave slot (8 waves per CU at full occupancy of these kernels)
        lines.append("| kernel | grid (workgroups) | dispatches | avg us | LDS busy % of CU cycles | bank-conflict "
                     "stall % | LDS read B/clk/CU | LDS write B/clk/CU | LDS-issue wait % of 8 wave slots |")
        lines.append("|---|---|---|---|---|---|---|---|---|")
        for k in sorted(agg, key=lambda k: -avg(agg[k].get("_us", [0])) * len(agg[k].get("_us", [0]))):
            a = agg[k]
            gui = avg(a.get("GRBM_GUI_ACTIVE", [])) / XCD_COUNT
            if not gui or not a.get("SQ_LDS_IDX_ACTIVE") or avg(a["SQ_LDS_IDX_ACTIVE"]) < 0.01 * CU_COUNT * gui:
                continue
            cyc = CU_COUNT * gui
            lines.append(f"| `{k[0]}` | {k[1:]} | {len(a['GRBM_GUI_ACTIVE'])} | {avg(a.get('_us', [])):.2f} | "
                         f"{100 * avg(a['SQ_LDS_IDX_ACTIVE']) / cyc:.1f} | "
                         f"{100 * avg(a.get('SQ_LDS_BANK_CONFLICT', [0])) / cyc:.2f} | "
                         f"{64 * avg(a.get('SQ_INSTS_LDS_LOAD_BANDWIDTH', [0])) / cyc:.1f} | "
                         f"{64 * avg(a.get('SQ_INSTS_LDS_STORE_BANDWIDTH', [0])) / cyc:.1f} | "
                         f"{100 * 4 * avg(a.get('SQ_WAIT_INST_LDS', [0])) / (8 * cyc):.1f} |")
        return "\n".join(lines)
    lines.append("| kernel | grid (workgroups) | dispatches | avg us | MFMA busy % | clock MHz | bf16 MFMA MOPS |")
    lines.append("|---|---|---|---|---|---|---|")
    for k in sorted(agg, key=lambda k: -avg(agg[k].get("_us", [0])) * len(agg[k].get("_us", [0]))):
        a = agg[k]
        gui = avg(a.get("GRBM_GUI_ACTIVE", [])) / XCD_COUNT
        # SQ_VALU_MFMA_BUSY_CYCLES is summed over the 4 * 256 SIMDs
        util = 100.0 * avg(a.get("SQ_VALU_MFMA_BUSY_CYCLES", [])) / (4 * CU_COUNT * gui) if gui else float("nan")
        lines.append(f"| `{k[0]}` | {k[1:]} | {len(a.get('GRBM_GUI_ACTIVE', []))} | {avg(a.get('_us', [])):.2f} | "
                     f"{util:.1f} | {avg(a.get('_mhz', [])):.0f} | "
                     f"{avg(a.get('SQ_INSTS_VALU_MFMA_MOPS_BF16', [])):.4g} |")
    return "\n".join(lines)


# ------------------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workloads", default="c4,c2,c3,c5,c1",
                    help="comma list of c1..c5 (c4, the headline, always runs)")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed steps before each workload's warmup steps (clock settling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device-to-device copy 5 times (scale for HBM byte counters)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time torch.matmul (hipBLASLt) on the headline workload's projection shapes")
    ap.add_argument("--summarize-rocprof", metavar="DB", help="print a markdown summary of a rocprofv3 database")
    ap.add_argument("--mode", default="trace", choices=["trace", "traffic", "traffic-json", "mfma", "issue", "lds"],
                    help="summary kind; traffic modes take the FETCH_SIZE and WRITE_SIZE databases, comma-separated")
    args = ap.parse_args()
    if args.summarize_rocprof:
        print(summarize_rocprof(args.summarize_rocprof, args.mode))
        return
    global settle_seconds
    settle_seconds = max(0.0, args.settle)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path: the layer's kernels run on one GPU's share of the work.", file=sys.stderr)
        sys.exit(2)
    keys = ["c4"] + [k.strip() for k in args.workloads.split(",") if k.strip() and k.strip() != "c4"]
    for k in keys:
        if k not in SHORT:
            ap.error(f"unknown workload {k}")

    import torch
    import seeded_inputs as si
    from transformer_decoder_layer_rmsnorm_amd import _native as nat
    nat.lib()
    torch.cuda.set_device(0)
    wls = {k: si.WORKLOADS[SHORT[k]] for k in keys}
    cpu = not args.no_cpu_baseline

    calib = None
    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        ms, _ = time_steps(torch, lambda: dst.copy_(src), 5, 1)
        calib = {"bytes_read": n, "bytes_written": n, "avg_ms": round(ms, 4),
                 "gbs": round(2 * n / (ms * 1e-3) / 1e9, 1)}
        del src, dst

    gpu_y, inputs, records = {}, {}, {}
    w8 = None
    for k in keys:
        wl = wls[k]
        print(f"[bench] {wl.name}", file=sys.stderr, flush=True)
        if k in ("c1", "c2", "c4"):
            w_np = x_np = None
            if cpu or k == "c1":
                w_np = si.layer_weights(wl.cfg, seed=wl.seed)
                x_np = si.layer_input(wl.cfg, wl.batch, wl.seq_len, seed=wl.seed)
                inputs[k] = (w_np, x_np)
                if k == "c4":
                    w8 = w_np
            steps = args.steps if k != "c1" else max(args.steps, 50)
            res, y = bench_prefill(torch, si, nat, wl, steps, args.warmup, w_np, x_np)
            gpu_y[k] = y
            records[k] = res
        elif k == "c3":
            records[k] = bench_stack(torch, si, nat, wl, max(2, args.steps // 10), 1)
            if cpu:
                w_np = si.layer_weights(wl.cfg, layer=0, seed=wl.seed)
                x_np = si.layer_input(wl.cfg, wl.batch, wl.seq_len, seed=wl.seed)
                inputs[k] = (w_np, x_np)
                _, gpu_y[k] = bench_prefill(torch, si, nat, wl, 1, 0, w_np, x_np)
        elif k == "c5":
            records[k] = bench_decode(torch, si, nat, wl, args.steps, args.warmup, w8)
            if cpu:
                w_np = w8 if w8 is not None else si.layer_weights(wl.cfg, seed=wl.seed)
                inputs[k] = decode_parity_inputs(torch, si, nat, wl, w_np)
        torch.cuda.empty_cache()

    head = records["c4"]
    wl4 = wls["c4"]
    ceiling = mfma_ceiling(torch, nat)
    ceiling["kernel_frac_of_ceiling"] = round(head["roofline"]["achieved"] / ceiling["tflops"], 4)
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": settle_seconds,
        "ms_per_step": head["ms_per_step"],
        "median_ms_per_step": head["median_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and inputs of the workload's shapes)",
        "config": {"workload": wl4.name, "batch": wl4.batch, "seq_len": wl4.seq_len,
                   "hidden_size": wl4.cfg.hidden_size,
                   "heads": [wl4.cfg.num_attention_heads, wl4.cfg.num_key_value_heads],
                   "head_dim": wl4.cfg.head_dim, "intermediate_size": wl4.cfg.intermediate_size},
        "roofline": dict(head["roofline"], mfma_ceiling=ceiling),
        "layer_tflops": head["layer_tflops"],
        "layer_frac_of_bf16_peak": head["layer_frac_of_bf16_peak"],
        "kernels": head["kernels"],
        "workloads": {wls[k].name: records[k] for k in keys if k != "c4"},
    }
    if calib:
        line["copy_calibration"] = calib
    if args.library_gemm:
        line["library_gemm"] = library_gemm(torch, wl4.cfg, wl4.batch * wl4.seq_len, 10, 3, head["kernels"])
    if cpu:
        base = run_cpu_baselines(torch, si, nat, wls, gpu_y, inputs)
        info = cpu_info()
        head_b = base.pop(wl4.name)
        line["cpu_baseline"] = {"value": head_b["value"], "unit": head_b["unit"],
                                "cores": info["blas_threads"] or info["affinity_cores"], "kind": "oracle",
                                "sample": head_b["sample"], "seconds": head_b["seconds"],
                                "parity_vs_gpu": head_b["parity_vs_gpu"], **info,
                                "workloads": base}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
