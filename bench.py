"""Benchmark of the Qwen3-style decoder layer on one MI355X.

A step is one full layer prefill (RMSNorm, QKV projection, QK-norm + RoPE + cache write,
GQA causal attention, o_proj + residual, RMSNorm, gate/up + SwiGLU, down + residual) of the
0.6B-shaped layer on one batch of B1 x T2048 synthetic tokens, inputs resident in HBM.
Each workload first runs untimed for --settle seconds (0.25 by default: the board's clocks and
power state settle under load), then --warmup untimed steps, then the timed steps.
Prints ONE JSON line: tokens/s of that step, the roofline fraction of its dominant kernel
(per-kernel durations from HIP events recorded by the library around each launch, on the
launch stream), the float64 CPU oracle timed on a bounded sample of the same workload, and,
as extra context, the 8B-shaped layer prefill (B1 T8192), the 28-layer 0.6B-shaped stack with its
final norm (B4 T4096) and the 8B-shaped decode step on a 32768-key cache (decode attention
achieved GB/s against HBM peak).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E peak
METRIC = "Qwen3-layer prefill tokens/s & % MFMA peak; 32K decode attn % HBM BW"


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


def setup_prefill(torch, si, nat, wl, device):
    cfg = wl.cfg
    g = torch.Generator(device=device).manual_seed(wl.seed)
    dt = torch.bfloat16
    w = {}
    for name, shape in si.weight_shapes(cfg).items():
        z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        w[name] = ((1 + 0.1 * z) if name in si.GAIN_NAMES else 0.02 * z).to(dt)
    layer = nat.Layer(cfg, w)
    x = torch.randn((wl.batch, wl.seq_len, cfg.hidden_size), generator=g, device=device).to(dt)
    y = torch.empty_like(x)
    cap = wl.seq_len + wl.cached
    kc = torch.zeros((wl.batch, cfg.num_key_value_heads, cap, cfg.head_dim), dtype=dt, device=device)
    vc = torch.zeros_like(kc)
    ws = torch.empty(layer.workspace_size(wl.batch, wl.seq_len, cap), dtype=torch.uint8, device=device)
    return layer, w, x, y, kc, vc, ws


# Seconds of the same step run before its warmup steps.  The board's clocks and power state take
# a fraction of a second to settle under load: with the 10 default warmup steps alone (under 2 ms
# of work) the 0.6B layer's timed steps ran about 8 % slower than after 0.2 s of running.
SETTLE_S = 0.25
settle_seconds = SETTLE_S    # set from --settle


def settle(torch, fn, seconds):
    """Run fn until `seconds` of wall time have passed (untimed); returns the number of runs."""
    t0, n = time.perf_counter(), 0
    while seconds > 0:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
        n += 8
        if time.perf_counter() - t0 >= seconds:
            break
    return n


def time_steps(torch, fn, steps, warmup, settle_s=None):
    settle(torch, fn, settle_seconds if settle_s is None else settle_s)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def profile_steps(torch, layer, fn, steps):
    layer.set_profiling(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    prof = layer.read_profile()
    layer.set_profiling(False)
    return {k: v[1] / v[0] for k, v in prof.items()}     # average ms per launch


# stages that run a GEMM of the table above with more work fused into its epilogue
FUSED_ALIASES = {"gemm_qkv_qknorm_rope": "gemm_qkv"}


def stage_flops(flops, stage):
    return flops.get(stage, flops.get(FUSED_ALIASES.get(stage, ""), None))


def kernel_table(avg_ms, flops):
    out = {}
    for k, ms in avg_ms.items():
        e = {"avg_ms": round(ms, 5)}
        f = stage_flops(flops, k)
        if f is not None:
            tf = f / (ms * 1e-3) / 1e12
            e.update(tflops=round(tf, 1), frac_of_bf16_peak=round(tf / PEAK_BF16_TFLOPS, 4))
        out[k] = e
    return out


def bench_prefill(torch, si, nat, wl, steps, warmup, device):
    layer, w, x, y, kc, vc, ws = setup_prefill(torch, si, nat, wl, device)
    run = lambda: layer.prefill(x, y, kc, vc, ws)
    ms = time_steps(torch, run, steps, warmup)
    avg = profile_steps(torch, layer, run, steps)
    flops = layer_flops(wl.cfg, wl.batch, wl.seq_len)
    total = sum(flops.values())
    res = dict(ms_per_step=ms, tokens_per_s=wl.batch * wl.seq_len / (ms * 1e-3),
               layer_tflops=total / (ms * 1e-3) / 1e12, kernels=kernel_table(avg, flops))
    dominant = max((k for k in avg if stage_flops(flops, k) is not None), key=lambda k: avg[k])
    res["dominant"] = dominant
    res["dominant_flops"] = stage_flops(flops, dominant)
    res["dominant_ms"] = avg[dominant]
    layer.close()
    return res


def bench_decode(torch, si, nat, wl, steps, warmup, device):
    cfg = wl.cfg
    layer, w, x, y, kc, vc, ws = setup_prefill(torch, si, nat, wl, device)
    g = torch.Generator(device=device).manual_seed(wl.seed + 1)
    n = wl.cached
    kc[:, :, :n].copy_(torch.randn(kc[:, :, :n].shape, generator=g, device=device).to(kc.dtype))
    vc[:, :, :n].copy_(torch.randn(vc[:, :, :n].shape, generator=g, device=device).to(vc.dtype))
    lens = [n] * wl.batch
    run = lambda: layer.decode(x, y, lens, kc, vc, ws)
    ms = time_steps(torch, run, steps, warmup)
    avg = profile_steps(torch, layer, run, steps)
    attn_ms = avg["attention_decode_split"]
    byts = decode_attention_bytes(cfg, wl.batch, n)
    gbs = byts / (attn_ms * 1e-3) / 1e9
    layer.close()
    return dict(ms_per_step=ms, tokens_per_s=wl.batch / (ms * 1e-3), attention_ms=attn_ms,
                attention_bytes=byts, attention_gbs=gbs, attention_frac_of_hbm_peak=gbs / PEAK_HBM_GBS,
                kernels={k: {"avg_ms": round(v, 5)} for k, v in avg.items()})


def bench_stack(torch, si, nat, wl, steps, warmup, device):
    """The layer stack with its final RMSNorm: one step runs every layer's prefill in turn, each
    with its own random-init weights and K/V cache, then the final norm (one shared workspace,
    one stream)."""
    cfg = wl.cfg
    dt = torch.bfloat16
    g = torch.Generator(device=device).manual_seed(wl.seed)
    layers, caches = [], []
    for _ in range(wl.layers):
        w = {}
        for name, shape in si.weight_shapes(cfg).items():
            z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
            w[name] = ((1 + 0.1 * z) if name in si.GAIN_NAMES else 0.02 * z).to(dt)
        layers.append((nat.Layer(cfg, w), w))
        kc = torch.zeros((wl.batch, cfg.num_key_value_heads, wl.seq_len, cfg.head_dim), dtype=dt, device=device)
        caches.append((kc, torch.zeros_like(kc)))
    gain = (1 + 0.1 * torch.randn(cfg.hidden_size, generator=g, device=device)).to(dt)
    x = torch.randn((wl.batch, wl.seq_len, cfg.hidden_size), generator=g, device=device).to(dt)
    bufs = (torch.empty_like(x), torch.empty_like(x))
    out = torch.empty_like(x)
    ws = torch.empty(layers[0][0].workspace_size(wl.batch, wl.seq_len, wl.seq_len), dtype=torch.uint8, device=device)

    def run():
        cur = x
        for i, ((layer, _), (kc, vc)) in enumerate(zip(layers, caches)):
            nxt = bufs[i & 1]
            layer.prefill(cur, nxt, kc, vc, ws)
            cur = nxt
        nat.rmsnorm(cur, gain, out, cfg.rms_norm_eps)

    ms = time_steps(torch, run, steps, warmup)
    flops = sum(layer_flops(cfg, wl.batch, wl.seq_len).values()) * wl.layers
    for layer, _ in layers:
        layer.close()
    return dict(ms_per_step=ms, tokens_per_s=wl.batch * wl.seq_len / (ms * 1e-3),
                ms_per_layer=ms / wl.layers, stack_tflops=flops / (ms * 1e-3) / 1e12)


def cpu_baseline(si, wl, min_s=10.0, budget_s=30.0):
    """The float64 oracle, untuned, on a bounded sample of the same workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    cfg = wl.cfg
    w = si.layer_weights(cfg, seed=wl.seed)
    x = si.layer_input(cfg, wl.batch, wl.seq_len, seed=wl.seed)
    t0 = time.perf_counter()
    runs = 0
    while True:
        oracle.layer_prefill(x, w, cfg)
        runs += 1
        el = time.perf_counter() - t0
        if el >= min_s or el * (runs + 1) / runs > budget_s:
            break
    tok_s = runs * wl.batch * wl.seq_len / el
    return {"value": round(tok_s, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{runs} full float64 oracle prefill(s) of the {wl.name} workload "
                      f"(B{wl.batch} x T{wl.seq_len}), {el:.1f} s"}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the 8B prefill, 28-layer stack and 32K decode measurements")
    ap.add_argument("--extra-steps", type=int, default=10, help="timed steps of the 8B prefill / decode runs")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed steps before each workload's warmup steps (clock settling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device-to-device copy 5 times (scale for HBM byte counters)")
    args = ap.parse_args()
    global settle_seconds
    settle_seconds = max(0.0, args.settle)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import seeded_inputs as si
    from transformer_decoder_layer_rmsnorm_amd import _native as nat
    nat.lib()
    device = "cuda:0"
    torch.cuda.set_device(0)

    calib = None
    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        ms = time_steps(torch, lambda: dst.copy_(src), 5, 1)
        calib = {"bytes_read": n, "bytes_written": n, "avg_ms": round(ms, 4),
                 "gbs": round(2 * n / (ms * 1e-3) / 1e9, 1)}
        del src, dst

    wl = si.WORKLOADS["qwen3-0.6b-layer-prefill"]
    print(f"[bench] {wl.name}: {args.warmup} warmup + {args.steps} timed steps", file=sys.stderr, flush=True)
    res = bench_prefill(torch, si, nat, wl, args.steps, args.warmup, device)
    dom_tf = res["dominant_flops"] / (res["dominant_ms"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": settle_seconds,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.seq_len,
                   "hidden_size": wl.cfg.hidden_size, "heads": [wl.cfg.num_attention_heads,
                                                                wl.cfg.num_key_value_heads],
                   "head_dim": wl.cfg.head_dim, "intermediate_size": wl.cfg.intermediate_size},
        "roofline": {"bound": "mfma", "kernel": res["dominant"], "achieved": round(dom_tf, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(dom_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(res["dominant"], wl.name)},
        "layer_tflops": round(res["layer_tflops"], 1),
        "layer_frac_of_bf16_peak": round(res["layer_tflops"] / PEAK_BF16_TFLOPS, 4),
        "kernels": res["kernels"],
    }
    if not args.no_extra:
        wl4 = si.WORKLOADS["qwen3-8b-layer-prefill"]
        print(f"[bench] {wl4.name}", file=sys.stderr, flush=True)
        r4 = bench_prefill(torch, si, nat, wl4, args.extra_steps, 3, device)
        line["qwen3_8b_layer_prefill"] = {
            "tokens_per_s": round(r4["tokens_per_s"], 1), "ms_per_step": round(r4["ms_per_step"], 4),
            "layer_tflops": round(r4["layer_tflops"], 1),
            "layer_frac_of_bf16_peak": round(r4["layer_tflops"] / PEAK_BF16_TFLOPS, 4), "kernels": r4["kernels"]}
        wl3 = si.WORKLOADS["qwen3-0.6b-stack28-prefill"]
        print(f"[bench] {wl3.name}", file=sys.stderr, flush=True)
        r3 = bench_stack(torch, si, nat, wl3, max(2, args.extra_steps // 2), 1, device)
        line["qwen3_0p6b_stack28_prefill"] = {
            "tokens_per_s": round(r3["tokens_per_s"], 1), "ms_per_step": round(r3["ms_per_step"], 4),
            "ms_per_layer": round(r3["ms_per_layer"], 4), "stack_tflops": round(r3["stack_tflops"], 1),
            "stack_frac_of_bf16_peak": round(r3["stack_tflops"] / PEAK_BF16_TFLOPS, 4)}
        wl5 = si.WORKLOADS["qwen3-8b-layer-decode-32k"]
        print(f"[bench] {wl5.name}", file=sys.stderr, flush=True)
        r5 = bench_decode(torch, si, nat, wl5, 2 * args.extra_steps, 5, device)
        line["decode_32k"] = {
            "tokens_per_s": round(r5["tokens_per_s"], 1), "ms_per_step": round(r5["ms_per_step"], 4),
            "roofline": {"bound": "hbm", "kernel": "attention_decode_split", "achieved": round(r5["attention_gbs"], 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(r5["attention_frac_of_hbm_peak"], 4),
                         "traffic": measured_traffic("attention_decode_split", wl5.name)},
            "kernels": r5["kernels"]}
    if calib:
        line["copy_calibration"] = calib
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (float64 oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(si, wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
