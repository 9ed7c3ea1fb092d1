"""The allocation-free decode entry point (qwen3_layer_decode_noalloc) against the workspace
decode (qwen3_layer_decode) on the 8B-shaped layer: same kernels and launch shapes, so the
outputs and the new cache slots must be bit-identical.  Two calls in a row, the second on a
smaller input, so the second runs on what the first left in the library's scratch array."""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from gpu_support import GpuLayer, assert_bf16_parity, log, to_dev, to_np

pytestmark = pytest.mark.gpu


def _seeded_cache(cfg, lens, cap, seed):
    b, hkv, d = len(lens), cfg.num_key_value_heads, cfg.head_dim
    kc = np.zeros((b, hkv, cap, d), np.float32)
    vc = np.zeros((b, hkv, cap, d), np.float32)

    def sink(i, h, kb, vb):
        kc[i, h, :lens[i]] = kb
        vc[i, h, :lens[i]] = vb

    si.fill_decode_cache(cfg, b, lens, sink, seed=seed)
    return kc, vc


def _compare(gl, lens, cap, seed, oracle_rows=2):
    cfg = gl.cfg
    b = len(lens)
    log(f"decode_noalloc vs decode: B{b}, capacity {cap}, lengths {min(lens)}..{max(lens)}")
    kc, vc = _seeded_cache(cfg, lens, cap, seed)
    k1, v1 = to_dev(kc, cfg), to_dev(vc, cfg)
    k2, v2 = k1.clone(), v1.clone()
    x = si.layer_input(cfg, b, 1, seed=seed)
    xd = to_dev(x, cfg)
    y_ref, _ = gl.decode(xd, lens, k1, v1)
    y = torch.empty_like(xd)
    gl.layer.decode_noalloc(xd, y, lens, k2, v2)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref), "outputs differ from the workspace decode"
    assert torch.equal(k1, k2) and torch.equal(v1, v2), "new cache slots differ from the workspace decode"
    # and the oracle on a few of the rows (the first sequences' caches as the GPU holds them)
    rows = list(range(min(oracle_rows, b)))
    ref, _, _ = oracle.layer_decode(x[rows], gl.w_np, cfg, kc[rows], vc[rows], [lens[i] for i in rows])
    assert_bf16_parity(to_np(y)[rows], ref, f"decode_noalloc rows {rows} vs oracle")


def test_decode_noalloc_equals_workspace_decode_two_calls():
    cfg = si.QWEN3_8B
    gl = GpuLayer.seeded(cfg, seed=21)
    rng = np.random.default_rng(21)
    # first call: 70 sequences (over 64: the lengths go through the scratch array's lens region)
    lens1 = [int(v) for v in rng.integers(0, 1500, 70)]
    lens1[:4] = [0, 1, 511, 1499]
    _compare(gl, lens1, 1500, 21)
    # second call, smaller: 3 sequences over 700 slots
    _compare(gl, [600, 5, 699], 700, 22)
