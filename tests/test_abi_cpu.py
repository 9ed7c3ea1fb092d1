"""The C ABI without a GPU: the library loads, exports every function include/*.h declares,
and every validation error is returned on the host before anything is launched.
Only host-side paths are exercised here (no kernel is ever launched)."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

import seeded_inputs as si
from transformer_decoder_layer_rmsnorm_amd import _native as nat

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000        # an aligned, never dereferenced stand-in for a device pointer


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(qwen3_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 10
    L = nat.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", nat.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (qwen3_\w+)$", out, flags=re.M))
    assert set(names) <= exported
    assert set(nat.EXPORTED) == set(names)


def fake_weights():
    return nat.Weights(*[FAKE] * len(nat.WEIGHT_NAMES))


def create(cfg, weights=None):
    c = nat.make_config(cfg)
    h = ctypes.c_void_p()
    st = nat.lib().qwen3_layer_create(ctypes.byref(c), ctypes.byref(weights or fake_weights()), ctypes.byref(h))
    return st, h


def err():
    return nat.lib().qwen3_last_error().decode()


@pytest.mark.parametrize("change,status", [
    (dict(head_dim=31), nat.QWEN3_ERR_INVALID_ARGUMENT),            # odd: no rotate-half pairing
    (dict(hidden_size=0), nat.QWEN3_ERR_INVALID_ARGUMENT),
    (dict(num_key_value_heads=-1), nat.QWEN3_ERR_INVALID_ARGUMENT),
    (dict(rope_theta=0.0), nat.QWEN3_ERR_INVALID_ARGUMENT),
    (dict(rms_norm_eps=-1e-6), nat.QWEN3_ERR_INVALID_ARGUMENT),
    (dict(num_attention_heads=6, num_key_value_heads=4), nat.QWEN3_ERR_UNSUPPORTED),  # Hq % Hkv
    (dict(hidden_size=60), nat.QWEN3_ERR_UNSUPPORTED),
    (dict(head_dim=256), nat.QWEN3_ERR_UNSUPPORTED),
    (dict(rotary_dim=31), nat.QWEN3_ERR_INVALID_ARGUMENT),          # odd rotated width
    (dict(rotary_dim=34), nat.QWEN3_ERR_INVALID_ARGUMENT),          # wider than head_dim 32
    (dict(rope_position_scale=-0.5), nat.QWEN3_ERR_INVALID_ARGUMENT),
    (dict(rope_position_scale=float("inf")), nat.QWEN3_ERR_INVALID_ARGUMENT),
])
def test_create_rejects_bad_f32_configs(change, status):
    cfg = si.LayerConfig(**{**si.TINY_F32.__dict__, **change})
    st, h = create(cfg)
    assert st == status, err()
    assert not h.value


@pytest.mark.parametrize("change,status", [
    (dict(head_dim=64), nat.QWEN3_ERR_UNSUPPORTED),
    (dict(intermediate_size=3000), nat.QWEN3_ERR_UNSUPPORTED),
    (dict(num_attention_heads=48, num_key_value_heads=2), nat.QWEN3_ERR_UNSUPPORTED),  # g = 24
])
def test_create_rejects_unsupported_bf16_configs(change, status):
    cfg = si.LayerConfig(**{**si.QWEN3_0P6B.__dict__, **change})
    st, _ = create(cfg)
    assert st == status, err()


def test_create_accepts_rope_and_norm_variants():
    for change in [dict(rotary_dim=16), dict(rope_adjacent_pairs=True), dict(rope_position_scale=0.25),
                   dict(norm_unit_offset=True), dict(rotary_dim=0)]:
        cfg = si.LayerConfig(**{**si.TINY_F32.__dict__, **change})
        st, h = create(cfg)
        assert st == nat.QWEN3_OK, (change, err())
        nat.lib().qwen3_layer_destroy(h)
    c = nat.make_config(si.TINY_F32)
    c.rope_adjacent_pairs = 2
    h = ctypes.c_void_p()
    assert nat.lib().qwen3_layer_create(ctypes.byref(c), ctypes.byref(fake_weights()), ctypes.byref(h)) \
        == nat.QWEN3_ERR_INVALID_ARGUMENT


def test_create_accepts_bf16_hidden_above_4096():
    """hidden 5120 (a family width): every bf16 kernel has a form for rows over 4096 wide, so
    create and workspace sizing accept it (the kernels themselves run in the GPU tests)."""
    cfg = si.LayerConfig(**{**si.QWEN3_0P6B.__dict__, "hidden_size": 5120, "num_attention_heads": 64,
                            "intermediate_size": 25600})
    st, h = create(cfg)
    assert st == nat.QWEN3_OK, err()
    n = ctypes.c_size_t()
    assert nat.lib().qwen3_layer_workspace_size(h, 1, 2048, 2048, ctypes.byref(n)) == nat.QWEN3_OK, err()
    assert n.value >= 2048 * 5120 * (2 + 4 + 2)
    nat.lib().qwen3_layer_destroy(h)


def test_create_rejects_null_and_misaligned_weights():
    w = fake_weights()
    w.q_norm = None
    assert create(si.QWEN3_0P6B, w)[0] == nat.QWEN3_ERR_INVALID_ARGUMENT
    w = fake_weights()
    w.down_proj = FAKE + 2
    assert create(si.QWEN3_0P6B, w)[0] == nat.QWEN3_ERR_INVALID_ARGUMENT
    c = nat.make_config(si.QWEN3_0P6B)
    assert nat.lib().qwen3_layer_create(ctypes.byref(c), None, None) == nat.QWEN3_ERR_INVALID_ARGUMENT


@pytest.fixture
def layer():
    st, h = create(si.QWEN3_0P6B)
    assert st == nat.QWEN3_OK, err()
    yield h
    nat.lib().qwen3_layer_destroy(h)


def test_workspace_size_and_layout(layer):
    L = nat.lib()
    n = ctypes.c_size_t()
    assert L.qwen3_layer_workspace_size(layer, 1, 2048, 2048, ctypes.byref(n)) == nat.QWEN3_OK
    lay = nat.WorkspaceLayout()
    assert L.qwen3_layer_workspace_layout(layer, 1, 2048, 2048, ctypes.byref(lay)) == nat.QWEN3_OK
    m, h, i = 2048, 1024, 3072
    # regions in order, 256-byte aligned, each large enough
    offs = [lay.h, lay.qkv, lay.qhat, lay.attn, lay.x1, lay.h2, lay.act]
    sizes = [m * h * 2, m * 4096 * 2, m * 2048 * 2, m * 2048 * 2, m * h * 4, m * h * 2, m * i * 2]
    for k in range(len(offs)):
        assert offs[k] % 256 == 0
        if k + 1 < len(offs):
            assert offs[k + 1] - offs[k] >= sizes[k]
    assert n.value >= lay.act + sizes[-1]
    assert lay.decode_splits == -(-2048 // lay.split_keys)
    assert L.qwen3_layer_workspace_size(layer, 0, 5, 5, ctypes.byref(n)) == nat.QWEN3_ERR_INVALID_ARGUMENT


def test_workspace_split_k_slabs_only_for_few_output_tiles(layer):
    """0.6B-shaped o_proj and down (N = 1024, K = 2048 and 3072): at 2048 tokens the deep-ring GEMM
    (at least 128 tiles of 64 x 128) covers them with K unsplit, so the layout holds no fp32 partial
    slabs; at 300 tokens (40 such tiles) K is split in two and the [2, M, H] slabs are there."""
    L = nat.lib()
    for t, slabs in ((2048, 0), (300, 2)):
        lay = nat.WorkspaceLayout()
        assert L.qwen3_layer_workspace_layout(layer, 1, t, t, ctypes.byref(lay)) == nat.QWEN3_OK
        region = lay.lens - lay.part_gemm
        assert region >= slabs * t * 1024 * 4
        assert region < (slabs * t * 1024 * 4) + 256, (t, region)


def prefill(layer, b=1, t=16, cap=16, ws_bytes=1 << 30, x=FAKE, kc=FAKE):
    return nat.lib().qwen3_layer_prefill(layer, x, FAKE, b, t, kc, FAKE, cap, FAKE, ws_bytes, None)


def test_prefill_validation_before_launch(layer):
    assert prefill(layer, t=17, cap=16) == nat.QWEN3_ERR_OUT_OF_RANGE           # T > capacity
    assert prefill(layer, t=40961, cap=50000) == nat.QWEN3_ERR_OUT_OF_RANGE     # T > max positions
    assert prefill(layer, ws_bytes=1000) == nat.QWEN3_ERR_WORKSPACE_TOO_SMALL
    assert prefill(layer, x=None) == nat.QWEN3_ERR_INVALID_ARGUMENT
    assert prefill(layer, kc=FAKE + 8) == nat.QWEN3_ERR_INVALID_ARGUMENT
    assert prefill(layer, b=0) == nat.QWEN3_ERR_INVALID_ARGUMENT
    assert prefill(layer, t=-3) == nat.QWEN3_ERR_INVALID_ARGUMENT


def decode(layer, lens, cap=64, ws_bytes=1 << 30):
    arr = (ctypes.c_int32 * len(lens))(*lens)
    return nat.lib().qwen3_layer_decode(layer, FAKE, FAKE, len(lens), arr, FAKE, FAKE, cap, FAKE, ws_bytes, None)


def test_decode_validation_before_launch(layer):
    assert decode(layer, [10, 64]) == nat.QWEN3_ERR_OUT_OF_RANGE       # no free slot
    assert decode(layer, [10, -1]) == nat.QWEN3_ERR_OUT_OF_RANGE
    assert decode(layer, [40960], cap=50000) == nat.QWEN3_ERR_OUT_OF_RANGE   # position limit
    assert decode(layer, [3, 4], ws_bytes=100) == nat.QWEN3_ERR_WORKSPACE_TOO_SMALL
    assert nat.lib().qwen3_layer_decode(layer, FAKE, FAKE, 1, None, FAKE, FAKE, 8, FAKE, 1 << 30, None) \
        == nat.QWEN3_ERR_INVALID_ARGUMENT


def prefill_at(layer, starts, t=4, cap=16, ws_bytes=1 << 30):
    arr = None if starts is None else (ctypes.c_int32 * len(starts))(*starts)
    b = 1 if starts is None else len(starts)
    return nat.lib().qwen3_layer_prefill_at(layer, FAKE, FAKE, b, t, arr, FAKE, FAKE, cap, FAKE, ws_bytes, None)


def test_prefill_at_validation_before_launch(layer):
    assert prefill_at(layer, [0, -1]) == nat.QWEN3_ERR_OUT_OF_RANGE           # negative start
    assert prefill_at(layer, [12, 13]) == nat.QWEN3_ERR_OUT_OF_RANGE          # 13 + 4 > capacity 16
    assert prefill_at(layer, [40958], cap=50000) == nat.QWEN3_ERR_OUT_OF_RANGE  # passes the position limit
    assert prefill_at(layer, [3, 4], ws_bytes=100) == nat.QWEN3_ERR_WORKSPACE_TOO_SMALL
    # more than 64 sequences with starts: the positions need the workspace's `lens` region too
    lay = nat.WorkspaceLayout()
    assert nat.lib().qwen3_layer_workspace_layout(layer, 65, 4, 0, ctypes.byref(lay)) == nat.QWEN3_OK
    assert prefill_at(layer, [1] * 65, ws_bytes=lay.lens) == nat.QWEN3_ERR_WORKSPACE_TOO_SMALL
    size = ctypes.c_size_t()
    assert nat.lib().qwen3_layer_workspace_size(layer, 65, 4, 0, ctypes.byref(size)) == nat.QWEN3_OK
    assert size.value >= lay.lens + 65 * 4
    assert nat.lib().qwen3_layer_prefill_at(layer, None, FAKE, 1, 4, None, FAKE, FAKE, 16, FAKE, 1 << 30, None) \
        == nat.QWEN3_ERR_INVALID_ARGUMENT



def prefill_padded(layer, pads, starts=None, t=4, cap=16, ws_bytes=1 << 30):
    b = len(pads)
    sa = None if starts is None else (ctypes.c_int32 * b)(*starts)
    pa = (ctypes.c_int32 * b)(*pads)
    return nat.lib().qwen3_layer_prefill_padded(layer, FAKE, FAKE, b, t, sa, pa, FAKE, FAKE, cap, FAKE, ws_bytes,
                                                None)


def test_prefill_padded_validation_before_launch(layer):
    assert prefill_padded(layer, [0, -1]) == nat.QWEN3_ERR_OUT_OF_RANGE         # negative padding
    assert prefill_padded(layer, [5]) == nat.QWEN3_ERR_OUT_OF_RANGE             # more padding than tokens
    assert prefill_padded(layer, [1], starts=[13]) == nat.QWEN3_ERR_OUT_OF_RANGE   # 13 + 4 > 16
    assert prefill_padded(layer, [1, 2], ws_bytes=100) == nat.QWEN3_ERR_WORKSPACE_TOO_SMALL
    # more than 64 padded sequences: the per-sequence values go through the `lens` region
    lay = nat.WorkspaceLayout()
    assert nat.lib().qwen3_layer_workspace_layout(layer, 65, 4, 0, ctypes.byref(lay)) == nat.QWEN3_OK
    assert prefill_padded(layer, [1] * 65, ws_bytes=lay.lens) == nat.QWEN3_ERR_WORKSPACE_TOO_SMALL
    assert lay.part_o - lay.lens >= 3 * 65 * 4


def decode_padded(layer, lens, pad_starts, pad_lens, cap=64, ws_bytes=1 << 30):
    b = len(lens)
    la = (ctypes.c_int32 * b)(*lens)
    sa = None if pad_starts is None else (ctypes.c_int32 * b)(*pad_starts)
    pa = None if pad_lens is None else (ctypes.c_int32 * b)(*pad_lens)
    return nat.lib().qwen3_layer_decode_padded(layer, FAKE, FAKE, b, la, sa, pa, FAKE, FAKE, cap, FAKE, ws_bytes,
                                               None)


def test_decode_padded_validation_before_launch(layer):
    assert decode_padded(layer, [10], [0], None) == nat.QWEN3_ERR_INVALID_ARGUMENT     # one array only
    assert decode_padded(layer, [10], [4], [7]) == nat.QWEN3_ERR_OUT_OF_RANGE          # run past the cache
    assert decode_padded(layer, [10], [-1], [2]) == nat.QWEN3_ERR_OUT_OF_RANGE
    assert decode_padded(layer, [10], [0], [-2]) == nat.QWEN3_ERR_OUT_OF_RANGE
    assert decode_padded(layer, [10, 64], [0, 0], [1, 1]) == nat.QWEN3_ERR_OUT_OF_RANGE   # no free slot
    assert decode_padded(layer, [10], [0], [3], ws_bytes=100) == nat.QWEN3_ERR_WORKSPACE_TOO_SMALL



def test_window_entry_points_validation_before_launch(layer):
    L = nat.lib()
    # negative window or sinks
    assert L.qwen3_layer_prefill_window(layer, FAKE, FAKE, 1, 4, None, -1, 0, FAKE, FAKE, 16, FAKE, 1 << 30,
                                        None) == nat.QWEN3_ERR_INVALID_ARGUMENT
    assert L.qwen3_layer_prefill_window(layer, FAKE, FAKE, 1, 4, None, 8, -2, FAKE, FAKE, 16, FAKE, 1 << 30,
                                        None) == nat.QWEN3_ERR_INVALID_ARGUMENT
    # the banded prefill keeps the linear-cache rules
    assert L.qwen3_layer_prefill_window(layer, FAKE, FAKE, 1, 17, None, 8, 0, FAKE, FAKE, 16, FAKE, 1 << 30,
                                        None) == nat.QWEN3_ERR_OUT_OF_RANGE

    def dec(pos, window, sinks, rolling, cap, ws_bytes=1 << 30):
        arr = (ctypes.c_int32 * len(pos))(*pos)
        return L.qwen3_layer_decode_window(layer, FAKE, FAKE, len(pos), arr, window, sinks, rolling, FAKE, FAKE, cap,
                                           FAKE, ws_bytes, None)

    assert dec([5], 0, 0, 1, 8) == nat.QWEN3_ERR_INVALID_ARGUMENT          # rolling without a window
    assert dec([5], 8, 2, 1, 8) == nat.QWEN3_ERR_INVALID_ARGUMENT          # buffer is sinks + window = 10
    assert dec([5], 8, -1, 0, 64) == nat.QWEN3_ERR_INVALID_ARGUMENT
    assert dec([64], 8, 2, 0, 64) == nat.QWEN3_ERR_OUT_OF_RANGE            # linear cache: no free slot
    assert dec([40960], 8, 2, 1, 10) == nat.QWEN3_ERR_OUT_OF_RANGE         # position limit
    assert dec([100], 8, 2, 1, 10, ws_bytes=100) == nat.QWEN3_ERR_WORKSPACE_TOO_SMALL   # past the capacity is fine


def test_rmsnorm_validation_and_status_strings():
    L = nat.lib()
    assert L.qwen3_rmsnorm(FAKE, FAKE, FAKE, 4, 12, 1e-6, nat.QWEN3_BF16, None) == nat.QWEN3_ERR_UNSUPPORTED
    assert L.qwen3_rmsnorm(None, FAKE, FAKE, 4, 16, 1e-6, nat.QWEN3_BF16, None) == nat.QWEN3_ERR_INVALID_ARGUMENT
    assert L.qwen3_rmsnorm(FAKE, FAKE, FAKE, 0, 16, 1e-6, nat.QWEN3_BF16, None) == nat.QWEN3_ERR_INVALID_ARGUMENT
    assert L.qwen3_rmsnorm_gain_offset(FAKE, FAKE, FAKE, 4, 12, 1e-6, 1.0, nat.QWEN3_BF16, None) \
        == nat.QWEN3_ERR_UNSUPPORTED
    assert L.qwen3_rmsnorm_gain_offset(FAKE, FAKE, FAKE, 4, 16, 1e-6, float("nan"), nat.QWEN3_BF16, None) \
        == nat.QWEN3_ERR_INVALID_ARGUMENT
    for s in range(6):
        assert L.qwen3_status_string(s)
    assert "unknown" in L.qwen3_status_string(99).decode()


def test_python_binding_raises_with_message():
    with pytest.raises(nat.Qwen3Error) as e:
        nat.check(nat.QWEN3_ERR_OUT_OF_RANGE, "probe")
    assert e.value.status == nat.QWEN3_ERR_OUT_OF_RANGE


def test_decode_noalloc_rejects_before_any_device_call(layer):
    """The allocation-free decode validates on the host first: a decode too large for its
    32 MiB scratch array, bad lengths and NULL pointers are refused before the array is looked
    up on a device (there is none here)."""
    L = nat.lib()
    lens = (ctypes.c_int32 * 64)(*([32768] * 64))
    # 64 sequences over 65537 cache slots: 65 key splits of 1024, about 34 MB of partials
    st = L.qwen3_layer_decode_noalloc(layer, FAKE, FAKE, 64, lens, FAKE, FAKE, 65537, None)
    assert st == nat.QWEN3_ERR_WORKSPACE_TOO_SMALL, err()
    assert "32 MiB" in err() or "bytes of scratch" in err()
    one = (ctypes.c_int32 * 1)(5)
    assert L.qwen3_layer_decode_noalloc(layer, None, FAKE, 1, one, FAKE, FAKE, 16, None) == \
        nat.QWEN3_ERR_INVALID_ARGUMENT
    assert L.qwen3_layer_decode_noalloc(layer, FAKE, FAKE, 0, one, FAKE, FAKE, 16, None) == \
        nat.QWEN3_ERR_INVALID_ARGUMENT


def test_mfma_probe_rejects_bad_arguments_before_any_launch():
    L = nat.lib()
    assert L.qwen3_probe_mfma_rate(None, 4, 4, None) == nat.QWEN3_ERR_INVALID_ARGUMENT
    assert "non-NULL" in err()
    for wg, it in [(0, 4), (4, 0), (-1, 4)]:
        assert L.qwen3_probe_mfma_rate(FAKE, wg, it, None) == nat.QWEN3_ERR_INVALID_ARGUMENT
        assert "positive" in err()
