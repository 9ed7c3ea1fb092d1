"""ctypes binding of libqwen3layer.so (include/qwen3_layer.h).

Argument marshalling only: every step of the layer runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  torch is imported before the
library is loaded so that the library binds to the HIP runtime torch already loaded
(both carry the soname libamdhip64.so.7), i.e. one runtime and one set of streams.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede loading the library)

from .build import LIB_PATH

QWEN3_OK = 0
QWEN3_ERR_INVALID_ARGUMENT = 1
QWEN3_ERR_UNSUPPORTED = 2
QWEN3_ERR_OUT_OF_RANGE = 3
QWEN3_ERR_WORKSPACE_TOO_SMALL = 4
QWEN3_ERR_DEVICE = 5
QWEN3_F32 = 0
QWEN3_BF16 = 1

EXPORTED = (
    "qwen3_layer_create", "qwen3_layer_destroy", "qwen3_layer_workspace_size",
    "qwen3_layer_workspace_layout", "qwen3_layer_prefill", "qwen3_layer_prefill_at",
    "qwen3_layer_prefill_padded", "qwen3_layer_prefill_window", "qwen3_layer_decode",
    "qwen3_layer_decode_padded", "qwen3_layer_decode_window", "qwen3_layer_decode_noalloc",
    "qwen3_rmsnorm", "qwen3_rmsnorm_gain_offset", "qwen3_layer_set_profiling", "qwen3_layer_read_profile",
    "qwen3_probe_mfma_rate", "qwen3_status_string", "qwen3_last_error",
)

WEIGHT_NAMES = (
    "input_layernorm", "q_proj", "k_proj", "v_proj", "q_norm", "k_norm", "o_proj",
    "post_attention_layernorm", "gate_proj", "up_proj", "down_proj",
)


class Config(ctypes.Structure):
    _fields_ = [
        ("hidden_size", ctypes.c_int32), ("num_attention_heads", ctypes.c_int32),
        ("num_key_value_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("intermediate_size", ctypes.c_int32), ("max_position_embeddings", ctypes.c_int32),
        ("rope_theta", ctypes.c_double), ("rms_norm_eps", ctypes.c_float), ("dtype", ctypes.c_int),
        ("rotary_dim", ctypes.c_int32), ("rope_adjacent_pairs", ctypes.c_int32),
        ("rope_position_scale", ctypes.c_double), ("norm_unit_offset", ctypes.c_int32),
    ]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_NAMES]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("h", "qkv", "qhat", "attn", "x1", "h2", "act", "part_gemm", "lens", "part_o", "part_ml", "total")] + \
               [("decode_splits", ctypes.c_int32), ("split_keys", ctypes.c_int32)]


class StageTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


class Qwen3Error(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(or python -m transformer_decoder_layer_rmsnorm_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    sig = {
        "qwen3_layer_create": ([ctypes.POINTER(Config), ctypes.POINTER(Weights), ctypes.POINTER(P)], ctypes.c_int),
        "qwen3_layer_destroy": ([P], None),
        "qwen3_layer_workspace_size": ([P, I32, I32, I32, ctypes.POINTER(SZ)], ctypes.c_int),
        "qwen3_layer_workspace_layout": ([P, I32, I32, I32, ctypes.POINTER(WorkspaceLayout)], ctypes.c_int),
        "qwen3_layer_prefill": ([P, P, P, I32, I32, P, P, I32, P, SZ, P], ctypes.c_int),
        "qwen3_layer_prefill_at": ([P, P, P, I32, I32, ctypes.POINTER(I32), P, P, I32, P, SZ, P], ctypes.c_int),
        "qwen3_layer_prefill_padded": ([P, P, P, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32), P, P, I32, P,
                                        SZ, P], ctypes.c_int),
        "qwen3_layer_prefill_window": ([P, P, P, I32, I32, ctypes.POINTER(I32), I32, I32, P, P, I32, P, SZ, P],
                                       ctypes.c_int),
        "qwen3_layer_decode_window": ([P, P, P, I32, ctypes.POINTER(I32), I32, I32, I32, P, P, I32, P, SZ, P],
                                      ctypes.c_int),
        "qwen3_layer_decode": ([P, P, P, I32, ctypes.POINTER(I32), P, P, I32, P, SZ, P], ctypes.c_int),
        "qwen3_layer_decode_padded": ([P, P, P, I32, ctypes.POINTER(I32), ctypes.POINTER(I32), ctypes.POINTER(I32),
                                       P, P, I32, P, SZ, P], ctypes.c_int),
        "qwen3_layer_decode_noalloc": ([P, P, P, I32, ctypes.POINTER(I32), P, P, I32, P], ctypes.c_int),
        "qwen3_rmsnorm": ([P, P, P, I64, I32, F32, ctypes.c_int, P], ctypes.c_int),
        "qwen3_rmsnorm_gain_offset": ([P, P, P, I64, I32, F32, F32, ctypes.c_int, P], ctypes.c_int),
        "qwen3_layer_set_profiling": ([P, I32], ctypes.c_int),
        "qwen3_probe_mfma_rate": ([P, I32, I32, P], ctypes.c_int),
        "qwen3_layer_read_profile": ([P, ctypes.POINTER(StageTime), I32, ctypes.POINTER(I32)], ctypes.c_int),
        "qwen3_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "qwen3_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def check(status: int, what: str) -> None:
    if status != QWEN3_OK:
        L = lib()
        msg = L.qwen3_last_error().decode()
        raise Qwen3Error(status, f"{what}: {L.qwen3_status_string(status).decode()}: {msg}")


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_config(cfg) -> Config:
    """cfg: any object with the config.json field names (e.g. seeded_inputs.LayerConfig)."""
    return Config(cfg.hidden_size, cfg.num_attention_heads, cfg.num_key_value_heads, cfg.head_dim,
                  cfg.intermediate_size, cfg.max_position_embeddings, float(cfg.rope_theta),
                  float(cfg.rms_norm_eps), QWEN3_BF16 if cfg.dtype == "bf16" else QWEN3_F32,
                  int(getattr(cfg, "rotary_dim", 0)), 1 if getattr(cfg, "rope_adjacent_pairs", False) else 0,
                  float(getattr(cfg, "rope_position_scale", 1.0)),
                  1 if getattr(cfg, "norm_unit_offset", False) else 0)


class Layer:
    """One decoder layer bound to device weights (the tensors must outlive the layer)."""

    def __init__(self, cfg, weights: dict):
        self.cfg = cfg
        self._weights = dict(weights)          # keep the tensors alive
        self._c = make_config(cfg)
        w = Weights(*[_ptr(weights[n]) for n in WEIGHT_NAMES])
        handle = ctypes.c_void_p()
        check(lib().qwen3_layer_create(ctypes.byref(self._c), ctypes.byref(w), ctypes.byref(handle)),
              "qwen3_layer_create")
        self._h = handle

    def close(self):
        if getattr(self, "_h", None):
            lib().qwen3_layer_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self, batch: int, seq_len: int, cache_capacity: int = 0) -> int:
        n = ctypes.c_size_t()
        check(lib().qwen3_layer_workspace_size(self._h, batch, seq_len, cache_capacity, ctypes.byref(n)),
              "qwen3_layer_workspace_size")
        return n.value

    def workspace_layout(self, batch: int, seq_len: int, cache_capacity: int = 0) -> WorkspaceLayout:
        out = WorkspaceLayout()
        check(lib().qwen3_layer_workspace_layout(self._h, batch, seq_len, cache_capacity, ctypes.byref(out)),
              "qwen3_layer_workspace_layout")
        return out

    def prefill(self, x, y, k_cache, v_cache, workspace, stream=None, start_positions=None, pad_lens=None) -> None:
        """Prefill; with start_positions (one int per sequence) the tokens continue a cache that
        already holds that many keys and values (qwen3_layer_prefill_at); with pad_lens the first
        pad_lens[b] tokens of sequence b are left padding (qwen3_layer_prefill_padded)."""
        b, t = x.shape[0], x.shape[1]
        nbytes = workspace.numel() * workspace.element_size()
        if pad_lens is not None:
            starts = None if start_positions is None else (ctypes.c_int32 * b)(*[int(v) for v in start_positions])
            pads = (ctypes.c_int32 * b)(*[int(v) for v in pad_lens])
            check(lib().qwen3_layer_prefill_padded(self._h, _ptr(x), _ptr(y), b, t, starts, pads, _ptr(k_cache),
                                                   _ptr(v_cache), k_cache.shape[2], _ptr(workspace), nbytes,
                                                   _stream(stream)), "qwen3_layer_prefill_padded")
        elif start_positions is None:
            check(lib().qwen3_layer_prefill(self._h, _ptr(x), _ptr(y), b, t, _ptr(k_cache), _ptr(v_cache),
                                            k_cache.shape[2], _ptr(workspace), nbytes, _stream(stream)),
                  "qwen3_layer_prefill")
        else:
            starts = (ctypes.c_int32 * b)(*[int(v) for v in start_positions])
            check(lib().qwen3_layer_prefill_at(self._h, _ptr(x), _ptr(y), b, t, starts, _ptr(k_cache),
                                               _ptr(v_cache), k_cache.shape[2], _ptr(workspace), nbytes,
                                               _stream(stream)), "qwen3_layer_prefill_at")

    def decode(self, x, y, cache_lens, k_cache, v_cache, workspace, stream=None, pad_starts=None,
               pad_lens=None) -> None:
        """One token per sequence; with pad_starts / pad_lens, the cache slots
        [pad_starts[b], pad_starts[b] + pad_lens[b]) are left padding (qwen3_layer_decode_padded)."""
        b = x.shape[0]
        lens = (ctypes.c_int32 * b)(*[int(v) for v in cache_lens])
        nbytes = workspace.numel() * workspace.element_size()
        if pad_lens is not None or pad_starts is not None:
            starts = None if pad_starts is None else (ctypes.c_int32 * b)(*[int(v) for v in pad_starts])
            pads = None if pad_lens is None else (ctypes.c_int32 * b)(*[int(v) for v in pad_lens])
            check(lib().qwen3_layer_decode_padded(self._h, _ptr(x), _ptr(y), b, lens, starts, pads, _ptr(k_cache),
                                                  _ptr(v_cache), k_cache.shape[2], _ptr(workspace), nbytes,
                                                  _stream(stream)), "qwen3_layer_decode_padded")
            return
        check(lib().qwen3_layer_decode(self._h, _ptr(x), _ptr(y), b, lens, _ptr(k_cache), _ptr(v_cache),
                                       k_cache.shape[2], _ptr(workspace), nbytes, _stream(stream)),
              "qwen3_layer_decode")

    def decode_noalloc(self, x, y, cache_lens, k_cache, v_cache, stream=None) -> None:
        """One token per sequence with the intermediates in the library's static device array
        (qwen3_layer_decode_noalloc): no workspace, nothing allocated."""
        b = x.shape[0]
        lens = (ctypes.c_int32 * b)(*[int(v) for v in cache_lens])
        check(lib().qwen3_layer_decode_noalloc(self._h, _ptr(x), _ptr(y), b, lens, _ptr(k_cache), _ptr(v_cache),
                                               k_cache.shape[2], _stream(stream)), "qwen3_layer_decode_noalloc")

    def prefill_window(self, x, y, k_cache, v_cache, workspace, window, sinks=0, start_positions=None,
                       stream=None) -> None:
        """Prefill of a local layer: banded mask of `window` tokens plus `sinks` attention sinks
        (qwen3_layer_prefill_window)."""
        b, t = x.shape[0], x.shape[1]
        starts = None if start_positions is None else (ctypes.c_int32 * b)(*[int(v) for v in start_positions])
        check(lib().qwen3_layer_prefill_window(self._h, _ptr(x), _ptr(y), b, t, starts, int(window), int(sinks),
                                               _ptr(k_cache), _ptr(v_cache), k_cache.shape[2], _ptr(workspace),
                                               workspace.numel() * workspace.element_size(), _stream(stream)),
              "qwen3_layer_prefill_window")

    def decode_window(self, x, y, positions, k_cache, v_cache, workspace, window, sinks=0, rolling=False,
                      stream=None) -> None:
        """Decode of a local layer on a linear cache or a rolling buffer (qwen3_layer_decode_window)."""
        b = x.shape[0]
        pos = (ctypes.c_int32 * b)(*[int(v) for v in positions])
        check(lib().qwen3_layer_decode_window(self._h, _ptr(x), _ptr(y), b, pos, int(window), int(sinks),
                                              1 if rolling else 0, _ptr(k_cache), _ptr(v_cache), k_cache.shape[2],
                                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                                              _stream(stream)), "qwen3_layer_decode_window")

    def set_profiling(self, enabled: bool) -> None:
        check(lib().qwen3_layer_set_profiling(self._h, 1 if enabled else 0), "qwen3_layer_set_profiling")

    def read_profile(self) -> dict:
        buf = (StageTime * 32)()
        n = ctypes.c_int32()
        check(lib().qwen3_layer_read_profile(self._h, buf, 32, ctypes.byref(n)), "qwen3_layer_read_profile")
        return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(n.value)}


def probe_mfma_rate(out, workgroups: int, iterations: int, stream=None) -> None:
    """Matrix-core rate probe (qwen3_probe_mfma_rate): out is a float32 CUDA tensor of at least
    workgroups * 256 elements."""
    if out.dtype != torch.float32 or out.numel() < workgroups * 256 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor of at least workgroups * 256 elements")
    check(lib().qwen3_probe_mfma_rate(_ptr(out), int(workgroups), int(iterations), _stream(stream)),
          "qwen3_probe_mfma_rate")


def rmsnorm(x, weight, y, eps: float, stream=None, gain_offset: float = 0.0) -> None:
    width = x.shape[-1]
    rows = x.numel() // width
    dtype = QWEN3_BF16 if x.dtype == torch.bfloat16 else QWEN3_F32
    if gain_offset:
        check(lib().qwen3_rmsnorm_gain_offset(_ptr(x), _ptr(weight), _ptr(y), rows, width, float(eps),
                                              float(gain_offset), dtype, _stream(stream)), "qwen3_rmsnorm_gain_offset")
        return
    check(lib().qwen3_rmsnorm(_ptr(x), _ptr(weight), _ptr(y), rows, width, float(eps), dtype, _stream(stream)),
          "qwen3_rmsnorm")
