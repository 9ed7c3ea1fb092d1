"""Qwen3-style pre-norm decoder layer (prefill and decode) on AMD Instinct MI355X.

The layer runs in hand-written gfx950 HIP kernels behind the C ABI of
include/qwen3_layer.h; this package is its thin Python binding.
"""
from ._native import Layer, Qwen3Error, lib, rmsnorm  # noqa: F401
