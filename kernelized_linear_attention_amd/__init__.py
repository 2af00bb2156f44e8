"""Causal SLAY attention (Spherical Linearized Attention with Yat kernels) on
AMD Instinct MI355X: hand-written HIP kernels for gfx950 behind the C ABI in
include/slay.h, with a thin PyTorch binding (``kernelized_linear_attention_amd.ops``)
for device memory and streams.
"""
from ._lib import LIB_PATH, SlayError, load  # noqa: F401

__all__ = ["LIB_PATH", "SlayError", "load"]
