"""Gated ReLU linear-attention token mixer for AMD MI355X (gfx950).

The compute path is the HIP library ``libgla.so`` (C ABI declared in
``include/gla.h``); :mod:`relu_linear_attention_amd.gla` is its thin ctypes
binding.  Nothing is loaded at import time.
"""
__all__ = ["gla", "inputs"]
