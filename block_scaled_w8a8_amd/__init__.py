"""block_scaled_w8a8_amd — block-scaled W8A8 (e4m3fn / int8) linear layer for MI355X (gfx950).

The computation lives in libbfq.so (hand-written HIP kernels behind the C-ABI of
include/bfq.h); ``block_scaled_w8a8_amd.bfq`` is its ctypes binding. Importing the package
itself loads nothing, so the input generators (``synth``) and the metric helpers (``perf``)
work on machines without the built library; touching any binding name loads libbfq.so and
raises ImportError if it is missing.
"""
from __future__ import annotations

import importlib

__all__ = ["bfq", "synth", "perf"]


def __getattr__(name):
    if name in ("bfq", "synth", "perf", "build", "sweep"):
        return importlib.import_module(f"{__name__}.{name}")
    mod = importlib.import_module(f"{__name__}.bfq")
    if hasattr(mod, name):
        return getattr(mod, name)
    raise AttributeError(name)
